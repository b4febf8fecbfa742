// Host-side launch descriptors shared between the C ABI layer and the
// kernel files. Arguments here are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

struct CompressLaunch {
  const void *Ca, *Cb, *Za, *Zb;
  const float *Ba, *Bb;
  void* out;
  int64_t B, n_rows, tok_begin, blk_begin, blk_end, out_cap;
  int d, m;
  bool overlap, joint;
  int in_dt, out_dt;
};
hipError_t run_compress(const CompressLaunch& a, hipStream_t st);

struct IndexerLaunch {
  const void* q_idx;
  const float* w;
  const void* k_idx;
  const void* k_scale;  // fp8: fp32 per entry; MXFP4: E8M0 byte per 32 dims
  const int32_t* q_pos;
  const int32_t* n_comp;
  int64_t B, Tq, N_max;
  int H_I, D_I, m;
  int q_dt, k_dt;
  float* scores;
};
hipError_t run_indexer(const IndexerLaunch& a, hipStream_t st);
// a decode step's compression and indexer scan in one launch where the scan
// kernel can carry the compression's workgroups; otherwise the two in turn
hipError_t run_compress_indexer(const CompressLaunch& c, const IndexerLaunch& a, hipStream_t st);

struct TopkLaunch {
  const float* scores;
  const int32_t* q_pos;
  const int32_t* n_comp;
  int64_t B, Tq, N_max;
  int m, top_k;
  int32_t* idx;
  float* out_score;
  void* ws;
  size_t ws_bytes;
};
size_t topk_ws_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k);
hipError_t run_topk(const TopkLaunch& a, hipStream_t st);

struct AttnLaunch {
  int src;  // 0 sparse decode, 1 HCA decode, 2 sparse prefill, 3 HCA prefill
  const void* q;
  const void* kv_comp;
  const int32_t* idx;
  const void* kv_win;  // decode: [B, W, D]; prefill: kv_tok [T_tok, D]
  const int32_t* win_len;
  const int32_t* n_comp;
  const int32_t* q_pos;
  const float* sink;
  float scale;
  int64_t nq;     // queries (decode: B)
  int64_t N_max;  // decode: per-sequence capacity; prefill: N
  int64_t T_tok;
  int H, D, top_k, W, m_rate;
  int kv_dt, out_dt;
  int slots, split_rows, nsplit;
  int Tq, Wb;  // sparse decode: queries per sequence, window buffer rows (0: 1 and W)
  float* part_o;
  float* part_ml;
  void* out;
  float* lse;
};
hipError_t run_attn(const AttnLaunch& a, hipStream_t st);

enum { NR_NORM = 1, NR_ROPE = 2, NR_ROPE_INV = 4 };
struct NormRopeLaunch {
  const void* x;
  void* out;
  const float* gamma;
  const int32_t* pos;
  int64_t T;
  int H, D, R;
  float eps, theta;
  int flags, dt;
};
hipError_t run_norm_rope(const NormRopeLaunch& a, hipStream_t st);

}  // namespace csa
