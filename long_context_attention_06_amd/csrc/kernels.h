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

// Indexer query dtype beside common.h's storage tags (the ABI's
// CSA_BF16_MXFP4): bf16 values that the scan quantises to MXFP4 for an FP4 x
// FP4 product with MXFP4 keys.
constexpr int DT_BF16_MXFP4 = 5;

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
  // top-k support (nullable): the rows' digit histograms [B*Tq, 2048] that the
  // scan adds to or writes (see indexer_hint_mode), and counters it zeroes
  uint32_t* hint;
  uint32_t* zero;
  int64_t zero_n;
};
hipError_t run_indexer(const IndexerLaunch& a, hipStream_t st);
// TOPK_HINT_* that run_indexer produces for these arguments when hint is set
int indexer_hint_mode(const IndexerLaunch& a);
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
  // where the digit histogram at the start of ws comes from (TOPK_HINT_*)
  int hint_mode;
};
enum {
  TOPK_HINT_NONE = 0,         // no histogram: the top-k builds what it needs
  TOPK_HINT_ACCUMULATED = 1,  // added to by this call's scan; the top-k clears it once consumed
  TOPK_HINT_WRITTEN = 2,      // written whole by this call's scan
};
// from_scan: the call's scan provides the histogram (and zeroes the counters)
size_t topk_ws_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k, bool from_scan);
size_t topk_hint_bytes(int64_t rows, int64_t N_max, bool from_scan);
// byte offset of the arrival counters in the top-k workspace (long rows)
size_t topk_counter_offset(int64_t rows, int64_t N_max);
bool topk_long_rows(int64_t N_max);
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
  // HCA decode: the step's append of entry app_blk of every sequence (single
  // branch, m = app_m tokens of bf16 app_Ca / app_Za from row app_tok_begin
  // of app_n_rows), written to kv_comp by the workgroup whose split holds it
  // before it gathers that row (app_Ca NULL: none)
  const void* app_Ca;
  const void* app_Za;
  const float* app_Ba;
  int64_t app_n_rows, app_tok_begin, app_blk;
  int app_m;
  void* app_out;
  // sparse decode on raw queries: RMSNorm (qk_flags & 1, weights qk_gamma or
  // ones) and rotation of the last qk_R dims by q_pos (qk_flags & 2, also the
  // output's inverse rotation); 0: none
  int qk_flags;
  const float* qk_gamma;
  float qk_eps;
  int qk_R;
  float qk_theta;
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

// Phase marks of the decode calls (csa_trace_phases): records the caller's
// event i, if one is set on this thread, on stream st.
enum { PHASE_START = 0, PHASE_SCAN = 1, PHASE_TOPK = 2, PHASE_ATTN = 3, PHASE_END = 4, PHASES = 5 };
void phase_mark(int i, hipStream_t st);

}  // namespace csa
