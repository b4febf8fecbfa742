// C ABI of the CSA/HCA attention library: argument validation (host only,
// before any HIP call), workspace sizing, split planning and kernel dispatch.
// The operations and their sources are documented in include/csa_hca.h.
#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/csa_hca.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define REQ(cond, code, msg)          \
  do {                                \
    if (!(cond)) return fail(code, msg); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char* op) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_HIP_ERROR, std::string(op) + ": " + hipGetErrorString(e));
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Rows per split of the sparse decode attention: 128 per query token of a
// sequence, so a step with Tq tokens per sequence keeps about the same number
// of workgroups per sequence as a one-token step (longer splits rather than
// more of them). Depends only on per-sequence shape arguments, so a
// sequence's result never depends on the batch.
constexpr int SPARSE_SPLIT_ROWS = 128;
constexpr int HCA_MAX_SPLITS = 16;  // dense rows are long: at most 16 splits of whole 32-row tiles

int nsplit_for(int64_t slots, int rows) { return slots <= rows ? 1 : (int)((slots + rows - 1) / rows); }

// at most 1024 rows: the fp32 decode kernel stages a split's top-k codes in
// 1024 LDS slots (the bf16 kernel's row table holds 2048)
int64_t sparse_split_rows(int64_t Tq) { return std::min<int64_t>(SPARSE_SPLIT_ROWS * std::max<int64_t>(1, Tq), 1024); }

int hca_split_rows(int64_t slots) {
  const int64_t per = (slots + HCA_MAX_SPLITS - 1) / HCA_MAX_SPLITS;
  return (int)std::max<int64_t>(32, (per + 31) / 32 * 32);
}

size_t attn_ws(int64_t nq, int H, int D, int nsplit) {
  if (nsplit <= 1) return 0;
  return round256((size_t)nq * nsplit * H * D * 4) + round256((size_t)nq * nsplit * H * 2 * 4);
}

bool attn_supported(int H, int D, int kv_dt) {
  return ((kv_dt == CSA_BF16 || kv_dt == CSA_KV_FP8) && D == 512 && H > 48 && H <= 64) ||
         (kv_dt == CSA_F32 && D == 64 && H >= 1 && H <= 16);
}

// Pointers may be NULL where the call has nothing to read or write through
// them (no query, no row of that source).
int check_attn_common(const void* q, const void* out, float scale, int H, int D, int kv_dt, int out_dt, int W,
                      int top_k, int64_t nq) {
  REQ(nq == 0 || (q && out), CSA_INVALID_ARG, "q and out must not be NULL");
  REQ(scale > 0.0f && scale <= 3.0e38f, CSA_INVALID_ARG, "scale must be positive and finite");
  REQ(H > 0 && D > 0, CSA_INVALID_ARG, "H and D must be positive");
  REQ(W >= 0 && top_k >= 0, CSA_INVALID_ARG, "W and top_k must be >= 0");
  REQ(kv_dt == CSA_F32 || kv_dt == CSA_BF16 || kv_dt == CSA_FP8_E4M3 || kv_dt == CSA_MXFP4 || kv_dt == CSA_KV_FP8,
      CSA_INVALID_ARG, "unknown kv_dt");
  REQ(out_dt == CSA_F32 || out_dt == CSA_BF16 || out_dt == CSA_FP8_E4M3, CSA_INVALID_ARG, "unknown out_dt");
  REQ(out_dt != CSA_FP8_E4M3, CSA_UNSUPPORTED, "out_dt must be F32 or BF16");
  REQ(attn_supported(H, D, kv_dt), CSA_UNSUPPORTED,
      "unsupported (H, D, kv_dt): supported are (49..64, 512, BF16 or KV_FP8) and (1..16, 64, F32)");
  REQ(aligned16(q), CSA_INVALID_ARG, "q must be 16-byte aligned");
  REQ(aligned16(out), CSA_INVALID_ARG, "out must be 16-byte aligned");
  return CSA_OK;
}

int check_indexer(const void* q_idx, const float* w, const void* k_idx, const void* k_scale, const int32_t* q_pos,
                  const int32_t* n_comp, int64_t B, int64_t Tq, int H_I, int D_I, int64_t N_max, int m, int q_dt,
                  int k_dt) {
  REQ(B >= 0 && Tq >= 0 && N_max >= 0, CSA_INVALID_ARG, "B, Tq, N_max must be >= 0");
  REQ(B * Tq == 0 || (q_idx && w && q_pos && n_comp), CSA_INVALID_ARG, "q_idx, w, q_pos, n_comp must not be NULL");
  REQ(B * Tq * N_max == 0 || k_idx, CSA_INVALID_ARG, "k_idx must not be NULL");
  REQ(H_I > 0 && D_I > 0, CSA_INVALID_ARG, "H_I and D_I must be positive");
  REQ(m >= 1, CSA_INVALID_ARG, "m must be >= 1");
  REQ(((q_dt >= CSA_F32 && q_dt <= CSA_FP8_E4M3) || q_dt == CSA_BF16_MXFP4) && k_dt >= CSA_F32 && k_dt <= CSA_MXFP4,
      CSA_INVALID_ARG, "unknown dtype");
  REQ((k_dt != CSA_FP8_E4M3 && k_dt != CSA_MXFP4) || k_scale, CSA_INVALID_ARG, "fp8 and MXFP4 keys need k_scale");
  REQ(k_dt != CSA_MXFP4 || D_I % 32 == 0, CSA_INVALID_ARG, "MXFP4 keys need D_I a multiple of 32");
  REQ(N_max <= (int64_t(1) << 24), CSA_UNSUPPORTED, "N_max above 2^24");
  REQ(B * Tq <= 65535, CSA_UNSUPPORTED, "B*Tq above 65535 rows per call");
  const bool big = H_I == 64 && D_I == 128 &&
                   ((q_dt == CSA_BF16 && (k_dt == CSA_BF16 || k_dt == CSA_FP8_E4M3 || k_dt == CSA_MXFP4)) ||
                    (q_dt == CSA_BF16_MXFP4 && k_dt == CSA_MXFP4));
  const bool tiny = H_I <= 32 && D_I == 32 && q_dt == CSA_F32 && k_dt == CSA_F32;
  REQ(big || tiny, CSA_UNSUPPORTED,
      "unsupported indexer shape/dtype: (64, 128) bf16 q with bf16/fp8/MXFP4 keys, FP4-quantised q with MXFP4 "
      "keys, or (<=32, 32) fp32");
  REQ(aligned16(q_idx) && aligned16(k_idx), CSA_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
  REQ(!k_scale || ((uintptr_t)k_scale & 3) == 0, CSA_INVALID_ARG, "k_scale must be 4-byte aligned");
  return CSA_OK;
}

int check_topk(const float* scores, const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq,
               int64_t N_max, int m, int top_k, const int32_t* topk_idx) {
  REQ(B * Tq == 0 || (scores && q_pos && n_comp && topk_idx), CSA_INVALID_ARG,
      "scores, q_pos, n_comp, topk_idx must not be NULL");
  REQ(B >= 0 && Tq >= 0 && N_max >= 0, CSA_INVALID_ARG, "B, Tq, N_max must be >= 0");
  REQ(m >= 1, CSA_INVALID_ARG, "m must be >= 1");
  REQ(top_k >= 1, CSA_INVALID_ARG, "top_k must be >= 1");
  REQ(top_k <= 4096, CSA_UNSUPPORTED, "top_k above 4096");
  REQ(N_max <= (int64_t(1) << 24), CSA_UNSUPPORTED, "N_max above 2^24");
  REQ(B * Tq <= 65535, CSA_UNSUPPORTED, "B*Tq above 65535 rows per call");
  return CSA_OK;
}

}  // namespace

namespace csa {
namespace {
thread_local hipEvent_t t_phase_ev[PHASES] = {};
thread_local int t_phase_n = 0;
}  // namespace
void phase_mark(int i, hipStream_t st) {
  if (i < t_phase_n && t_phase_ev[i]) (void)hipEventRecord(t_phase_ev[i], st);
}
}  // namespace csa

extern "C" {

int csa_hca_version(void) { return CSA_HCA_VERSION; }

int csa_trace_phases(void* const* events, int n) {
  REQ(n >= 0 && n <= csa::PHASES, CSA_INVALID_ARG, "csa_trace_phases: n must be in [0, 5]");
  REQ(n == 0 || events, CSA_INVALID_ARG, "csa_trace_phases: events must not be NULL");
  for (int i = 0; i < csa::PHASES; ++i) csa::t_phase_ev[i] = i < n ? (hipEvent_t)events[i] : nullptr;
  csa::t_phase_n = n;
  return CSA_OK;
}

const char* csa_last_error(void) { return g_err.c_str(); }

}  // extern "C"

static int prep_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                         const float* Bb, void* out, int64_t B, int64_t n_rows, int64_t tok_begin, int d, int m,
                         int64_t blk_begin, int64_t blk_end, int64_t out_cap, int flags, int in_dt, int out_dt,
                         csa::CompressLaunch* L) {
  REQ((flags & ~(CSA_OVERLAP | CSA_JOINT_SOFTMAX)) == 0, CSA_INVALID_ARG, "unknown flags");
  const bool overlap = flags & CSA_OVERLAP, joint = flags & CSA_JOINT_SOFTMAX;
  REQ(!joint || overlap, CSA_INVALID_ARG, "CSA_JOINT_SOFTMAX needs CSA_OVERLAP");
  const bool empty = B == 0 || blk_end <= blk_begin;  // nothing to read or write
  REQ(empty || (Ca && Za && Ba && out), CSA_INVALID_ARG, "Ca, Za, Ba, out must not be NULL");
  REQ(empty || !overlap || (Cb && Zb && Bb), CSA_INVALID_ARG, "CSA_OVERLAP needs Cb, Zb, Bb");
  REQ(B >= 0 && n_rows >= 0 && tok_begin >= 0, CSA_INVALID_ARG, "B, n_rows, tok_begin must be >= 0");
  REQ(d > 0, CSA_INVALID_ARG, "d must be positive");
  REQ(m >= 1 && m <= 1024, CSA_INVALID_ARG, "m must be in [1, 1024]");
  REQ(0 <= blk_begin && blk_begin <= blk_end, CSA_INVALID_ARG, "need 0 <= blk_begin <= blk_end");
  REQ(blk_end <= out_cap, CSA_INVALID_ARG, "blk_end exceeds out_cap");
  REQ(in_dt == CSA_F32 || in_dt == CSA_BF16 || in_dt == CSA_FP8_E4M3, CSA_INVALID_ARG, "unknown in_dt");
  REQ(out_dt == CSA_F32 || out_dt == CSA_BF16 || out_dt == CSA_FP8_E4M3 || out_dt == CSA_MXFP4 ||
          out_dt == CSA_KV_FP8,
      CSA_INVALID_ARG, "unknown out_dt");
  REQ(in_dt != CSA_FP8_E4M3 && out_dt != CSA_FP8_E4M3 && out_dt != CSA_MXFP4, CSA_UNSUPPORTED,
      "compress reads F32 or BF16 and writes F32, BF16 or KV_FP8 rows");
  REQ(d % 8 == 0, CSA_UNSUPPORTED, "d must be a multiple of 8");
  REQ(out_dt != CSA_KV_FP8 || d > 64, CSA_UNSUPPORTED, "KV_FP8 rows need d > 64 (64 bf16 RoPE channels)");
  if (blk_end > blk_begin) {
    REQ(m * blk_end <= tok_begin + n_rows, CSA_INVALID_ARG,
        "block range needs tokens beyond the provided rows (a block is formed only from m complete tokens)");
    REQ(m * blk_begin >= tok_begin, CSA_INVALID_ARG, "block range starts before tok_begin");
    REQ(!overlap || blk_begin == 0 || m * (blk_begin - 1) >= tok_begin, CSA_INVALID_ARG,
        "overlap branch of blk_begin needs the previous block's tokens");
  }
  REQ(aligned16(Ca) && aligned16(Za) && aligned16(Ba) && aligned16(out), CSA_INVALID_ARG,
      "tensors must be 16-byte aligned");
  REQ(!overlap || (aligned16(Cb) && aligned16(Zb) && aligned16(Bb)), CSA_INVALID_ARG,
      "tensors must be 16-byte aligned");
  *L = csa::CompressLaunch{Ca, Cb, Za, Zb, Ba, Bb, out, B, n_rows, tok_begin, blk_begin, blk_end, out_cap, d, m,
                           overlap, joint, in_dt, out_dt};
  return CSA_OK;
}

extern "C" {

int csa_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba, const float* Bb,
                 void* out, int64_t B, int64_t n_rows, int64_t tok_begin, int d, int m, int64_t blk_begin,
                 int64_t blk_end, int64_t out_cap, int flags, int in_dt, int out_dt, void* stream) {
  csa::CompressLaunch a{};
  int rc = prep_compress(Ca, Cb, Za, Zb, Ba, Bb, out, B, n_rows, tok_begin, d, m, blk_begin, blk_end, out_cap, flags,
                         in_dt, out_dt, &a);
  if (rc) return rc;
  return hip_status(csa::run_compress(a, (hipStream_t)stream), "csa_compress");
}

int indexer_score(const void* q_idx, const float* w, const void* k_idx, const void* k_scale, const int32_t* q_pos,
                  const int32_t* n_comp, int64_t B, int64_t Tq, int H_I, int D_I, int64_t N_max, int m, int q_dt,
                  int k_dt, float* scores, void* stream) {
  int rc = check_indexer(q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, H_I, D_I, N_max, m, q_dt, k_dt);
  if (rc) return rc;
  REQ(B * Tq * N_max == 0 || scores, CSA_INVALID_ARG, "scores must not be NULL");
  csa::IndexerLaunch a{q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, N_max, H_I, D_I, m, q_dt, k_dt, scores};
  return hip_status(csa::run_indexer(a, (hipStream_t)stream), "indexer_score");
}

int csa_compress_indexer_score(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                               const float* Bb, void* kv_out, int64_t Bc, int64_t n_rows, int64_t tok_begin, int d,
                               int m_c, int64_t blk_begin, int64_t blk_end, int64_t out_cap, int flags, int in_dt,
                               int out_dt, const void* q_idx, const float* w, const void* k_idx, const void* k_scale,
                               const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq, int H_I, int D_I,
                               int64_t N_max, int m, int q_dt, int k_dt, float* scores, void* stream) {
  csa::CompressLaunch c{};
  int rc = prep_compress(Ca, Cb, Za, Zb, Ba, Bb, kv_out, Bc, n_rows, tok_begin, d, m_c, blk_begin, blk_end, out_cap,
                         flags, in_dt, out_dt, &c);
  if (rc) return rc;
  rc = check_indexer(q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, H_I, D_I, N_max, m, q_dt, k_dt);
  if (rc) return rc;
  REQ(B * Tq * N_max == 0 || scores, CSA_INVALID_ARG, "scores must not be NULL");
  csa::IndexerLaunch a{q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, N_max, H_I, D_I, m, q_dt, k_dt, scores};
  return hip_status(csa::run_compress_indexer(c, a, (hipStream_t)stream), "csa_compress_indexer_score");
}

size_t indexer_topk_workspace_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k) {
  if (B < 0 || Tq < 0 || N_max < 0) return 0;
  return round256(csa::topk_ws_bytes(B, Tq, N_max, top_k, false));
}

int indexer_topk(const float* scores, const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq,
                 int64_t N_max, int m, int top_k, int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                 void* stream) {
  int rc = check_topk(scores, q_pos, n_comp, B, Tq, N_max, m, top_k, topk_idx);
  if (rc) return rc;
  const size_t need = indexer_topk_workspace_bytes(B, Tq, N_max, top_k);
  REQ(ws_bytes >= need, CSA_WORKSPACE_TOO_SMALL, "workspace too small");
  REQ(need == 0 || ws, CSA_INVALID_ARG, "ws must not be NULL");
  REQ(need == 0 || ((uintptr_t)ws & 255u) == 0, CSA_INVALID_ARG, "ws must be 256-byte aligned");
  csa::TopkLaunch a{scores, q_pos, n_comp, B, Tq, N_max, m, top_k, topk_idx, topk_score, ws, ws_bytes,
                    csa::TOPK_HINT_NONE};
  return hip_status(csa::run_topk(a, (hipStream_t)stream), "indexer_topk");
}

size_t indexer_score_topk_workspace_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k) {
  if (B < 0 || Tq < 0 || N_max < 0) return 0;
  return round256((size_t)B * Tq * N_max * 4) + round256(csa::topk_ws_bytes(B, Tq, N_max, top_k, true));
}

// The scan (scores into the workspace, plus the digit histogram and zeroed
// counters the top-k reads), then the top-k.
static int score_then_topk(const csa::CompressLaunch* c, csa::IndexerLaunch a, int top_k, int32_t* topk_idx,
                           float* topk_score, void* ws, size_t ws_bytes, hipStream_t st, const char* what) {
  const int64_t rows = a.B * a.Tq;
  const size_t sbytes = round256((size_t)rows * a.N_max * 4);
  a.scores = reinterpret_cast<float*>(ws);
  uint8_t* tw = reinterpret_cast<uint8_t*>(ws) + sbytes;
  const int mode = csa::indexer_hint_mode(a);
  a.hint = mode != csa::TOPK_HINT_NONE ? reinterpret_cast<uint32_t*>(tw) : nullptr;
  if (csa::topk_long_rows(a.N_max)) {
    a.zero = reinterpret_cast<uint32_t*>(tw + csa::topk_counter_offset(rows, a.N_max));
    a.zero_n = rows;
  }
  csa::phase_mark(csa::PHASE_START, st);
  int rc = hip_status(c ? csa::run_compress_indexer(*c, a, st) : csa::run_indexer(a, st), what);
  csa::phase_mark(csa::PHASE_SCAN, st);
  if (rc) return rc;
  csa::TopkLaunch t{a.scores, a.q_pos, a.n_comp, a.B, a.Tq, a.N_max, a.m, top_k, topk_idx, topk_score,
                    tw, ws_bytes - sbytes, mode};
  rc = hip_status(csa::run_topk(t, st), what);
  for (int i = csa::PHASE_TOPK; i < csa::PHASES; ++i) csa::phase_mark(i, st);
  return rc;
}

int indexer_score_topk(const void* q_idx, const float* w, const void* k_idx, const void* k_scale,
                       const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq, int H_I, int D_I,
                       int64_t N_max, int m, int top_k, int q_dt, int k_dt, int32_t* topk_idx, float* topk_score,
                       void* ws, size_t ws_bytes, void* stream) {
  int rc = check_indexer(q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, H_I, D_I, N_max, m, q_dt, k_dt);
  if (rc) return rc;
  REQ(B * Tq == 0 || topk_idx, CSA_INVALID_ARG, "topk_idx must not be NULL");
  REQ(top_k >= 1, CSA_INVALID_ARG, "top_k must be >= 1");
  REQ(top_k <= 4096, CSA_UNSUPPORTED, "top_k above 4096");
  const size_t need = indexer_score_topk_workspace_bytes(B, Tq, N_max, top_k);
  REQ(ws_bytes >= need, CSA_WORKSPACE_TOO_SMALL, "workspace too small");
  REQ(need == 0 || ws, CSA_INVALID_ARG, "ws must not be NULL");
  REQ(((uintptr_t)ws & 255u) == 0, CSA_INVALID_ARG, "ws must be 256-byte aligned");
  if (B * Tq == 0) return CSA_OK;
  csa::IndexerLaunch a{q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, N_max, H_I, D_I, m, q_dt, k_dt, nullptr};
  return score_then_topk(nullptr, a, top_k, topk_idx, topk_score, ws, ws_bytes, (hipStream_t)stream,
                         "indexer_score_topk");
}

int csa_compress_indexer_score_topk(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                                    const float* Bb, void* kv_out, int64_t Bc, int64_t n_rows, int64_t tok_begin,
                                    int d, int m_c, int64_t blk_begin, int64_t blk_end, int64_t out_cap, int flags,
                                    int in_dt, int out_dt, const void* q_idx, const float* w, const void* k_idx,
                                    const void* k_scale, const int32_t* q_pos, const int32_t* n_comp, int64_t B,
                                    int64_t Tq, int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt, int k_dt,
                                    int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes, void* stream) {
  csa::CompressLaunch c{};
  int rc = prep_compress(Ca, Cb, Za, Zb, Ba, Bb, kv_out, Bc, n_rows, tok_begin, d, m_c, blk_begin, blk_end, out_cap,
                         flags, in_dt, out_dt, &c);
  if (rc) return rc;
  rc = check_indexer(q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, H_I, D_I, N_max, m, q_dt, k_dt);
  if (rc) return rc;
  REQ(B * Tq == 0 || topk_idx, CSA_INVALID_ARG, "topk_idx must not be NULL");
  REQ(top_k >= 1, CSA_INVALID_ARG, "top_k must be >= 1");
  REQ(top_k <= 4096, CSA_UNSUPPORTED, "top_k above 4096");
  const size_t need = indexer_score_topk_workspace_bytes(B, Tq, N_max, top_k);
  REQ(ws_bytes >= need, CSA_WORKSPACE_TOO_SMALL, "workspace too small");
  REQ(need == 0 || ws, CSA_INVALID_ARG, "ws must not be NULL");
  REQ(((uintptr_t)ws & 255u) == 0, CSA_INVALID_ARG, "ws must be 256-byte aligned");
  if (B * Tq == 0) return hip_status(csa::run_compress(c, (hipStream_t)stream), "csa_compress_indexer_score_topk");
  csa::IndexerLaunch a{q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, N_max, H_I, D_I, m, q_dt, k_dt, nullptr};
  return score_then_topk(&c, a, top_k, topk_idx, topk_score, ws, ws_bytes, (hipStream_t)stream,
                         "csa_compress_indexer_score_topk");
}

// A decode step: [blocks of kv_comp completed by the step's tokens], scores,
// top-k and sparse MQA with the split merge. The workspace holds the scores,
// the top-k's scratch (its digit histogram first, which the scan fills) and
// the attention's split partials.
// The query prologue / output epilogue of csa_decode_step_qk.
struct QkOpts {
  int flags;  // CSA_RMSNORM | CSA_ROPE
  const float* gamma;
  float eps;
  int R;
  float theta;
};

static size_t step_split_rows(int slots, int64_t Tq, int* nsplit) {
  const int rows = (int)sparse_split_rows(Tq);
  *nsplit = nsplit_for(slots, rows);
  return *nsplit > 1 ? rows : slots;
}

size_t csa_decode_step_workspace_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k, int H, int D, int W) {
  if (B < 0 || Tq < 1 || N_max < 0 || top_k < 1 || H <= 0 || D <= 0 || W < 0) return 0;
  const int64_t nq = B * Tq;
  int ns = 0;
  const int sr = (int)step_split_rows(top_k + W, Tq, &ns);
  (void)sr;
  return round256((size_t)nq * N_max * 4) + round256(csa::topk_ws_bytes(B, Tq, N_max, top_k, true)) +
         round256(attn_ws(nq, H, D, ns));
}

static int decode_step_impl(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                            const float* Bb, int64_t n_rows, int64_t tok_begin, int d, int m_c, int64_t blk_begin,
                            int64_t blk_end, int flags, int in_dt, const void* q_idx, const float* w,
                            const void* k_idx, const void* k_scale, const int32_t* q_pos, const int32_t* n_comp,
                            int64_t B, int64_t Tq, int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt,
                            int k_dt, const void* q, void* kv_comp, const void* kv_win, const int32_t* win_len,
                            const float* sink, float scale, int H, int D, int W, int kv_dt, int out_dt,
                            int32_t* topk_idx, float* topk_score, void* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream, const QkOpts* qk = nullptr) {
  REQ(B >= 0 && N_max >= 0, CSA_INVALID_ARG, "B and N_max must be >= 0");
  REQ(Tq >= 1 && Tq <= 64, CSA_INVALID_ARG, "Tq must be in [1, 64]");
  const int64_t nq = B * Tq;
  csa::CompressLaunch c{};
  int rc = prep_compress(Ca, Cb, Za, Zb, Ba, Bb, kv_comp, B, n_rows, tok_begin, d, m_c, blk_begin, blk_end, N_max,
                         flags, in_dt, kv_dt, &c);
  if (rc) return rc;
  REQ(blk_begin == blk_end || d == D, CSA_INVALID_ARG, "the compressed rows must have the attention's D channels");
  rc = check_indexer(q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, H_I, D_I, N_max, m, q_dt, k_dt);
  if (rc) return rc;
  REQ(top_k >= 1, CSA_INVALID_ARG, "top_k must be >= 1");
  REQ(top_k <= 4096, CSA_UNSUPPORTED, "top_k above 4096");
  REQ(nq == 0 || topk_idx, CSA_INVALID_ARG, "topk_idx must not be NULL");
  rc = check_attn_common(q, out, scale, H, D, kv_dt, out_dt, W, top_k, nq);
  if (rc) return rc;
  REQ(nq == 0 || kv_comp, CSA_INVALID_ARG, "kv_comp must not be NULL");
  REQ(nq == 0 || W == 0 || (kv_win && win_len), CSA_INVALID_ARG, "kv_win and win_len must not be NULL");
  REQ((int64_t)top_k + W <= (1 << 24), CSA_UNSUPPORTED, "too many rows per query");
  const size_t base_need = csa_decode_step_workspace_bytes(B, Tq, N_max, top_k, H, D, W);
  const bool qk_on = qk && qk->flags;
  const size_t need = base_need + (qk_on ? round256((size_t)nq * H * D * 2) : 0);
  REQ(ws_bytes >= need, CSA_WORKSPACE_TOO_SMALL, "workspace too small");
  REQ(need == 0 || ws, CSA_INVALID_ARG, "ws must not be NULL");
  REQ(((uintptr_t)ws & 255u) == 0, CSA_INVALID_ARG, "ws must be 256-byte aligned");
  REQ(!qk_on || out_dt == CSA_BF16 || out_dt == CSA_F32, CSA_UNSUPPORTED, "out_dt must be F32 or BF16");
  hipStream_t st = (hipStream_t)stream;
  if (nq == 0) return hip_status(csa::run_compress(c, st), "csa_decode_step");
  REQ(nq <= 0x7fffffff, CSA_UNSUPPORTED, "B * Tq too large");

  const int slots = top_k + W;
  int ns = 0;
  const int sr = (int)step_split_rows(slots, Tq, &ns);
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  float* scores = reinterpret_cast<float*>(p);
  p += round256((size_t)nq * N_max * 4);
  uint8_t* tw = p;  // top-k scratch, digit histogram first
  p += round256(csa::topk_ws_bytes(B, Tq, N_max, top_k, true));
  uint8_t* xw = p;  // the attention's split partials

  csa::IndexerLaunch a{q_idx, w, k_idx, k_scale, q_pos, n_comp, B, Tq, N_max, H_I, D_I, m, q_dt, k_dt, scores};
  const int mode = csa::indexer_hint_mode(a);
  a.hint = mode != csa::TOPK_HINT_NONE ? reinterpret_cast<uint32_t*>(tw) : nullptr;
  if (csa::topk_long_rows(N_max)) {
    a.zero = reinterpret_cast<uint32_t*>(tw + csa::topk_counter_offset(nq, N_max));
    a.zero_n = nq;
  }
  csa::phase_mark(csa::PHASE_START, st);
  rc = hip_status(csa::run_compress_indexer(c, a, st), "csa_decode_step");
  csa::phase_mark(csa::PHASE_SCAN, st);
  if (rc) return rc;
  csa::TopkLaunch tk{scores, q_pos, n_comp, B, Tq, N_max, m, top_k, topk_idx, topk_score, tw,
                     csa::topk_ws_bytes(B, Tq, N_max, top_k, true), mode};
  rc = hip_status(csa::run_topk(tk, st), "csa_decode_step");
  csa::phase_mark(csa::PHASE_TOPK, st);
  if (rc) return rc;
  // the query prologue and the output's inverse rotation ride in the
  // attention and merge kernels (D = 512 rows; each rotated pair's angle is
  // formed in one lane of a wave, so R / 2 <= 64); otherwise the standalone
  // kernels run around the attention
  const bool qk_fold = qk_on && D == 512 && kv_dt != CSA_F32 && (!(qk->flags & CSA_ROPE) || qk->R <= 128);
  const void* q_att = q;
  if (qk_on && !qk_fold) {
    void* qn = reinterpret_cast<uint8_t*>(ws) + base_need;
    csa::NormRopeLaunch nr{q, qn, qk->gamma, q_pos, nq, H, D, (qk->flags & CSA_ROPE) ? qk->R : 2, qk->eps,
                           qk->theta, qk->flags & (CSA_RMSNORM | CSA_ROPE), CSA_BF16};
    rc = hip_status(csa::run_norm_rope(nr, st), "csa_decode_step_qk");
    if (rc) return rc;
    q_att = qn;
  }
  csa::AttnLaunch at{};
  at.src = 0;
  at.q = q_att;
  at.kv_comp = kv_comp;
  at.idx = topk_idx;
  at.kv_win = kv_win;
  at.win_len = W == 0 ? nullptr : win_len;
  at.sink = sink;
  at.scale = scale;
  at.nq = nq;
  at.N_max = N_max;
  at.H = H;
  at.D = D;
  at.top_k = top_k;
  at.W = W;
  at.Tq = (int)Tq;
  at.Wb = W + (int)Tq - 1;
  at.m_rate = 1;
  at.kv_dt = kv_dt;
  at.out_dt = out_dt;
  at.slots = slots;
  at.split_rows = sr;
  at.nsplit = ns;
  at.part_o = reinterpret_cast<float*>(xw);
  at.part_ml = reinterpret_cast<float*>(xw + round256((size_t)nq * ns * H * D * 4));
  at.out = out;
  at.lse = lse;
  if (qk_fold) {
    at.q_pos = q_pos;
    at.qk_flags = ((qk->flags & CSA_RMSNORM) ? 1 : 0) | ((qk->flags & CSA_ROPE) ? 2 : 0);
    at.qk_gamma = qk->gamma;
    at.qk_eps = qk->eps;
    at.qk_R = qk->R;
    at.qk_theta = qk->theta;
  }
  rc = hip_status(csa::run_attn(at, st), "csa_decode_step");
  if (rc == CSA_OK && qk_on && !qk_fold && (qk->flags & CSA_ROPE)) {
    csa::NormRopeLaunch nr{out, out, nullptr, q_pos, nq, H, D, qk->R, 0.0f, qk->theta, CSA_ROPE_INVERSE, out_dt};
    rc = hip_status(csa::run_norm_rope(nr, st), "csa_decode_step_qk");
  }
  csa::phase_mark(csa::PHASE_END, st);
  return rc;
}

int csa_decode_step(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba, const float* Bb,
                    int64_t n_rows, int64_t tok_begin, int d, int m_c, int64_t blk_begin, int64_t blk_end,
                    int flags, int in_dt, const void* q_idx, const float* w, const void* k_idx,
                    const void* k_scale, const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq,
                    int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt, int k_dt, const void* q,
                    void* kv_comp, const void* kv_win, const int32_t* win_len, const float* sink, float scale, int H,
                    int D, int W, int kv_dt, int out_dt, int32_t* topk_idx, float* topk_score, void* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream) {
  return decode_step_impl(Ca, Cb, Za, Zb, Ba, Bb, n_rows, tok_begin, d, m_c, blk_begin, blk_end, flags, in_dt, q_idx,
                          w, k_idx, k_scale, q_pos, n_comp, B, Tq, H_I, D_I, N_max, m, top_k, q_dt, k_dt, q, kv_comp,
                          kv_win, win_len, sink, scale, H, D, W, kv_dt, out_dt, topk_idx, topk_score, out, lse, ws,
                          ws_bytes, stream);
}

size_t csa_decode_step_qk_workspace_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k, int H, int D, int W) {
  const size_t base = csa_decode_step_workspace_bytes(B, Tq, N_max, top_k, H, D, W);
  return base == 0 ? 0 : base + round256((size_t)(B * Tq) * H * D * 2);
}

int csa_decode_step_qk(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                       const float* Bb, int64_t n_rows, int64_t tok_begin, int d, int m_c, int64_t blk_begin,
                       int64_t blk_end, int flags, int in_dt, const void* q_idx, const float* w, const void* k_idx,
                       const void* k_scale, const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq,
                       int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt, int k_dt, const void* q,
                       void* kv_comp, const void* kv_win, const int32_t* win_len, const float* sink, float scale,
                       int H, int D, int W, int kv_dt, int out_dt, int32_t* topk_idx, float* topk_score, void* out,
                       float* lse, const float* q_gamma, float eps, int rope_dims, float rope_theta, int qk_flags,
                       void* ws, size_t ws_bytes, void* stream) {
  REQ((qk_flags & ~(CSA_RMSNORM | CSA_ROPE)) == 0, CSA_INVALID_ARG, "qk_flags: CSA_RMSNORM and/or CSA_ROPE");
  const bool rope = qk_flags & CSA_ROPE;
  REQ(!rope || (rope_dims >= 2 && rope_dims <= D && rope_dims % 2 == 0), CSA_INVALID_ARG,
      "rope_dims must be even and in [2, D]");
  REQ(!rope || (rope_theta > 0.0f && rope_theta <= 3.0e38f), CSA_INVALID_ARG, "rope_theta must be positive and finite");
  REQ(!(qk_flags & CSA_RMSNORM) || (eps >= 0.0f && eps <= 3.0e38f), CSA_INVALID_ARG, "eps must be >= 0 and finite");
  REQ(D % 8 == 0 && D <= 512, CSA_UNSUPPORTED, "D must be a multiple of 8, at most 512");
  const QkOpts qk{qk_flags, q_gamma, eps, rope ? rope_dims : 2, rope_theta};
  return decode_step_impl(Ca, Cb, Za, Zb, Ba, Bb, n_rows, tok_begin, d, m_c, blk_begin, blk_end, flags, in_dt, q_idx,
                          w, k_idx, k_scale, q_pos, n_comp, B, Tq, H_I, D_I, N_max, m, top_k, q_dt, k_dt, q, kv_comp,
                          kv_win, win_len, sink, scale, H, D, W, kv_dt, out_dt, topk_idx, topk_score, out, lse, ws,
                          ws_bytes, stream, &qk);
}

}  // extern "C"

// ---- the decode step for callers that cannot allocate: its scratch is the
// file-scope device array below (each device holds its own copy, at its own
// address, from the library's load until the process ends). In host code the
// array's name is only a stand-in: kernels get the address that
// hipGetSymbolAddress returned for the current device.
static __device__ __align__(256) uint8_t scratch[CSA_STEP_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_DEVICES = 64;
struct ScratchDev {
  void* ptr = nullptr;    // this device's address of `scratch`
  int64_t shape[7] = {};  // the previous call's shape, which fixes the scratch layout
  bool used = false;
};
std::mutex g_scratch_mu;
ScratchDev g_scratch[SCRATCH_DEVICES];

__global__ void zero_fill_kernel(uint4* p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}
}  // namespace

extern "C" {

int csa_decode_step_noalloc(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                            const float* Bb, int64_t n_rows, int64_t tok_begin, int d, int m_c, int64_t blk_begin,
                            int64_t blk_end, int flags, int in_dt, const void* q_idx, const float* w,
                            const void* k_idx, const void* k_scale, const int32_t* q_pos, const int32_t* n_comp,
                            int64_t B, int64_t Tq, int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt,
                            int k_dt, const void* q, void* kv_comp, const void* kv_win, const int32_t* win_len,
                            const float* sink, float scale, int H, int D, int W, int kv_dt, int out_dt,
                            int32_t* topk_idx, float* topk_score, void* out, float* lse, void* stream) {
  const size_t need = csa_decode_step_workspace_bytes(B, Tq, N_max, top_k, H, D, W);
  REQ(need <= CSA_STEP_SCRATCH_BYTES, CSA_WORKSPACE_TOO_SMALL,
      "csa_decode_step_noalloc: the step needs " + std::to_string(need) + " bytes of scratch, above the " +
          std::to_string((size_t)CSA_STEP_SCRATCH_BYTES) + " this form holds; use csa_decode_step");
  int dev = 0;
  int rc = hip_status(hipGetDevice(&dev), "csa_decode_step_noalloc: hipGetDevice");
  if (rc) return rc;
  REQ(dev >= 0 && dev < SCRATCH_DEVICES, CSA_UNSUPPORTED, "csa_decode_step_noalloc: device index above 63");
  void* ptr = nullptr;
  bool clear = false;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    ScratchDev& sd = g_scratch[dev];
    if (!sd.ptr) {
      void* p = nullptr;
      rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "csa_decode_step_noalloc: hipGetSymbolAddress");
      if (rc) return rc;
      REQ(p && ((uintptr_t)p & 255u) == 0, CSA_HIP_ERROR, "csa_decode_step_noalloc: scratch address not usable");
      sd.ptr = p;
    }
    const int64_t shape[7] = {B, Tq, N_max, top_k, H, D, W};
    clear = !sd.used || !std::equal(shape, shape + 7, sd.shape);
    std::copy(shape, shape + 7, sd.shape);
    sd.used = true;
    ptr = sd.ptr;
  }
  // Results never depend on the scratch's contents; zeros (or what a call of
  // the same shape left) let the selection use the scan's histogram. A new
  // layout is cleared by a fill kernel, which a graph capture can hold.
  if (clear && need > 0) {
    const size_t n16 = (need + 15) / 16;
    const unsigned blocks = (unsigned)std::min<size_t>((n16 + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<uint4*>(ptr), n16);
    rc = hip_status(hipGetLastError(), "csa_decode_step_noalloc: clear");
    if (rc) return rc;
  }
  return decode_step_impl(Ca, Cb, Za, Zb, Ba, Bb, n_rows, tok_begin, d, m_c, blk_begin, blk_end, flags, in_dt, q_idx,
                          w, k_idx, k_scale, q_pos, n_comp, B, Tq, H_I, D_I, N_max, m, top_k, q_dt, k_dt, q, kv_comp,
                          kv_win, win_len, sink, scale, H, D, W, kv_dt, out_dt, topk_idx, topk_score, out, lse, ptr,
                          CSA_STEP_SCRATCH_BYTES, stream);
}

size_t sparse_mqa_decode_multi_workspace_bytes(int64_t B, int64_t Tq, int H, int D, int top_k, int W) {
  if (B < 0 || Tq < 1 || H <= 0 || D <= 0 || top_k < 0 || W < 0) return 0;
  int ns = 0;
  step_split_rows(top_k + W, Tq, &ns);
  return attn_ws(B * Tq, H, D, ns);
}

size_t sparse_mqa_decode_workspace_bytes(int64_t B, int H, int D, int top_k, int W) {
  return sparse_mqa_decode_multi_workspace_bytes(B, 1, H, D, top_k, W);
}

int sparse_mqa_decode_multi(const void* q, const void* kv_comp, const int32_t* topk_idx, const void* kv_win,
                            const int32_t* win_len, const float* sink, float scale, int64_t B, int64_t Tq, int H,
                            int D, int64_t N_max, int top_k, int W, int kv_dt, int out_dt, void* out, float* lse,
                            void* ws, size_t ws_bytes, void* stream) {
  REQ(B >= 0 && N_max >= 0, CSA_INVALID_ARG, "B and N_max must be >= 0");
  REQ(Tq >= 1 && Tq <= 64, CSA_INVALID_ARG, "Tq must be in [1, 64]");
  const int64_t nq = B * Tq;
  int rc = check_attn_common(q, out, scale, H, D, kv_dt, out_dt, W, top_k, nq);
  if (rc) return rc;
  REQ(nq == 0 || top_k == 0 || (kv_comp && topk_idx), CSA_INVALID_ARG, "kv_comp and topk_idx must not be NULL");
  REQ(nq == 0 || W == 0 || (kv_win && win_len), CSA_INVALID_ARG, "kv_win and win_len must not be NULL");
  REQ((int64_t)top_k + W <= (1 << 24), CSA_UNSUPPORTED, "too many rows per query");
  int ns = 0;
  const int sr = (int)step_split_rows(top_k + W, Tq, &ns);
  const size_t need = attn_ws(nq, H, D, ns);
  REQ(ws_bytes >= need, CSA_WORKSPACE_TOO_SMALL, "workspace too small");
  REQ(need == 0 || ws, CSA_INVALID_ARG, "ws must not be NULL");
  REQ(((uintptr_t)ws & 255u) == 0, CSA_INVALID_ARG, "ws must be 256-byte aligned");
  REQ(nq <= 0x7fffffff, CSA_UNSUPPORTED, "B * Tq too large");
  csa::AttnLaunch a{};
  a.src = 0;
  a.q = q;
  a.kv_comp = kv_comp;
  a.idx = topk_idx;
  a.kv_win = kv_win;
  a.win_len = win_len;
  a.sink = sink;
  a.scale = scale;
  a.nq = nq;
  a.N_max = N_max;
  a.H = H;
  a.D = D;
  a.top_k = top_k;
  a.W = W;
  a.Tq = (int)Tq;
  a.Wb = W + (int)Tq - 1;
  a.m_rate = 1;
  a.kv_dt = kv_dt;
  a.out_dt = out_dt;
  a.slots = top_k + W;
  a.split_rows = sr;
  a.nsplit = ns;
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + round256((size_t)nq * ns * H * D * 4));
  a.out = out;
  a.lse = lse;
  if (W == 0) a.win_len = nullptr;
  return hip_status(csa::run_attn(a, (hipStream_t)stream), "sparse_mqa_decode");
}

int sparse_mqa_decode(const void* q, const void* kv_comp, const int32_t* topk_idx, const void* kv_win,
                      const int32_t* win_len, const float* sink, float scale, int64_t B, int H, int D, int64_t N_max,
                      int top_k, int W, int kv_dt, int out_dt, void* out, float* lse, void* ws, size_t ws_bytes,
                      void* stream) {
  return sparse_mqa_decode_multi(q, kv_comp, topk_idx, kv_win, win_len, sink, scale, B, 1, H, D, N_max, top_k, W,
                                 kv_dt, out_dt, out, lse, ws, ws_bytes, stream);
}

size_t sparse_mqa_prefill_workspace_bytes(int64_t, int, int, int, int) { return 0; }

int sparse_mqa_prefill(const void* q, const void* kv_comp, const int32_t* topk_idx, const void* kv_tok,
                       const int32_t* q_pos, const float* sink, float scale, int64_t Tq, int H, int D, int64_t N,
                       int64_t T_tok, int top_k, int W, int kv_dt, int out_dt, void* out, float* lse, void* ws,
                       size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_attn_common(q, out, scale, H, D, kv_dt, out_dt, W, top_k, Tq);
  if (rc) return rc;
  REQ(Tq >= 0 && N >= 0 && T_tok >= 0, CSA_INVALID_ARG, "Tq, N, T_tok must be >= 0");
  REQ(Tq == 0 || q_pos, CSA_INVALID_ARG, "q_pos must not be NULL");
  REQ(Tq == 0 || top_k == 0 || (kv_comp && topk_idx), CSA_INVALID_ARG, "kv_comp and topk_idx must not be NULL");
  REQ(Tq == 0 || W == 0 || kv_tok, CSA_INVALID_ARG, "kv_tok must not be NULL");
  REQ((int64_t)top_k + W <= (1 << 24), CSA_UNSUPPORTED, "too many rows per query");
  REQ(Tq <= 0x7fffffff, CSA_UNSUPPORTED, "Tq too large");
  REQ(kv_dt != CSA_F32 || top_k <= 1024, CSA_UNSUPPORTED, "sparse_mqa_prefill on f32 rows supports top_k <= 1024");
  REQ(top_k + W <= 2048, CSA_UNSUPPORTED, "sparse_mqa_prefill supports top_k + W <= 2048 rows per query");
  csa::AttnLaunch a{};
  a.src = 2;
  a.q = q;
  a.kv_comp = kv_comp;
  a.idx = topk_idx;
  a.kv_win = kv_tok;
  a.q_pos = q_pos;
  a.sink = sink;
  a.scale = scale;
  a.nq = Tq;
  a.N_max = N;
  a.T_tok = T_tok;
  a.H = H;
  a.D = D;
  a.top_k = top_k;
  a.W = W;
  a.m_rate = 1;
  a.kv_dt = kv_dt;
  a.out_dt = out_dt;
  a.slots = top_k + W;
  a.split_rows = a.slots;
  a.nsplit = 1;
  a.out = out;
  a.lse = lse;
  return hip_status(csa::run_attn(a, (hipStream_t)stream), "sparse_mqa_prefill");
}

int qk_norm_rope(const void* x, void* out, const float* gamma, const int32_t* pos, int64_t T, int H, int D,
                 int rope_dims, float eps, float rope_theta, int flags, int dt, void* stream) {
  REQ(T * (int64_t)H == 0 || (x && out), CSA_INVALID_ARG, "x and out must not be NULL");
  REQ((flags & ~(CSA_RMSNORM | CSA_ROPE | CSA_ROPE_INVERSE)) == 0, CSA_INVALID_ARG, "unknown flags");
  REQ(!((flags & CSA_ROPE) && (flags & CSA_ROPE_INVERSE)), CSA_INVALID_ARG, "CSA_ROPE and CSA_ROPE_INVERSE together");
  REQ(T >= 0 && H >= 1 && D >= 1, CSA_INVALID_ARG, "need T >= 0, H >= 1, D >= 1");
  REQ(dt == CSA_F32 || dt == CSA_BF16, CSA_UNSUPPORTED, "dt must be F32 or BF16");
  REQ(D % 8 == 0 && D <= 512, CSA_UNSUPPORTED, "D must be a multiple of 8, at most 512");
  const bool rope = flags & (CSA_ROPE | CSA_ROPE_INVERSE);
  REQ(!rope || T == 0 || pos, CSA_INVALID_ARG, "pos must not be NULL with a rotation");
  REQ(!rope || (rope_dims >= 2 && rope_dims <= D && rope_dims % 2 == 0), CSA_INVALID_ARG,
      "rope_dims must be even and in [2, D]");
  REQ(!rope || (rope_theta > 0.0f && rope_theta <= 3.0e38f), CSA_INVALID_ARG, "rope_theta must be positive and finite");
  REQ(!(flags & CSA_RMSNORM) || (eps >= 0.0f && eps <= 3.0e38f), CSA_INVALID_ARG, "eps must be >= 0 and finite");
  REQ(aligned16(x) && aligned16(out), CSA_INVALID_ARG, "x and out must be 16-byte aligned");
  REQ(T * (int64_t)H <= ((int64_t)1 << 33), CSA_UNSUPPORTED, "too many rows");
  csa::NormRopeLaunch a{x, out, gamma, pos, T, H, D, rope ? rope_dims : 2, eps, rope_theta, flags, dt};
  return hip_status(csa::run_norm_rope(a, (hipStream_t)stream), "qk_norm_rope");
}

size_t hca_prefill_workspace_bytes(int64_t, int, int, int64_t, int) { return 0; }

int hca_prefill(const void* q, const void* kv_comp, const void* kv_tok, const int32_t* q_pos, const float* sink,
                float scale, int64_t Tq, int H, int D, int64_t N, int m, int64_t T_tok, int W, int kv_dt, int out_dt,
                void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_attn_common(q, out, scale, H, D, kv_dt, out_dt, W, 0, Tq);
  if (rc) return rc;
  REQ(Tq >= 0 && N >= 0 && T_tok >= 0, CSA_INVALID_ARG, "Tq, N, T_tok must be >= 0");
  REQ(m >= 1, CSA_INVALID_ARG, "m must be >= 1");
  REQ(Tq == 0 || q_pos, CSA_INVALID_ARG, "q_pos must not be NULL");
  REQ(Tq == 0 || N == 0 || kv_comp, CSA_INVALID_ARG, "kv_comp must not be NULL");
  REQ(Tq == 0 || W == 0 || kv_tok, CSA_INVALID_ARG, "kv_tok must not be NULL");
  REQ(N + W <= (1 << 24), CSA_UNSUPPORTED, "too many rows per query");
  REQ(Tq <= 0x7fffffff, CSA_UNSUPPORTED, "Tq too large");
  csa::AttnLaunch a{};
  a.src = 3;
  a.q = q;
  a.kv_comp = kv_comp;
  a.kv_win = kv_tok;
  a.q_pos = q_pos;
  a.sink = sink;
  a.scale = scale;
  a.nq = Tq;
  a.N_max = N;
  a.T_tok = T_tok;
  a.H = H;
  a.D = D;
  a.W = W;
  a.m_rate = m;
  a.kv_dt = kv_dt;
  a.out_dt = out_dt;
  a.slots = (int)(N + W);
  a.split_rows = a.slots;
  a.nsplit = 1;
  a.out = out;
  a.lse = lse;
  return hip_status(csa::run_attn(a, (hipStream_t)stream), "hca_prefill");
}

size_t hca_dense_mqa_workspace_bytes(int64_t B, int H, int D, int64_t N_max, int W) {
  if (B < 0 || H <= 0 || D <= 0 || N_max < 0 || W < 0) return 0;
  return attn_ws(B, H, D, nsplit_for(N_max + W, hca_split_rows(N_max + W)));
}

// Checks and the split plan of an HCA decode call (hca_dense_mqa and the
// attention of hca_decode_step).
static int hca_prep(const void* q, const void* kv_comp, const int32_t* n_comp, const int32_t* q_pos, int m,
                    const void* kv_win, const int32_t* win_len, const float* sink, float scale, int64_t B, int H,
                    int D, int64_t N_max, int W, int kv_dt, int out_dt, void* out, float* lse, void* ws,
                    size_t ws_bytes, csa::AttnLaunch* a) {
  int rc = check_attn_common(q, out, scale, H, D, kv_dt, out_dt, W, 0, B);
  if (rc) return rc;
  REQ(B >= 0 && N_max >= 0, CSA_INVALID_ARG, "B and N_max must be >= 0");
  REQ(m >= 1, CSA_INVALID_ARG, "m must be >= 1");
  REQ(B == 0 || N_max == 0 || (kv_comp && n_comp && q_pos), CSA_INVALID_ARG,
      "kv_comp, n_comp, q_pos must not be NULL");
  REQ(B == 0 || W == 0 || (kv_win && win_len), CSA_INVALID_ARG, "kv_win and win_len must not be NULL");
  REQ(N_max + W <= (1 << 24), CSA_UNSUPPORTED, "too many rows per query");
  const int hsr = hca_split_rows(N_max + W);
  const int ns = nsplit_for(N_max + W, hsr);
  const size_t need = attn_ws(B, H, D, ns);
  REQ(ws_bytes >= need, CSA_WORKSPACE_TOO_SMALL, "workspace too small");
  REQ(need == 0 || ws, CSA_INVALID_ARG, "ws must not be NULL");
  REQ(((uintptr_t)ws & 255u) == 0, CSA_INVALID_ARG, "ws must be 256-byte aligned");
  REQ(B <= 0x7fffffff, CSA_UNSUPPORTED, "B too large");
  *a = csa::AttnLaunch{};
  a->src = 1;
  a->q = q;
  a->kv_comp = kv_comp;
  a->kv_win = kv_win;
  a->win_len = win_len;
  a->n_comp = n_comp;
  a->q_pos = q_pos;
  a->sink = sink;
  a->scale = scale;
  a->nq = B;
  a->N_max = N_max;
  a->H = H;
  a->D = D;
  a->W = W;
  a->m_rate = m;
  a->kv_dt = kv_dt;
  a->out_dt = out_dt;
  a->slots = (int)(N_max + W);
  a->split_rows = ns > 1 ? hsr : a->slots;
  a->nsplit = ns;
  a->part_o = reinterpret_cast<float*>(ws);
  a->part_ml = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + round256((size_t)B * ns * H * D * 4));
  a->out = out;
  a->lse = lse;
  return CSA_OK;
}

int hca_dense_mqa(const void* q, const void* kv_comp, const int32_t* n_comp, const int32_t* q_pos, int m,
                  const void* kv_win, const int32_t* win_len, const float* sink, float scale, int64_t B, int H, int D,
                  int64_t N_max, int W, int kv_dt, int out_dt, void* out, float* lse, void* ws, size_t ws_bytes,
                  void* stream) {
  csa::AttnLaunch a;
  int rc = hca_prep(q, kv_comp, n_comp, q_pos, m, kv_win, win_len, sink, scale, B, H, D, N_max, W, kv_dt, out_dt,
                    out, lse, ws, ws_bytes, &a);
  if (rc) return rc;
  for (int i = csa::PHASE_START; i < csa::PHASE_ATTN; ++i) csa::phase_mark(i, (hipStream_t)stream);
  rc = hip_status(csa::run_attn(a, (hipStream_t)stream), "hca_dense_mqa");
  csa::phase_mark(csa::PHASE_END, (hipStream_t)stream);
  return rc;
}

size_t hca_decode_step_workspace_bytes(int64_t B, int H, int D, int64_t N_max, int W) {
  return hca_dense_mqa_workspace_bytes(B, H, D, N_max, W);
}

int hca_decode_step(const void* Ca, const void* Za, const float* Ba, int64_t n_rows, int64_t tok_begin, int d,
                    int m_c, int64_t blk_begin, int64_t blk_end, int in_dt, const void* q, void* kv_comp,
                    const int32_t* n_comp, const int32_t* q_pos, int m, const void* kv_win, const int32_t* win_len,
                    const float* sink, float scale, int64_t B, int H, int D, int64_t N_max, int W, int kv_dt,
                    int out_dt, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  csa::CompressLaunch c{};
  int rc = prep_compress(Ca, nullptr, Za, nullptr, Ba, nullptr, kv_comp, B, n_rows, tok_begin, d, m_c, blk_begin,
                         blk_end, N_max, 0, in_dt, kv_dt, &c);
  if (rc) return rc;
  REQ(blk_begin == blk_end || d == D, CSA_INVALID_ARG, "the compressed rows must have the attention's D channels");
  csa::AttnLaunch a;
  rc = hca_prep(q, kv_comp, n_comp, q_pos, m, kv_win, win_len, sink, scale, B, H, D, N_max, W, kv_dt, out_dt, out,
                lse, ws, ws_bytes, &a);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (B == 0) return CSA_OK;
  // the append rides in the attention's launch: the workgroup whose split
  // holds the new entry computes it first (bf16 inputs, one block, D = 512)
  const bool fold = blk_end - blk_begin == 1 && in_dt == CSA_BF16 && D == 512 && kv_dt != CSA_F32;
  csa::phase_mark(csa::PHASE_START, st);
  if (fold) {
    a.app_Ca = Ca;
    a.app_Za = Za;
    a.app_Ba = Ba;
    a.app_n_rows = n_rows;
    a.app_tok_begin = tok_begin;
    a.app_blk = blk_begin;
    a.app_m = m_c;
    a.app_out = kv_comp;
    csa::phase_mark(csa::PHASE_SCAN, st);
    csa::phase_mark(csa::PHASE_TOPK, st);
    rc = hip_status(csa::run_attn(a, st), "hca_decode_step");
    csa::phase_mark(csa::PHASE_END, st);
    return rc;
  }
  rc = hip_status(csa::run_compress(c, st), "hca_decode_step");
  if (rc) return rc;
  csa::phase_mark(csa::PHASE_SCAN, st);
  csa::phase_mark(csa::PHASE_TOPK, st);
  rc = hip_status(csa::run_attn(a, st), "hca_decode_step");
  csa::phase_mark(csa::PHASE_END, st);
  return rc;
}

}  // extern "C"
