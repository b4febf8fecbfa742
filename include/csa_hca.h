/*
 * csa_hca.h — C ABI of the MI355X (gfx950) library for DeepSeek-V4's hybrid
 * long-context attention: CSA (compressed sparse attention) and HCA (heavily
 * compressed attention).
 *
 * What the calls compute (sources are web pages on DeepSeek-V4, cited by
 * title and section):
 *   [CSDN]   "DeepSeek V4 脱离 CUDA 全栈国产化：1.6T MoE 逐层拆解 + 昇腾迁移数据"
 *            (deepseek.csdn.net), section 二 "CSA + HCA 混合注意力": CSA is
 *            compress -> lightning indexer + top-k -> shared-KV MQA (the
 *            CComp_i equation gives the compression); HCA compresses 128
 *            tokens per entry and attends densely, with a 128-token window.
 *   [LIDUOS] liduos.com "deepseek-v4-engineering-tradeoffs", section
 *            "1M Context 的结构与取舍": the sliding window keeps the latest 128
 *            raw tokens; an attention sink lets a head attend to nothing.
 *   [LQNN]   "Deepseek-V4 技术报告里最值得复现的三个改动" (m.lqnn.cn), section 3
 *            (m=4, 64x128 indexer, top_k 512, m'=128, 64 heads x 512, window
 *            128) and section 5 (tokens after the last full block of m are not
 *            compressed).
 *   [CSDN] section 八 (MegaMoE 超级内核与训练稳定性) also carries the
 *            batch-invariance remark: a token's output is bitwise the same
 *            wherever it sits in a batch.
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers owned by the caller, unless stated. The
 *     library allocates nothing, frees nothing and keeps no state between
 *     calls. Scratch memory comes in through (ws, ws_bytes); each op has a
 *     pure host-side query <op>_workspace_bytes(...). ws must be 256-byte
 *     aligned; its contents on entry do not matter.
 *   - stream is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     kernels on it: no host synchronisation, no device-to-host copy, no
 *     memset; they can be captured in a HIP graph.
 *   - Tensors are dense and row-major; the innermost index is the feature.
 *     Indices, positions and lengths are int32.
 *   - dtype codes: CSA_F32, CSA_BF16 (storage of activations and caches),
 *     CSA_FP8_E4M3 (OCP E4M3 "FN", indexer keys only, with a per-entry fp32
 *     scale), CSA_MXFP4 (OCP Microscaling MXFP4, indexer keys only: FP4 E2M1
 *     elements, two per byte with element 2j in the low nibble of byte j, and
 *     one E8M0 scale byte per block of 32 elements; the pages keep the
 *     indexer in FP4), CSA_KV_FP8 (the mixed-precision main KV row the pages
 *     describe: RoPE dims in BF16, the rest in FP8 -- for a row of D dims,
 *     bytes 0 .. D-65 are the OCP E4M3 codes of dims 0 .. D-65 and the next
 *     128 bytes the last 64 dims as bf16, little endian: D + 64 bytes per row,
 *     no scale), CSA_BF16_MXFP4 (indexer queries only: bf16 values that the
 *     call quantises to MXFP4 -- per 32-dim block of each head row, the OCP
 *     rule: E8M0 exponent floor(log2 amax) - 2 kept in 1..254, 127 for an
 *     all-zero block, elements rounded to nearest even on the E2M1 grid and
 *     saturated at 6 -- so that both operands of the indexer's QK product are
 *     FP4, the lightning indexer's FP4 QK path of [CSDN] CSA step 2 and
 *     其他辅助设计; with MXFP4 keys only).
 *     Arithmetic is fp32 (bf16 x bf16 products accumulate in fp32; fp8 and FP4
 *     keys against a bf16 query are widened to bf16 exactly first; FP4 x FP4
 *     products with their block scales run on the scaled FP4 MFMA, exact
 *     before the fp32 sum).
 *   - Return codes: CSA_OK, CSA_INVALID_ARG (a null pointer that must not be
 *     null, a negative or inconsistent size), CSA_UNSUPPORTED (a valid
 *     combination with no kernel instantiation), CSA_WORKSPACE_TOO_SMALL,
 *     CSA_HIP_ERROR (a launch failed). Argument checks finish before the first
 *     HIP call, so a rejected call touches neither the device nor the stream.
 *     csa_last_error() returns the calling thread's message for its last
 *     failed call. No C++ exception crosses this boundary.
 *   - A pointer may be NULL when the call reads or writes nothing through it
 *     (no sequence or query, no compressed entry, no window row): such calls
 *     return CSA_OK and launch nothing.
 *   - Device-side data (indices, positions, lengths) is not validated on the
 *     host; kernels clamp it: an index outside [0, N_max) is skipped, a
 *     length is clamped to its buffer, a position to the rows that exist.
 *   - Results are deterministic and batch invariant: reductions run in a
 *     fixed order and split counts depend on per-sequence shape arguments
 *     only, never on the batch size or on which sequence is which.
 */
#ifndef CSA_HCA_H
#define CSA_HCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_HCA_VERSION 1

enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2, CSA_MXFP4 = 3, CSA_KV_FP8 = 4, CSA_BF16_MXFP4 = 5 };

enum {
  CSA_OK = 0,
  CSA_INVALID_ARG = -1,
  CSA_UNSUPPORTED = -2,
  CSA_WORKSPACE_TOO_SMALL = -3,
  CSA_HIP_ERROR = -4
};

/* csa_compress flags */
enum { CSA_OVERLAP = 1, CSA_JOINT_SOFTMAX = 2 };

/* qk_norm_rope flags */
enum { CSA_RMSNORM = 1, CSA_ROPE = 2, CSA_ROPE_INVERSE = 4 };

int csa_hca_version(void);
const char* csa_last_error(void);

/*
 * csa_compress — KV compression, [CSDN] CSA step 1 (the CComp_i equation).
 *
 * For every sequence b < B and block i in [blk_begin, blk_end), channel c < d:
 *   out[b, i, c] = sum_j softmax_j(Za[t_a(j), c] + Ba[j, c]) * Ca[t_a(j), c]
 *                + sum_j softmax_j(Zb[t_b(j), c] + Bb[j, c]) * Cb[t_b(j), c]
 * with t_a(j) = m*i + j, t_b(j) = m*(i-1) + j, j < m; the second (overlap)
 * term is present only with CSA_OVERLAP and i >= 1. With CSA_JOINT_SOFTMAX
 * (requires CSA_OVERLAP) one softmax runs over all 2m logits of both blocks.
 *
 *   Ca, Cb, Za, Zb : [B, n_rows, d] in in_dt; row r of sequence b holds token
 *                    t = tok_begin + r. Cb, Zb, Bb may be NULL without
 *                    CSA_OVERLAP (single-branch compression, as for HCA).
 *   Ba, Bb         : [m, d] fp32 positional biases (index j = position in block).
 *   out            : [B, out_cap, d] in out_dt; only rows [blk_begin, blk_end)
 *                    are written (decode appends one block: blk_end-1 .. blk_end).
 * Requirements: m*blk_end <= tok_begin + n_rows (a block is formed only from m
 * complete tokens: trailing tokens form no entry, [LQNN] section 5);
 * m*blk_begin >= tok_begin, and with CSA_OVERLAP and blk_begin >= 1 also
 * m*(blk_begin-1) >= tok_begin; blk_end <= out_cap; 1 <= m <= 1024.
 * Supported: in_dt in {F32, BF16}, out_dt in {F32, BF16, KV_FP8 (d > 64; out
 * rows are d + 64 bytes: channels below d-64 rounded to E4M3 to nearest even,
 * saturating at +-448, the last 64 to bf16)}, d % 8 == 0.
 */
int csa_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb,
                 const float* Ba, const float* Bb, void* out,
                 int64_t B, int64_t n_rows, int64_t tok_begin, int d, int m,
                 int64_t blk_begin, int64_t blk_end, int64_t out_cap,
                 int flags, int in_dt, int out_dt, void* stream);

/*
 * indexer_score — lightning-indexer scores, [CSDN] CSA step 2.
 *
 * For query t of sequence b at position p = q_pos[b, t], the visible entries
 * are i < V = min(n_comp[b], floor((p+1)/m), N_max), and
 *   scores[b, t, i] = sum_h w[b, t, h] * max(0, sigma_i * <q_idx[b,t,h,:], k_idx[b,i,:]>)
 * where sigma_i = k_scale[b, i] for fp8 keys and 1 otherwise (MXFP4 block
 * scales are part of the key values).
 *
 *   q_idx   : [B, Tq, H_I, D_I] in q_dt          w      : [B, Tq, H_I] fp32
 *   k_idx   : [B, N_max, D_I] in k_dt (MXFP4: [B, N_max, D_I/2] bytes)
 *   k_scale : fp8 keys: [B, N_max] fp32; MXFP4 keys: [B, N_max, D_I/32] E8M0
 *             bytes, each in 1..254 (0 and the NaN byte 255 are not
 *             supported; the elements widen to bf16 exactly for bytes
 *             2..252, beyond which the largest or smallest magnitudes leave
 *             bf16's normal range); NULL otherwise. 4-byte aligned.
 *   q_pos   : [B, Tq] int32                      n_comp : [B] int32
 *   scores  : [B, Tq, N_max] fp32; entries i >= V are left unspecified.
 * Supported: (H_I, D_I) in {(64, 128) with q_dt BF16 and k_dt BF16, FP8_E4M3
 * or MXFP4, (64, 128) with q_dt BF16_MXFP4 and k_dt MXFP4 (the query's
 * quantised values take q_idx's place in the sum above), (4, 32) with
 * q_dt = k_dt = F32}. N_max <= 2^24.
 */
int indexer_score(const void* q_idx, const float* w, const void* k_idx, const void* k_scale,
                  const int32_t* q_pos, const int32_t* n_comp,
                  int64_t B, int64_t Tq, int H_I, int D_I, int64_t N_max, int m,
                  int q_dt, int k_dt, float* scores, void* stream);

/*
 * csa_compress_indexer_score — a decode step's csa_compress and indexer_score
 * in one call. The two are independent: the scan reads the indexer keys (a
 * separate input, one key per entry, which may include the new entry's),
 * never the main-KV row being written, so kv_out must not overlap q_idx, w,
 * k_idx, k_scale or scores (overlap is undefined). Arguments are those of csa_compress followed by
 * those of indexer_score (Bc is csa_compress's B, m_c its m); results are
 * bit for bit those of the two calls. Where the scan takes the bf16-key path
 * (Tq < 8) and the compression is bf16 in, bf16 or KV_FP8 out, with the
 * overlap branch or m < 16, the compression's few workgroups ride in the
 * scan's launch; otherwise the two run in turn.
 */
int csa_compress_indexer_score(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                               const float* Bb, void* kv_out, int64_t Bc, int64_t n_rows, int64_t tok_begin, int d,
                               int m_c, int64_t blk_begin, int64_t blk_end, int64_t out_cap, int flags, int in_dt,
                               int out_dt, const void* q_idx, const float* w, const void* k_idx, const void* k_scale,
                               const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq, int H_I, int D_I,
                               int64_t N_max, int m, int q_dt, int k_dt, float* scores, void* stream);

/*
 * indexer_topk — top-k selection over indexer scores, [CSDN] CSA step 2.
 *
 * Row (b, t) keeps K' = min(top_k, V) entries with the largest scores among
 * i < V (V as in indexer_score); equal scores go to the lower index. The
 * kept indices are written to topk_idx[b, t, 0..K'-1] in ascending index
 * order and the rest of the row is -1. topk_score (nullable) receives the
 * matching scores (rest: -inf). Exact: no approximate selection.
 *   scores : [B, Tq, N_max] fp32     topk_idx : [B, Tq, top_k] int32
 * Supported: 1 <= top_k <= 4096, N_max <= 2^24.
 */
int indexer_topk(const float* scores, const int32_t* q_pos, const int32_t* n_comp,
                 int64_t B, int64_t Tq, int64_t N_max, int m, int top_k,
                 int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes, void* stream);
size_t indexer_topk_workspace_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k);

/* indexer_score_topk — indexer_score followed by indexer_topk, the scores
 * living in the workspace. Same arguments and support as the two calls, and
 * the same results.
 * The workspace also carries, per query row, a 2048-bin histogram of the
 * scores' top 11 bits that the scan fills and the top-k reads to find the bin
 * holding the k-th score. The top-k counts the candidates it finds against
 * the scores themselves, so the histogram is only a hint: results never
 * depend on the workspace's contents on entry. Decode scans (Tq < 8) add to
 * the histogram and the top-k clears it after use, so a call runs its fast
 * path when the workspace was zero-filled once or last used by a call of the
 * same shape; otherwise it selects from the full score rows (exact, slower).
 * Prefill scans (Tq >= 8) write the histogram whole. */
int indexer_score_topk(const void* q_idx, const float* w, const void* k_idx, const void* k_scale,
                       const int32_t* q_pos, const int32_t* n_comp,
                       int64_t B, int64_t Tq, int H_I, int D_I, int64_t N_max, int m, int top_k,
                       int q_dt, int k_dt, int32_t* topk_idx, float* topk_score,
                       void* ws, size_t ws_bytes, void* stream);
size_t indexer_score_topk_workspace_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k);

/*
 * csa_compress_indexer_score_topk — a decode step's front half, [CSDN] CSA
 * steps 1 and 2 in one call: csa_compress (the entry the new token completes)
 * and indexer_score_topk. Arguments are those of csa_compress followed by
 * those of indexer_score_topk (Bc is csa_compress's B, m_c its m); the
 * workspace is indexer_score_topk_workspace_bytes(B, Tq, N_max, top_k) and
 * behaves as there. Results are bit for bit those of the separate calls. The
 * compression and the scan are independent: the scan reads the indexer keys,
 * a separate input, never the main-KV row being written, so kv_out must not
 * overlap q_idx, w, k_idx, k_scale or the workspace (overlap is undefined).
 * Where the scan takes the bf16-key path (Tq < 8) and the compression is bf16
 * in, bf16 or KV_FP8 out, with the overlap branch or m < 16, the
 * compression's few workgroups ride in the scan's launch.
 */
int csa_compress_indexer_score_topk(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                                    const float* Bb, void* kv_out, int64_t Bc, int64_t n_rows, int64_t tok_begin,
                                    int d, int m_c, int64_t blk_begin, int64_t blk_end, int64_t out_cap, int flags,
                                    int in_dt, int out_dt, const void* q_idx, const float* w, const void* k_idx,
                                    const void* k_scale, const int32_t* q_pos, const int32_t* n_comp, int64_t B,
                                    int64_t Tq, int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt, int k_dt,
                                    int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes, void* stream);

/*
 * Shared-KV multi-query attention with a sink ([CSDN] CSA step 3 and HCA;
 * [LIDUOS] window and sink). For one query token and every head h < H over a
 * multiset R of rows (each row is both key and value):
 *   l_r = scale * <q_h, r>,  M = max(sink_h, max_r l_r),
 *   Z_h = e^{sink_h - M} + sum_r e^{l_r - M},
 *   out_h = sum_r e^{l_r - M} r / Z_h,   lse_h = M + ln Z_h.
 * sink may be NULL (no sink: sink_h = -inf). With R empty and no sink,
 * out_h = 0 and lse_h = -inf. Rows present in two sources count twice.
 * Supported: D = 512 with kv_dt BF16 and 49 <= H <= 64, or D = 64 with
 * kv_dt F32 and 1 <= H <= 16; out_dt in {F32, BF16}; q has the dtype kv_dt.
 * The decode entry points (sparse_mqa_decode, hca_dense_mqa) also take
 * kv_dt KV_FP8 (D = 512, 49 <= H <= 64, bf16 q): kv_comp and kv_win rows are
 * then D + 64 = 576 bytes, 16-byte aligned.
 * scale must be positive and finite (CSA_INVALID_ARG otherwise); q and out
 * must be 16-byte aligned.
 */

/* sparse_mqa_decode — one query per sequence (position: the last token).
 *   q      : [B, H, D]           kv_comp : [B, N_max, D]
 *   topk_idx : [B, top_k] int32, -1 = empty slot; rows kv_comp[b, idx]
 *   kv_win : [B, W, D]; rows 0 .. win_len[b]-1 are the window (any order)
 *   win_len: [B] int32           sink    : [H] fp32 (nullable)
 *   out    : [B, H, D] in out_dt lse     : [B, H] fp32 (nullable)
 * R = {kv_comp[b, i] : i in topk_idx[b]} + the win_len[b] window rows. */
int sparse_mqa_decode(const void* q, const void* kv_comp, const int32_t* topk_idx,
                      const void* kv_win, const int32_t* win_len, const float* sink, float scale,
                      int64_t B, int H, int D, int64_t N_max, int top_k, int W,
                      int kv_dt, int out_dt, void* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream);
size_t sparse_mqa_decode_workspace_bytes(int64_t B, int H, int D, int top_k, int W);

/* sparse_mqa_decode_multi — Tq consecutive query tokens per sequence in one
 * decode step (the pages' configuration trains a depth-1 multi-token
 * predictor, [LQNN] section 3: a step can verify a drafted token beside the
 * current one). Query t of sequence b (t < Tq, the last Tq tokens, oldest
 * first) attends its own top-k rows and its own window:
 *   q      : [B, Tq, H, D]       topk_idx : [B, Tq, top_k] int32 (-1 = empty)
 *   kv_win : [B, W + Tq - 1, D]  a buffer of the latest raw tokens, oldest
 *            first; rows 0 .. wl-1 are valid (wl = min(win_len[b], W + Tq - 1))
 *            and row wl-1 is the newest token. Query t's own token is row
 *            wl - Tq + t; its window is the (at most) W rows ending there.
 *   out    : [B, Tq, H, D]       lse : [B, Tq, H] (nullable)
 * Everything else as sparse_mqa_decode, which is this call with Tq = 1.
 * 1 <= Tq <= 64. */
int sparse_mqa_decode_multi(const void* q, const void* kv_comp, const int32_t* topk_idx, const void* kv_win,
                            const int32_t* win_len, const float* sink, float scale, int64_t B, int64_t Tq, int H,
                            int D, int64_t N_max, int top_k, int W, int kv_dt, int out_dt, void* out, float* lse,
                            void* ws, size_t ws_bytes, void* stream);
size_t sparse_mqa_decode_multi_workspace_bytes(int64_t B, int64_t Tq, int H, int D, int top_k, int W);

/*
 * csa_decode_step — one CSA decode step for Tq query tokens per sequence,
 * [CSDN] CSA steps 1-3 in the pages' order: the compression of the blocks
 * the step's tokens complete (csa_compress into kv_comp, rows [blk_begin,
 * blk_end)), the indexer scores, the top-k and the shared-KV MQA with the
 * window and the sink. Results are bit for bit those of csa_compress,
 * indexer_score_topk and sparse_mqa_decode_multi in turn.
 *   compression: as csa_compress with B = B, out = kv_comp, out_cap = N_max,
 *                out_dt = kv_dt, d = D (blk_begin == blk_end: none).
 *   indexer    : as indexer_score_topk (q_idx [B, Tq, H_I, D_I], q_pos [B, Tq]);
 *                topk_idx [B, Tq, top_k] and topk_score (nullable) are outputs.
 *   attention  : as sparse_mqa_decode_multi (q [B, Tq, H, D], kv_win
 *                [B, W + Tq - 1, D], win_len [B], out [B, Tq, H, D], lse nullable).
 *   ws         : csa_decode_step_workspace_bytes(...); the scores occupy its
 *                first B * Tq * N_max * 4 bytes. As with indexer_score_topk,
 *                results never depend on its contents on entry, and a
 *                zero-filled workspace (or one last used by a call of the same
 *                shape) takes the fast path.
 * The step is four launches: the scan (with the compression's workgroups and,
 * for bf16 indexer queries, the top-k's digit histogram), the top-k, the
 * split attention and the merge of the splits. Ordinary stream launches: the
 * step can be captured in a HIP graph. Two calls that overlap on one device
 * (two streams) must not share a workspace.
 */
int csa_decode_step(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba, const float* Bb,
                    int64_t n_rows, int64_t tok_begin, int d, int m_c, int64_t blk_begin, int64_t blk_end,
                    int flags, int in_dt, const void* q_idx, const float* w, const void* k_idx,
                    const void* k_scale, const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq,
                    int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt, int k_dt, const void* q,
                    void* kv_comp, const void* kv_win, const int32_t* win_len, const float* sink, float scale, int H,
                    int D, int W, int kv_dt, int out_dt, int32_t* topk_idx, float* topk_score, void* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream);
size_t csa_decode_step_workspace_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k, int H, int D, int W);

/*
 * csa_decode_step_qk — csa_decode_step with the attention's prologue and
 * epilogue ([CSDN] 其他辅助设计: RMSNorm of the queries before the core
 * attention, rotary encoding of the last rope_dims dims only; [LIDUOS] 1M
 * Context 的结构与取舍: the output takes the inverse rotation, since rows are
 * both key and value). q holds the raw queries; the step attends with
 *   q' = rotate(RMSNorm(q) * q_gamma, q_pos)  (as qk_norm_rope with
 *        CSA_RMSNORM | CSA_ROPE and pos = q_pos, each part per qk_flags),
 * and writes out = rotate^-1(attention(q'), q_pos) (CSA_ROPE only).
 *   q_gamma : [D] fp32 or NULL (ones); eps, rope_dims, rope_theta as in
 *             qk_norm_rope; qk_flags a subset of CSA_RMSNORM | CSA_ROPE.
 *   ws      : csa_decode_step_qk_workspace_bytes(...) bytes.
 * With D = 512 bf16 or KV_FP8 rows and rope_dims <= 128, the prologue runs on
 * the attention kernel's query registers and the inverse rotation on the
 * merged output before its one rounding to out_dt; otherwise qk_norm_rope's
 * kernels run around the attention. q' is rounded to bf16 once in either
 * form.
 */
int csa_decode_step_qk(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                       const float* Bb, int64_t n_rows, int64_t tok_begin, int d, int m_c, int64_t blk_begin,
                       int64_t blk_end, int flags, int in_dt, const void* q_idx, const float* w, const void* k_idx,
                       const void* k_scale, const int32_t* q_pos, const int32_t* n_comp, int64_t B, int64_t Tq,
                       int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt, int k_dt, const void* q,
                       void* kv_comp, const void* kv_win, const int32_t* win_len, const float* sink, float scale,
                       int H, int D, int W, int kv_dt, int out_dt, int32_t* topk_idx, float* topk_score, void* out,
                       float* lse, const float* q_gamma, float eps, int rope_dims, float rope_theta, int qk_flags,
                       void* ws, size_t ws_bytes, void* stream);
size_t csa_decode_step_qk_workspace_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k, int H, int D, int W);

/*
 * csa_decode_step_noalloc — csa_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc). Arguments and results are those of
 * csa_decode_step without ws / ws_bytes: the scratch is a device array of
 * CSA_STEP_SCRATCH_BYTES inside the library, one per device, held from the
 * library's load until the process ends. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).
 *   Limit: csa_decode_step_workspace_bytes(B, Tq, N_max, top_k, H, D, W) must
 *   not exceed CSA_STEP_SCRATCH_BYTES (a C2-sized step, 32 sequences of 128K
 *   tokens, needs about 30 MB); above it the call returns
 *   CSA_WORKSPACE_TOO_SMALL before any GPU work.
 *   Every call on a device shares that device's array: calls that overlap on
 *   one device (two streams, two threads) race and must be serialised by the
 *   caller. Results never depend on what the array holds; the first call of a
 *   shape on a device clears the region it uses with a fill kernel (no
 *   hipMemset), so later calls of that shape take the fast path.
 */
#define CSA_STEP_SCRATCH_BYTES ((size_t)64 << 20)
int csa_decode_step_noalloc(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                            const float* Bb, int64_t n_rows, int64_t tok_begin, int d, int m_c, int64_t blk_begin,
                            int64_t blk_end, int flags, int in_dt, const void* q_idx, const float* w,
                            const void* k_idx, const void* k_scale, const int32_t* q_pos, const int32_t* n_comp,
                            int64_t B, int64_t Tq, int H_I, int D_I, int64_t N_max, int m, int top_k, int q_dt,
                            int k_dt, const void* q, void* kv_comp, const void* kv_win, const int32_t* win_len,
                            const float* sink, float scale, int H, int D, int W, int kv_dt, int out_dt,
                            int32_t* topk_idx, float* topk_score, void* out, float* lse, void* stream);

/*
 * csa_trace_phases — instrumentation of the decode calls, for timing their
 * phases with the caller's HIP events (no synchronisation, nothing
 * allocated). While set on the calling thread, csa_decode_step,
 * csa_decode_step_noalloc, hca_dense_mqa, indexer_score_topk and
 * csa_compress_indexer_score_topk record events[i] with hipEventRecord on
 * the call's stream at these points:
 *   [0] before the first launch   [1] after the indexer scan launch
 *   [2] after the top-k (or the fused top-k + attention + merge launch)
 *   [3] after the attention kernel, before its split merge   [4] at the end.
 * A phase a call does not have is recorded where it would start, so every
 * event of a traced call is recorded, in order. events: n (0..5) hipEvent_t
 * handles owned by the caller; n = 0 turns tracing off.
 * Errors: CSA_INVALID_ARG for n outside 0..5 or a NULL array with n > 0.
 */
int csa_trace_phases(void* const* events, int n);

/* sparse_mqa_prefill — Tq queries of one sequence.
 *   q      : [Tq, H, D]          kv_comp : [N, D]
 *   topk_idx : [Tq, top_k] int32 (-1 = empty)
 *   kv_tok : [T_tok, D] raw per-token KV; query t at position p = q_pos[t]
 *            uses window rows kv_tok[max(0, p-W+1) .. p] ([LIDUOS]: the latest
 *            W raw tokens, the current one included)
 *   out    : [Tq, H, D]          lse : [Tq, H] (nullable)
 * Supported: top_k + W <= 2048 (f32 rows: also top_k <= 1024). Needs no
 * workspace. */
int sparse_mqa_prefill(const void* q, const void* kv_comp, const int32_t* topk_idx,
                       const void* kv_tok, const int32_t* q_pos, const float* sink, float scale,
                       int64_t Tq, int H, int D, int64_t N, int64_t T_tok, int top_k, int W,
                       int kv_dt, int out_dt, void* out, float* lse,
                       void* ws, size_t ws_bytes, void* stream);
size_t sparse_mqa_prefill_workspace_bytes(int64_t Tq, int H, int D, int top_k, int W);

/* hca_dense_mqa — HCA decode: one query per sequence over ALL visible
 * compressed entries i < V = min(n_comp[b], floor((q_pos[b]+1)/m), N_max)
 * plus the win_len[b] window rows. Shapes as in sparse_mqa_decode, with
 * n_comp, q_pos : [B] int32. */
int hca_dense_mqa(const void* q, const void* kv_comp, const int32_t* n_comp, const int32_t* q_pos,
                  int m, const void* kv_win, const int32_t* win_len, const float* sink, float scale,
                  int64_t B, int H, int D, int64_t N_max, int W,
                  int kv_dt, int out_dt, void* out, float* lse,
                  void* ws, size_t ws_bytes, void* stream);
size_t hca_dense_mqa_workspace_bytes(int64_t B, int H, int D, int64_t N_max, int W);

/*
 * hca_decode_step — one HCA decode step ([CSDN] HCA: every m' tokens become
 * one entry, and a query attends densely to every entry it can see, plus the
 * [LIDUOS] window and sink): csa_compress of the blocks the step's token
 * completes, single branch (Cb, Zb, Bb NULL, no flags), into kv_comp rows
 * [blk_begin, blk_end), then hca_dense_mqa over the updated kv_comp.
 *   compression: as csa_compress with B, out = kv_comp, out_cap = N_max,
 *                out_dt = kv_dt, d = D (blk_begin == blk_end: none).
 *   attention  : as hca_dense_mqa (q [B, H, D], n_comp, q_pos [B], m).
 *   ws         : hca_decode_step_workspace_bytes(...) bytes (the split
 *                partials), 256-byte aligned; any contents on entry.
 * With D = 512, bf16 or KV_FP8 rows and one appended block of bf16 inputs,
 * the append rides in the attention's launch: the workgroup whose split
 * holds the new entry computes it first, stores it, and then gathers its
 * rows; the splits then merge in a second launch. Otherwise csa_compress's
 * kernel runs first. Results match the separate calls up to the summation
 * order of the new entry (fp32, then rounded to kv_dt).
 */
int hca_decode_step(const void* Ca, const void* Za, const float* Ba, int64_t n_rows, int64_t tok_begin, int d,
                    int m_c, int64_t blk_begin, int64_t blk_end, int in_dt, const void* q, void* kv_comp,
                    const int32_t* n_comp, const int32_t* q_pos, int m, const void* kv_win, const int32_t* win_len,
                    const float* sink, float scale, int64_t B, int H, int D, int64_t N_max, int W, int kv_dt,
                    int out_dt, void* out, float* lse, void* ws, size_t ws_bytes, void* stream);
size_t hca_decode_step_workspace_bytes(int64_t B, int H, int D, int64_t N_max, int W);

/* hca_prefill — HCA for Tq queries of one sequence ([CSDN] HCA: dense
 * attention over every compressed entry a query can see, plus the
 * [LIDUOS] window and sink). Query t at position p = q_pos[t] attends to
 *   R = kv_comp[0 .. V-1] + kv_tok[max(0, p-W+1) .. min(p, T_tok-1)],
 *   V = min(N, floor((p+1)/m))  (an entry exists once its m tokens are in).
 *   q      : [Tq, H, D]          kv_comp : [N, D] (the HCA entries, m = m')
 *   kv_tok : [T_tok, D] raw per-token KV      q_pos : [Tq] int32, >= 0
 *   out    : [Tq, H, D] in out_dt             lse   : [Tq, H] (nullable)
 * No limit on V beyond N + W <= 2^24 (rows are read in order, not from a
 * table). Needs no workspace (ws may be NULL). */
int hca_prefill(const void* q, const void* kv_comp, const void* kv_tok, const int32_t* q_pos, const float* sink,
                float scale, int64_t Tq, int H, int D, int64_t N, int m, int64_t T_tok, int W, int kv_dt,
                int out_dt, void* out, float* lse, void* ws, size_t ws_bytes, void* stream);
size_t hca_prefill_workspace_bytes(int64_t Tq, int H, int D, int64_t N, int W);

/*
 * qk_norm_rope — the attention's prologue and epilogue: QK RMSNorm and
 * partial rotary position encoding ([CSDN] 其他辅助设计: RMSNorm on queries
 * and keys before the core attention, rotation of the last 64 dims only),
 * and the inverse rotation of the output ([LIDUOS] 1M Context 的结构与取舍:
 * rows are both key and value, so the output is rotated back).
 *
 * For every row x[t, h, :] (D values), in this order:
 *   CSA_RMSNORM      : x <- x / sqrt(mean(x^2) + eps) * gamma  (gamma [D] fp32,
 *                      NULL = all ones);
 *   CSA_ROPE         : with s = D - rope_dims, the pair (x[s+2i], x[s+2i+1])
 *                      is rotated by the angle pos[t] * rope_theta^(-2i/rope_dims);
 *   CSA_ROPE_INVERSE : the same pairs rotated by minus that angle.
 *   x, out : [T, H, D] in dt (F32 or BF16), 16-byte aligned; out may be x.
 *   pos    : [T] int32 (needed with a rotation).
 * Arithmetic is fp32; angles are formed and reduced in double precision.
 * Supported: D % 8 == 0, D <= 512; rope_dims even in [2, D]. CSA_ROPE and
 * CSA_ROPE_INVERSE together are CSA_INVALID_ARG.
 */
int qk_norm_rope(const void* x, void* out, const float* gamma, const int32_t* pos, int64_t T, int H, int D,
                 int rope_dims, float eps, float rope_theta, int flags, int dt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_HCA_H */
