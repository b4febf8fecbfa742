// Shared-KV multi-query attention with a sliding window and a sink, for
// gfx950 (MI355X). One kernel template serves CSA sparse decode, CSA sparse
// prefill and HCA dense decode; they differ only in where the rows of the
// attended multiset come from.
//
// What is computed (DeepSeek V4 脱离 CUDA 全栈国产化, deepseek.csdn.net,
// section 二, CSA step 3 "共享 KV MQA" and the HCA paragraph; liduos.com
// deepseek-v4-engineering-tradeoffs, "1M Context 的结构与取舍", for the
// window and the sink): per query token and head h, a softmax over
// l_r = scale * <q_h, r> for every row r of the multiset plus a sink logit,
// then the weighted sum of the rows (each row is key and value at once).
//
// Design (MI355X-first):
//  * A workgroup owns one query token and a contiguous range of row slots (a
//    "split"). Rows are processed in tiles of 32 held row-major in LDS with
//    their 16-byte chunks XOR-swizzled.
//  * S^T = R Q^T on v_mfma_f32_16x16x32_bf16 (M = 16 rows, N = 16 heads,
//    K = 32 dims); Q stays in registers. The accumulator layout gives each
//    lane 8 rows of one head, which is exactly the P operand of the next
//    product once the 32 tile rows are taken in a permuted K order.
//  * O += P R on the same MFMA (M = 16 heads, N = 16 dims, K = 32 rows); its
//    R operand (4 consecutive rows of one dim per read) comes from the
//    row-major tile through ds_read_b64_tr_b16, in the same K order.
//  * Online softmax in the exp2 domain with a lazily moved reference: the O
//    accumulators are only rescaled when a logit exceeds the reference by
//    RESCALE_SLACK, which after the first tile is rare.
//  * Splits write unnormalised (O, m, l) partials (exp2 domain); a combine
//    kernel merges them in fixed split order and adds the sink. Split sizes
//    depend only on per-query shape arguments: results are batch invariant.
//  * bf16 rows of 512 dims (the model's shape) run attn_bf16_kernel: eight
//    waves, rows moved HBM -> LDS by DMA. fp32 rows of small dims (the tiny
//    reference shapes) run attn_f32_kernel on v_mfma_f32_16x16x4f32.
#include <type_traits>

#include "attn_core.h"
#include "compress_entry.h"
#include "kernels.h"

namespace csa {

// The HCA decode step's append (see AttnLaunch), as kernel arguments.
struct HcaAppend {
  const uint16_t* Ca;  // NULL: none
  const uint16_t* Za;
  const float* Ba;
  int64_t n_rows, tok_begin, blk;
  int m;
  void* out;  // kv_comp
};

template <int SRC, bool KV8>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_kernel(const uint16_t* __restrict__ q, RowSrc src, const int32_t* __restrict__ win_len,
                 const int32_t* __restrict__ n_comp, const int32_t* __restrict__ q_pos, int m_rate,
                 const float* __restrict__ sink, float scale_log2, int H, int slots, int split_rows,
                 float* __restrict__ part_o, float* __restrict__ part_ml, void* __restrict__ out,
                 float* __restrict__ lse, int out_dt, HcaAppend app, QkArgs qk) {
  using namespace bfk;
  constexpr int SROWB = DecRows<KV8>::SROWB, TB = DecRows<KV8>::TB;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NBUF * TB];
  __shared__ __attribute__((aligned(16))) f32x4_t xchg[NW][2][64];
  __shared__ __attribute__((aligned(16))) int tab[SRC == SRC_HCA_DEC ? 4 : TAB_MAX];
  __shared__ int cnt[2 * TAB_MAX / 64];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = l >> 4, l16 = l & 15;
  const int hg = w & 3, dh = w >> 2;
  const int64_t qi = blockIdx.x;  // query (decode: sequence)
  const int sp = blockIdx.y;      // split
  const int nsplit = gridDim.y;
  const int head = hg * 16 + l16;  // this lane's head in S^T / P / softmax

  QRows rr = query_rows<SRC, SROWB>(src, win_len, n_comp, q_pos, m_rate, qi, sp, slots, split_rows);

  // ---- Q^T operand (B of S^T = R Q^T): lane (head, G), dims 256 dh + 32 s + 8 G .. +7,
  // loaded unconditionally (the head is clamped) and zeroed after (loads
  // under a branch would each be waited for); for a sparse split the loads go
  // out right behind the split's slot codes, which then need not wait for them
  bf16x8_t qb[8];
  const bool hok = head < H;
  auto load_q = [&]() {
    const uint16_t* qp = q + (qi * H + (hok ? head : 0)) * (int64_t)D + dh * 256 + G * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[s] = as_bf16x8(ld16(qp + s * 32));
  };
  if constexpr (SRC != SRC_HCA_DEC)
    rr.n_rows = build_row_table<SRC, NT, TR, 1>(src, rr, qi, tab, cnt, nullptr, load_q);
  else
    load_q();
  if (!hok)
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[s] = as_bf16x8(u32x4_t{0, 0, 0, 0});
  if (SRC == SRC_SPARSE_DEC && qk.flags) qk_prologue(qb, reinterpret_cast<float*>(xchg), qk, qi);
  if constexpr (SRC == SRC_HCA_DEC) {
    if (app.Ca && sp == (int)(app.blk / split_rows)) {
      // the step's new entry is in this split: computed here and stored, and
      // the store complete, before any row of the split is gathered (the
      // gathers read it back through this CU's path to the cache)
      block_entry_wg<DT_BF16, KV8 ? DT_KV_FP8 : DT_BF16, NT>(app.Ca, app.Za, app.Ba,
                                                            qi * app.n_rows + (app.m * app.blk - app.tok_begin), D,
                                                            app.m, app.out, qi * src.N_max + app.blk,
                                                            reinterpret_cast<float*>(ring));
    }
  }

  f32x4_t o[16];
  float m_ref, l_run;
  dec_tiles<SRC, KV8>(rr, tab, ring, xchg, qb, scale_log2, o, m_ref, l_run);

  // ---- epilogue: O rows are heads 16 hg + 4G + r; their (m, l) live in lanes 4G + r
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  float mrr[4], lrr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mrr[r] = __shfl(m_ref, G * 4 + r, 64);
    lrr[r] = __shfl(l_run, G * 4 + r, 64);
  }
  const int dbase = dh * 256 + l16;
  if (part_o != nullptr) {
    const int64_t pbase = (qi * nsplit + sp) * (int64_t)H;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = hg * 16 + G * 4 + r;
      if (h >= H) continue;
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) part_o[(pbase + h) * D + dbase + nt * 16] = o[nt][r];
    }
    if (dh == 0 && G == 0 && head < H) {
      part_ml[(pbase + head) * 2 + 0] = m_ref;
      part_ml[(pbase + head) * 2 + 1] = l_run;
    }
  } else {
    float rope_c = 1.0f, rope_s = 0.0f;  // the output's inverse rotation: pair `lane`'s angle
    if (SRC == SRC_SPARSE_DEC) rope_lane(qk, qi, rope_c, rope_s);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = hg * 16 + G * 4 + r;
      if (h >= H) continue;
      const float s2 = sink ? sink[h] * LOG2E_F : -INFINITY;
      const float M = fmaxf(mrr[r], s2);
      float fac = 0.0f;
      if (M != -INFINITY) {
        const float a = exp2f(mrr[r] - M);
        fac = a / (lrr[r] * a + exp2f(s2 - M));
      }
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) {
        const int64_t oo = (qi * H + h) * (int64_t)D + dbase + nt * 16;
        float v = o[nt][r] * fac;
        if (SRC == SRC_SPARSE_DEC && (qk.flags & 2) && dh * 256 + nt * 16 + 16 > D - qk.R) {
          // the pair's other dim sits in the lane next door
          const int d = dbase + nt * 16, s0 = D - qk.R;
          const float other = shfl_xor(v, 1);
          const int src = d >= s0 ? (d - s0) >> 1 : 0;
          const float c = __shfl(rope_c, src, 64), sn = __shfl(rope_s, src, 64);
          if (d >= s0) v = (l16 & 1) ? v * c - other * sn : v * c + other * sn;
        }
        if (out_dt == DT_BF16)
          reinterpret_cast<uint16_t*>(out)[oo] = (uint16_t)f32_to_bf16(v);
        else
          reinterpret_cast<float*>(out)[oo] = v;
      }
    }
    if (lse && dh == 0 && G == 0 && head < H) {
      const float s2 = sink ? sink[head] * LOG2E_F : -INFINITY;
      const float M = fmaxf(m_ref, s2);
      float v = -INFINITY;
      if (M != -INFINITY) v = (M + log2f(l_run * exp2f(m_ref - M) + exp2f(s2 - M))) * LN2_F;
      lse[qi * H + head] = v;
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 prefill helpers
// ----------------------------------------------------------------------------

// Chunk swizzle of the prefill tiles (16-byte chunks; 64 banks of 4 bytes
// span 16 chunks): a 4-bit rotation of the row. Any 16 consecutive rows put
// one chunk in 16 distinct bank groups (the K reads of the QK chain), and the
// four rows 4i .. 4i+3 differ in the high bits, so a half-wave of transposed V
// reads (four rows x four aligned chunks) also covers all 64 banks once.
__device__ __forceinline__ int swz4(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ f32x16_t mfma32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ----------------------------------------------------------------------------
// bf16 prefill, rows split between the two waves of a head group
// ----------------------------------------------------------------------------
//
// Four waves, one per SIMD; wave w owns heads 32 (w%2) .. +31. For S the two
// waves of a head group split each 32-row tile: wave w computes S over all 512
// dims for rows 16 (w/2) .. +15 on v_mfma_f32_16x16x32_bf16 (Q^T of its 32
// heads, 128 registers, waits in accumulation registers). For O they split
// the dims: wave w accumulates O^T for dims 256 (w/2) .. +255 over all 32 rows
// on v_mfma_f32_32x32x16_bf16 (O^T in accumulation registers: a lane holds
// one head, so a rescale uses the lane's own factor and the epilogue packs 8
// consecutive dims per lane). The waves meet through P^T in LDS (bf16, [head][row],
// double-buffered by tile parity), so a tile needs one barrier.
//
// P of a tile is taken against the exponent reference the pair agreed on at
// the previous tile, which both waves hold without talking to each other. The
// fp32/bf16 range leaves room for that: P is allowed up to 2^GUARD. A tile
// with a logit more than GUARD above the reference (in particular the first
// tile with a finite logit) takes the slow path: the pair exchanges exact
// per-head maxima, moves the reference, rescales O and the running sums, and
// recomputes P.
//
// Software pipeline (iteration t): the QK products of tile t+1 are issued with
// the K reads of tile t+1 and the transposed V reads of tile t, then O += P V
// of tile t runs with the softmax of tile t+1 in the shadow of its products.
// One barrier per tile then covers the P^T exchange and the DMA ring.

namespace prs {
constexpr int D = 512, ROWB = 1024, TR = 32, NW = 4, NT = 256, NBUF = 4;
constexpr int TILEB = TR * ROWB;
constexpr int RPW = TR / NW;     // rows each wave gathers per tile
constexpr int TAB_MAX = 2048;
constexpr int PSTR = 40;         // bf16 per head row of a P^T buffer: 32 rows + 16 bytes of padding
constexpr float GUARD = 64.0f;   // log2 units a logit may sit above the shared reference
}  // namespace prs

template <int SRC, bool KV8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_prs_kernel(const uint16_t* __restrict__ q, RowSrc src, const int32_t* __restrict__ q_pos, int m_rate,
                const float* __restrict__ sink, float scale_log2, int H, int slots, void* __restrict__ out,
                float* __restrict__ lse, int out_dt) {
  using namespace prs;
  static_assert(SRC == SRC_SPARSE_PRE || SRC == SRC_HCA_PRE, "prefill row sources");
  // KV8 rows (448 E4M3 bytes, then the 64 RoPE dims as bf16: 576 bytes) sit
  // unswizzled in LDS at a 592-byte pitch, the second half of a tile 64
  // bytes further on, as in the decode kernel
  constexpr int SROWB = KV8 ? 576 : ROWB;
  constexpr int NOPE = 448;
  constexpr int PITCH = KV8 ? 592 : ROWB;
  constexpr int TB = KV8 ? TR * PITCH + 64 : TILEB;
  auto lrow = [](int r) { return KV8 ? r * PITCH + (r >> 4) * 64 : r * ROWB; };
  // the query's rows (64 heads x 1 KB) are staged from ring slot 2 on before
  // the first tiles reach slots 2 and 3
  constexpr int QOFF = 2 * TB;
  constexpr int RING = NBUF * TB > QOFF + 64 * ROWB ? NBUF * TB : QOFF + 64 * ROWB;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[RING];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[2][2][32 * PSTR];  // [tile parity][head group] P^T
  __shared__ __attribute__((aligned(16))) float lmx[2][2][2][64];          // [head group][row half][hq][lane]
  __shared__ __attribute__((aligned(16))) int flg[2][NW];                  // [tile parity][wave]: P must be redone
  __shared__ __attribute__((aligned(16))) int tab[SRC == SRC_HCA_PRE ? 4 : TAB_MAX];
  __shared__ int cnt[2 * TAB_MAX / 64];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = l >> 5, l32 = l & 31, g16 = l >> 4, l16 = l & 15;
  const int hg = w & 1, dh = w >> 1;
  const int64_t qi = blockIdx.x;
  // S / softmax layout: lane holds tile rows 16 dh + 4 g16 + i (i < 4) of heads
  // 32 hg + 16 hq + l16 (hq < 2). O^T layout: lane holds head 32 hg + l32 = the
  // softmax head of hq = (l >> 4) & 1, dims 256 dh + 32 nt + 8 (r/4) + 4 h + r%4.
  const int ohq = (l >> 4) & 1;

  QRows rr = query_rows<SRC, SROWB>(src, nullptr, nullptr, q_pos, m_rate, qi, 0, slots, slots);

  // ---- the first memory round trip carries everything that does not depend
  // on the row table: (sparse) the slots' top-k codes, by DMA into the
  // table's own words (top-k slots only; the window slots are arithmetic),
  // then the query's head rows, by DMA into LDS (one coalesced 1 KB row per
  // instruction; wave w takes heads w, w + 4, ..., rows past H repeat row
  // H - 1 so every wave issues QPW of them). Chunk c of head row h sits at
  // chunk c ^ (h & 15) of its LDS row, so the operand reads below (16 heads
  // at one dim offset) fall in 16 distinct bank groups.
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  if constexpr (SRC == SRC_SPARSE_PRE) {
    const int32_t* codes = src.idx + qi * src.top_k;
    const uint32_t tab_lds = (uint32_t)(uintptr_t)tab;
#pragma unroll
    for (int c = 0; c < TAB_MAX / 64; c += NW) {
      const int j0 = (c + w) * 64;  // this wave's 64 slots
      if (j0 < src.top_k)
        dma_dword(uniform_ptr(codes), (uint32_t)(min(j0 + l, src.top_k - 1) * 4), tab_lds + (uint32_t)(j0 * 4));
    }
  }
  constexpr int QPW = 64 / NW;  // head rows per wave
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int hh = min(w + NW * i, H - 1);
    dma_row(uniform_ptr(reinterpret_cast<const uint8_t*>(q + (qi * H + hh) * (int64_t)D)),
            (uint32_t)((l ^ ((w + NW * i) & 15)) * 16), ring_lds + QOFF + (w + NW * i) * ROWB);
  }

  // sparse: a row table in LDS; HCA: rows are entries 0 .. V-1 and then the
  // window tokens, addressed arithmetically
  int n_comp_rows = rr.len1;
  if constexpr (SRC == SRC_SPARSE_PRE) {
    vm_barrier<QPW>();  // every wave's codes have landed (only query rows in flight)
    // compacted in place: every code is read before the first table write
    rr.n_rows = build_row_table_from<SRC, NT, TR, TAB_MAX / NT>(
        src, rr, qi, tab, cnt, &n_comp_rows, [&](int j) { return tab[j]; }, [] {});
  }
  const int n_rows = rr.n_rows;
  const int ntiles = (n_rows + TR - 1) / TR;
  // table entries below ncb are compressed rows, the rest window rows (the
  // padded tail repeats the last row, so it belongs to the last row's cache)
  const int ncb = (n_rows == n_comp_rows) ? ntiles * TR : n_comp_rows;
  // rows of both caches below 2^22: a row's byte offset fits the DMA's 32-bit
  // lane offset, so rows from one cache need no per-row 64-bit address
  const bool off32 = src.N_max < (1 << 22) && src.T_tok < (1 << 22);

  uint32_t voff[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) voff[i] = KV8 ? (uint32_t)(l * 16) : (uint32_t)((l ^ swz4(RPW * w + i)) * 16);
  // a KV8 row is 36 lanes x 16 bytes; the other lanes' LDS slots belong to the next row
  auto row_dma = [&](const uint8_t* base, uint32_t off, uint32_t lds) {
    if (!KV8 || l < SROWB / 16) dma_row(base, off, __builtin_amdgcn_readfirstlane(lds));
  };
  // a tile's gathers in two parts: its eight table entries per wave (LDS
  // reads that can go out early) and the row DMAs
  auto tab_entries = [&](int t, u32x4_t& e0, u32x4_t& e1) {
    if constexpr (SRC == SRC_SPARSE_PRE) {
      const int c0 = t * TR + RPW * w;
      e0 = *reinterpret_cast<const u32x4_t*>(&tab[c0]);
      e1 = *reinterpret_cast<const u32x4_t*>(&tab[c0 + 4]);
    }
  };
  auto issue_dma = [&](int t, const u32x4_t& e0, const u32x4_t& e1) {
    const int c0 = t * TR + RPW * w;
    const uint32_t dst = ring_lds + (uint32_t)((t & (NBUF - 1)) * TB);
    if constexpr (SRC == SRC_HCA_PRE) {
      // rows past the end repeat the last row (they are masked)
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int c = min(c0 + i, n_rows - 1);
        const uint8_t* rp = c < rr.len1 ? rr.comp_base + (int64_t)c * SROWB
                                        : rr.win_base + (int64_t)(rr.w0 + c - rr.len1) * SROWB;
        row_dma(uniform_ptr(rp), voff[i], dst + lrow(RPW * w + i));
      }
      return;
    }
    const bool comp_only = c0 + RPW <= ncb, win_only = c0 >= ncb;
    if (off32 && (comp_only || win_only)) {
      // one base for the wave's eight rows; the shift drops the window flag
      const uint8_t* base = comp_only ? rr.comp_base : rr.win_base;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const uint32_t e = i < 4 ? e0[i & 3] : e1[i & 3];
        row_dma(uniform_ptr(base), (e & 0x7fffffffu) * SROWB + voff[i], dst + lrow(RPW * w + i));
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int e = (int)__builtin_amdgcn_readfirstlane(i < 4 ? e0[i & 3] : e1[i & 3]);
        row_dma(uniform_ptr(tab_row<SROWB>(rr, e)), voff[i], dst + lrow(RPW * w + i));
      }
    }
  };
  auto issue = [&](int t) {
    u32x4_t e0{0u, 0u, 0u, 0u}, e1{0u, 0u, 0u, 0u};
    tab_entries(t, e0, e1);
    issue_dma(t, e0, e1);
  };

  // tiles 0 and 1 go out behind the query rows; once those have landed, each
  // wave reads its Q^T operand and slot 2 is free for tile 2
  for (int t = 0; t < ntiles && t < 2; ++t) issue(t);
  if (ntiles >= 2)
    vm_barrier<2 * RPW>();
  else if (ntiles == 1)
    vm_barrier<RPW>();
  else
    vm_barrier<0>();
  // ---- Q^T operand (B of S = K Q^T): head 32 hg + 16 hq + l16, dims 32 ks + 8 gc
  // .. +7 with gc = the two bits of g16 swapped (the K operand takes the same
  // dims; the order only decides which 16-byte chunk each lane group reads)
  const int gc = ((g16 & 1) << 1) | (g16 >> 1);
  bf16x8_t qb[2][16];
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    const int head = 32 * hg + 16 * hq + l16;
    const uint8_t* qr = ring + QOFF + head * ROWB;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qb[hq][ks] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qr + (((4 * ks + gc) ^ (head & 15)) * 16)));
    if (head >= H)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qb[hq][ks] = as_bf16x8(u32x4_t{0, 0, 0, 0});
  }
  // Q^T waits in accumulation registers (MFMA reads its A/B operands from
  // either file), leaving the VGPRs to the reads in flight
#pragma unroll
  for (int hq = 0; hq < 2; ++hq)
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(qb[hq][ks]));
  // every wave's reads of the staged rows are done before tile 2 lands there
  vm_barrier<2 * RPW>();

  f32x16_t o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[nt][r] = 0.0f;
  // per softmax head hq: exponent reference (log2 units), the raw score above
  // which a logit exceeds it by GUARD, and the running sum of this lane's P
  float m_ref[2] = {-INFINITY, -INFINITY}, thr[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};

  // K operand (A of the 16x16x32 products): row 16 dh + l16, dims 32 ks + 8 gc
  //   -> chunk 4 ks + gc = 16 (ks / 4) + ((4 (ks % 4) + gc) ^ swz4(row)).
  // A b128 read is served in passes of lanes that share lane bits 2 and 4 (as
  // measured: eight rows x two lane groups); with gc those two groups differ
  // in chunk bit 0, which the rotation of the eight rows leaves fixed, so the
  // sixteen chunks of a pass fall in sixteen distinct bank groups
  int kofs[4];
  {
    const int row = 16 * dh + l16;
#pragma unroll
    for (int v = 0; v < 4; ++v) kofs[v] = row * ROWB + (((4 * v + gc) ^ swz4(row)) * 16);
  }
  // V^T operand (transpose reads, rows in natural order): 16-lane group g16
  // takes rows k0 .. k0+3 (k0 = 16 ks + 8 h, +4 for the second read) and
  // columns n0 .. n0+15 (n0 = 256 dh + 32 nt + 16 (g16 % 2)); lane j = l16
  // supplies row k0 + j/4, columns n0 + 4 (j%4) .. +3, so lane l receives dim
  // n0 + j of rows k0 .. k0+3: chunk 32 dh + 4 nt + 2 (g16%2) + (j%4)/2
  int pofs[2][2][4];  // [ks][first/second read][nt % 4], plus 256 bytes for nt >= 4
  {
    const int cl = 2 * (g16 & 1) + ((l16 & 3) >> 1), cb = (l16 & 1) * 8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int row = 16 * ks + 8 * h + 4 * rd + (l16 >> 2);
#pragma unroll
        for (int u = 0; u < 4; ++u) pofs[ks][rd][u] = row * ROWB + (((4 * u + cl) ^ swz4(row)) * 16) + cb + dh * 512;
      }
  }
  // P^T operand (B of O^T += V^T P^T): head l32, rows 16 ks + 8 h .. +7
  const int prd = l32 * PSTR + 8 * h;
  // P^T write: this lane's four rows 16 dh + 4 g16 .. +3 of head 16 hq + l16
  const int pwr = l16 * PSTR + 16 * dh + 4 * g16;

  // KV8: the K operand of k-steps below 14 (dims < 448) is 8 E4M3 bytes per
  // lane, widened at the product; k-steps 14, 15 read the bf16 RoPE dims.
  // V^T of the E4M3 dims comes from the 8-bit transposed read: within a
  // 16-lane group, lanes 2k and 2k+1 address row 16 ks + 8 h + k (columns 0-7
  // and 8-15 of a 16-dim block) and lane j receives column j of those eight
  // rows (P^T's K order); the RoPE N-tiles (dims 448-511) use the 16-bit
  // transposed read, with the same lane roles as the bf16 layout.
  const int kofs8 = lrow(16 * dh + l16) + 8 * gc;
  const int kofs8r = lrow(16 * dh + l16) + NOPE + 16 * gc;
  int vofs8[2], rofs8[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    vofs8[ks] = lrow(16 * ks + 8 * h + (l16 >> 1)) + 16 * (g16 & 1) + 8 * (l16 & 1) + 256 * dh;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
      rofs8[ks][rd] = lrow(16 * ks + 8 * h + 4 * rd + (l16 >> 2)) + NOPE + 32 * (g16 & 1) + 8 * (l16 & 3);
  }
  auto k_at = [&](const uint8_t* RK, int ks) -> u32x4_t {
    if constexpr (KV8) {
      if (ks < 14) {
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(RK + kofs8 + 32 * ks);
        return u32x4_t{v[0], v[1], 0u, 0u};
      }
      return *reinterpret_cast<const u32x4_t*>(RK + kofs8r + 64 * (ks - 14));
    } else {
      return *reinterpret_cast<const u32x4_t*>(RK + kofs[ks & 3] + (ks >> 2) * 256);
    }
  };
  auto kop = [&](const u32x4_t& k, int ks) -> bf16x8_t {
    if (KV8 && ks < 14)
      return as_bf16x8(u32x4_t{fp8x2_to_bf16x2(k[0], false), fp8x2_to_bf16x2(k[0], true),
                               fp8x2_to_bf16x2(k[1], false), fp8x2_to_bf16x2(k[1], true)});
    return as_bf16x8(k);
  };
  auto k_reads = [&](const uint8_t* RK, u32x4_t* kr) {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) kr[ks] = k_at(RK, ks);
  };
  auto qk = [&](const u32x4_t* kr, f32x4_t* s) {
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) s[hq] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // the two heads' chains alternate, so each product finds the previous one
    // of its chain finished (MFMAs stay in this order; everything else moves)
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) s[hq] = mfma16(kop(kr[ks], ks), qb[hq][ks], s[hq]);
      __builtin_amdgcn_sched_barrier(0x7F6);
    }
  };
  // padding rows of the last tile (every row of a tile past it) leave the
  // softmax; branch-free, so it schedules with the products around it
  auto mask_tail = [&](f32x4_t* s, int u) {
    const int nvalid = n_rows - u * TR;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool pad = 16 * dh + 4 * g16 + i >= nvalid;
      s[0][i] = pad ? -INFINITY : s[0][i];
      s[1][i] = pad ? -INFINITY : s[1][i];
    }
  };
  // P of tile u against the current reference: written to P^T buffer `buf`,
  // summed into l_run; returns whether a logit exceeds the reference by GUARD
  auto softmax = [&](const f32x4_t* s, int buf) {
    bool over = false;
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      const float mr = m_ref[hq] == -INFINITY ? 0.0f : m_ref[hq];
      const float mx = fmaxf(fmaxf(s[hq][0], s[hq][1]), fmaxf(s[hq][2], s[hq][3]));
      over |= mx > thr[hq];
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hq][i], scale_log2, -mr));
        l_run[hq] += p[i];  // fp32 weights: the log-sum-exp keeps fp32 accuracy
      }
      *reinterpret_cast<u32x2_t*>(&pbuf[buf][hg][pwr + 16 * hq * PSTR]) =
          u32x2_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    }
    return over;
  };
  // the pair agrees on exact per-head maxima of tile u, moves the reference,
  // rescales O and the sums, and redoes P (all four waves take this path)
  auto slow = [&](const f32x4_t* s, int buf, const float* l_prev) {
#pragma unroll
    for (int hq = 0; hq < 2; ++hq)
      lmx[hg][dh][hq][l] = fmaxf(fmaxf(s[hq][0], s[hq][1]), fmaxf(s[hq][2], s[hq][3]));
    vm_barrier<63>();
    float alpha[2];
    // before the first reference of a query O is zero and needs no scaling
    const bool o_live = (ohq ? m_ref[1] : m_ref[0]) != -INFINITY;
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      float tm = -INFINITY;
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) tm = fmaxf(tm, lmx[hg][d][hq][16 * gg + l16]);
      tm *= scale_log2;
      const float m_new = fmaxf(m_ref[hq], tm);
      alpha[hq] = m_ref[hq] == -INFINITY ? 0.0f : (m_new == m_ref[hq] ? 1.0f : __builtin_amdgcn_exp2f(m_ref[hq] - m_new));
      l_run[hq] = l_prev[hq] * alpha[hq];
      m_ref[hq] = m_new;
      thr[hq] = m_new == -INFINITY ? -INFINITY : (m_new + GUARD) / scale_log2;
    }
    const float ao = ohq ? alpha[1] : alpha[0];
    if (__any(o_live && ao != 1.0f)) {
      // every O^T register of this lane belongs to its own head
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // scaled where it lives: a plain multiply would make the compiler keep
          // a VGPR copy of all of O
          float tmp;
          asm volatile(
              "v_accvgpr_read_b32 %1, %0\n\t"
              "v_mul_f32 %1, %1, %2\n\t"
              "v_accvgpr_write_b32 %0, %1"
              : "+a"(o[nt][r]), "=&v"(tmp)
              : "v"(ao));
        }
    }
    softmax(s, buf);  // cannot exceed the new reference
    vm_barrier<63>();
  };
  auto post_flag = [&](bool over, int buf) {
    const bool any = __any(over);
    if (l == 0) flg[buf][w] = any ? 1 : 0;
  };
  auto flags_set = [&](int buf) {
    const u32x4_t f = *reinterpret_cast<const u32x4_t*>(&flg[buf][0]);
    return __builtin_amdgcn_readfirstlane(f[0] | f[1] | f[2] | f[3]) != 0;
  };
  auto p_reads = [&](int buf, u32x4_t* pc) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pc[ks] = *reinterpret_cast<const u32x4_t*>(&pbuf[buf][hg][prd + 16 * ks]);
  };

  u32x4_t pcur[2] = {u32x4_t{0, 0, 0, 0}, u32x4_t{0, 0, 0, 0}};  // P^T operand of the tile in hand
  // tiles 2 and 3 take the slots the query rows left
  if (ntiles > 2) issue(2);
  if (ntiles > 3) issue(3);
  // K operand of the next tile's first four k-steps: read right after the
  // barrier that makes the tile resident, so the first products need not
  // wait for LDS
  u32x4_t kr[16];
  if (ntiles > 0) {
    if (ntiles > 3)
      vm_barrier<2 * RPW>();  // tiles 0 and 1 resident, tiles 2 and 3 may be in flight
    else if (ntiles > 2)
      vm_barrier<RPW>();
    else
      vm_barrier<0>();
    k_reads(ring, kr);
    f32x4_t s[2];
    qk(kr, s);
    mask_tail(s, 0);
    const float l_prev[2] = {l_run[0], l_run[1]};
    post_flag(softmax(s, 0), 0);
    vm_barrier<63>();
    if (flags_set(0)) slow(s, 0, l_prev);
    p_reads(0, pcur);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kr[ks] = k_at(ring + (1 & (NBUF - 1)) * TB, ks);
  }
  for (int t = 0; t < ntiles; ++t) {
    // tile t+3 is in flight (issued after the last barrier); tile t+4 goes
    // out after this iteration's barrier, into tile t's slot
    const bool iss = t + NBUF - 1 < ntiles, nxt = t + 1 < ntiles, iss4 = t + NBUF < ntiles;
    const uint8_t* R = ring + (t & (NBUF - 1)) * TB;
    const uint8_t* RN = ring + ((t + 1) & (NBUF - 1)) * TB;

    // ---- S of tile t+1 and the transposed V reads of tile t, in a fixed
    // order: each k-step issues the K read four steps ahead and two V reads,
    // then its two products (the heads' chains alternate). The reads stay
    // spread over the products instead of queueing in one burst. On the last
    // tile the products read a stale slot and their result is dropped.
    auto k_read = [&](int ks) { return k_at(RN, ks); };
    s16x4_t vr[KV8 ? 2 : 8][2][2];  // [nt][ks][first/second four rows] (KV8: the RoPE N-tiles 6, 7)
    i32x2_t v8[8][2];                // KV8: [nt][ks] E4M3 V^T of eight rows
    auto v_read = [&](int i) {  // i = 4 nt + 2 ks + rd
      const int nt = i >> 2, ks = (i >> 1) & 1, rd = i & 1;
      if constexpr (KV8) {
        // N-tiles 6, 7 read both forms (dh = 0: E4M3 dims 192-255; dh = 1:
        // RoPE dims 448-511); the product takes the wave's own, so the
        // schedule has no branch
        if (rd == 0)
          v8[nt][ks] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (i32x2_t __attribute__((address_space(3)))*)(R + vofs8[ks] + 32 * nt));
        if (nt >= 6)
          vr[nt - 6][ks][rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4_t __attribute__((address_space(3)))*)(R + rofs8[ks][rd] + 64 * (nt - 6)));
      } else {
        vr[nt][ks][rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4_t __attribute__((address_space(3)))*)(R + pofs[ks][rd][nt & 3] + (nt >> 2) * 256));
      }
    };
    f32x4_t s[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
    // bf16 rows: the S products take the K reads and the V reads of N-tiles
    // 0 and 1 only; the other V reads go out during the PV products, two
    // N-tiles ahead, so each phase carries part of the LDS traffic
    constexpr bool VSPLIT = !KV8;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (ks + 4 < 16) kr[ks + 4] = k_read(ks + 4);
      if (VSPLIT) {
        if (ks >= 8) v_read(ks - 8);
      } else {
        v_read(2 * ks);
        v_read(2 * ks + 1);
      }
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) s[hq] = mfma16(kop(kr[ks], ks), qb[hq][ks], s[hq]);
      __builtin_amdgcn_sched_barrier(0x006);  // only VALU / SALU work moves across
    }
    __builtin_amdgcn_sched_barrier(0);

    u32x4_t te0{0u, 0u, 0u, 0u}, te1{0u, 0u, 0u, 0u};  // table entries of tile t+4
    if (iss4) tab_entries(t + NBUF, te0, te1);

    // ---- O^T += V^T P^T of tile t over this wave's 256 dims: 8 N-tiles of 32
    // dims, 2 k-steps of 16 rows; the softmax of tile t+1 runs between them.
    // bf16 rows: each N-tile's V reads go out two N-tiles ahead, in a
    // scheduling region of their own, so the reads keep their distance
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (VSPLIT && ks == 0) {
          if (nt + 2 < 8)
#pragma unroll
            for (int i = 0; i < 4; ++i) v_read(4 * (nt + 2) + i);
          __builtin_amdgcn_sched_barrier(0x006);  // only VALU / SALU work moves across
        }
        bf16x8_t bv;
        if constexpr (KV8) {
          const i32x2_t c = v8[nt][ks];
          bv = as_bf16x8(u32x4_t{fp8x2_to_bf16x2((uint32_t)c[0], false), fp8x2_to_bf16x2((uint32_t)c[0], true),
                                 fp8x2_to_bf16x2((uint32_t)c[1], false), fp8x2_to_bf16x2((uint32_t)c[1], true)});
          if (nt >= 6) {
            const bf16x8_t br = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(vr[nt - 6][ks][0], vr[nt - 6][ks][1], 0, 1, 2, 3, 4, 5, 6, 7));
            bv = dh ? br : bv;
          }
        } else {
          bv = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(vr[nt][ks][0], vr[nt][ks][1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
        o[nt] = mfma32x16(bv, as_bf16x8(pcur[ks]), o[nt]);
      }
    // (on the last tile this works on the stale S: its P^T and flag are never
    // read and the sums are restored below)
    const float l_prev[2] = {l_run[0], l_run[1]};
    mask_tail(s, t + 1);
    post_flag(softmax(s, (t + 1) & 1), (t + 1) & 1);
    if constexpr (!VSPLIT) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 1);  // VALU
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // P^T of tile t+1 written, tile t+2 resident (tile t+3 may be in flight),
    // tile t's reads done
    if (iss)
      vm_barrier<RPW>();
    else
      vm_barrier<0>();
    if (nxt) {
      // the flags, the next P^T and the first K reads of tile t+2 go out
      // together, then tile t+4's gathers, and only then is the flag word
      // waited for
      const u32x4_t f = *reinterpret_cast<const u32x4_t*>(&flg[(t + 1) & 1][0]);
      p_reads((t + 1) & 1, pcur);
      const uint8_t* RN2 = ring + ((t + 2) & (NBUF - 1)) * TB;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kr[ks] = k_at(RN2, ks);
      if (iss4) issue_dma(t + NBUF, te0, te1);
      if (__builtin_amdgcn_readfirstlane(f[0] | f[1] | f[2] | f[3]) != 0) {
        slow(s, (t + 1) & 1, l_prev);
        p_reads((t + 1) & 1, pcur);
      }
    } else {
      l_run[0] = l_prev[0];
      l_run[1] = l_prev[1];
    }
  }

  // ---- epilogue: l of each head over both row halves and the four row groups
  // of a lane's head (lmx is free: the last reads of it preceded a barrier)
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) lmx[hg][dh][hq][l] = l_run[hq];
  vm_barrier<63>();
  float lsum = 0.0f;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) lsum += lmx[hg][d][ohq][16 * gg + l16];
  const int head = hg * 32 + l32;
  const bool hok = head < H;
  const float mo = ohq ? m_ref[1] : m_ref[0];
  const float s2 = (sink && hok) ? sink[head] * LOG2E_F : -INFINITY;
  const float M = fmaxf(mo, s2);
  float fac = 0.0f;
  if (M != -INFINITY) {
    const float a = exp2f(mo - M);
    fac = a / (lsum * a + exp2f(s2 - M));
  }
  const int64_t orow = (qi * H + (hok ? head : 0)) * (int64_t)D + dh * 256;
  if (out_dt == DT_BF16) {
    // the two lane halves hold alternate groups of four dims; one swap per
    // dword gives each lane eight consecutive dims (16 bytes)
    uint16_t* op = reinterpret_cast<uint16_t*>(out) + orow + 8 * h;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int r0 = 8 * p;
        const uint32_t x0 = pack_bf16x2(o[nt][r0] * fac, o[nt][r0 + 1] * fac);
        const uint32_t x1 = pack_bf16x2(o[nt][r0 + 2] * fac, o[nt][r0 + 3] * fac);
        const uint32_t y0 = pack_bf16x2(o[nt][r0 + 4] * fac, o[nt][r0 + 5] * fac);
        const uint32_t y1 = pack_bf16x2(o[nt][r0 + 6] * fac, o[nt][r0 + 7] * fac);
        const auto sa = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto sb = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        if (hok) *reinterpret_cast<u32x4_t*>(op + nt * 32 + p * 16) = u32x4_t{sa[0], sb[0], sa[1], sb[1]};
      }
  } else if (hok) {
    float* op = reinterpret_cast<float*>(out) + orow + 4 * h;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<f32x4_t*>(op + nt * 32 + qd * 8) =
            f32x4_t{o[nt][4 * qd] * fac, o[nt][4 * qd + 1] * fac, o[nt][4 * qd + 2] * fac, o[nt][4 * qd + 3] * fac};
  }
  if (lse && dh == 0 && h == 0 && hok) {
    float v = -INFINITY;
    if (M != -INFINITY) v = (M + log2f(lsum * exp2f(mo - M) + exp2f(s2 - M))) * LN2_F;
    lse[qi * H + head] = v;
  }
}

// ----------------------------------------------------------------------------
// fp32 rows (small head dims): four-wave heads split, register-staged tiles
// ----------------------------------------------------------------------------

template <int D, int NWAV, int SRC>
__global__ void __launch_bounds__(64 * NWAV) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_f32_kernel(const float* __restrict__ q, RowSrc src, const int32_t* __restrict__ win_len,
            const int32_t* __restrict__ n_comp, const int32_t* __restrict__ q_pos, int m_rate,
            const float* __restrict__ sink, float scale_log2, int H, int slots, int split_rows,
            float* __restrict__ part_o, float* __restrict__ part_ml, void* __restrict__ out,
            float* __restrict__ lse, int out_dt) {
  constexpr int KSTEP = 4;
  constexpr int ES = 4;
  constexpr int NT = 64 * NWAV;
  constexpr int TR = 32;                         // rows per tile
  constexpr int ROWB = D * ES;                   // bytes per row
  constexpr int RPITCH = ROWB + 4;               // LDS row pitch (bytes), padded
  constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row
  constexpr int RPP = NT / CPR;                  // rows per load pass
  constexpr int PASSES = TR / RPP;
  constexpr int KSQ = D / KSTEP;                 // QK k-steps
  constexpr int NTD = D / 16;                    // PV N-tiles
  static_assert(NT % CPR == 0 && TR % RPP == 0, "tile load mapping");

  constexpr int PF = 2;            // tiles in flight in the register ring
  constexpr int CODE_MAX = 1024;   // top-k slots per split staged in LDS
  __shared__ __attribute__((aligned(16))) uint8_t lds_r[2][TR * RPITCH];
  __shared__ int lds_valid[2][TR];
  __shared__ int lds_code[(SRC == SRC_HCA_DEC || SRC == SRC_HCA_PRE) ? 1 : CODE_MAX];

  const int tid = threadIdx.x;
  const int l = tid & 63, wv = tid >> 6;
  const int G = l >> 4, l16 = l & 15;
  const int64_t qi = blockIdx.x;  // query (decode: sequence)
  const int sp = blockIdx.y;      // split
  const int nsplit = gridDim.y;
  const int head = wv * 16 + l16;  // this lane's head in S^T / P / softmax

  int lim0 = 0, lim1 = 0;
  if (SRC == SRC_SPARSE_DEC) {
    lim1 = dec_window(src, win_len, qi / src.Tq, (int)(qi % src.Tq), &lim0);
  } else if (SRC == SRC_HCA_DEC) {
    if (n_comp) {
      const int64_t v = min((int64_t)n_comp[qi], ((int64_t)q_pos[qi] + 1) / m_rate);
      lim0 = (int)max((int64_t)0, min(v, src.N_max));
    }
    lim1 = win_len ? min(max(win_len[qi], 0), src.W) : 0;
  } else if (SRC == SRC_HCA_PRE) {
    lim1 = q_pos[qi];
    lim0 = (int)max((int64_t)0, min(((int64_t)lim1 + 1) / m_rate, src.N_max));
  } else {
    lim1 = q_pos[qi];
  }
  const int s_begin = sp * split_rows;
  const int s_end = min(slots, s_begin + split_rows);
  const int ntiles = (s_end > s_begin) ? (s_end - s_begin + TR - 1) / TR : 0;

  // ---- Q^T operand (B of S^T = R Q^T): lane (head, G), dims s*KSTEP + G*VPL + 0..VPL-1
  float qb[KSQ];
  {
    const bool hok = head < H;
    const float* qp = q + (qi * H + (hok ? head : 0)) * (int64_t)D + G;
#pragma unroll
    for (int s = 0; s < KSQ; ++s) qb[s] = hok ? qp[s * 4] : 0.0f;
  }

  // ---- top-k indices of this split, staged once in LDS (sparse row sources)
  if (SRC == SRC_SPARSE_DEC || SRC == SRC_SPARSE_PRE) {
    const int ncode = min(s_end, src.top_k) - s_begin;  // slots of this split that are top-k slots
    for (int i = tid; i < ncode; i += NT) lds_code[i] = slot_code<SRC>(src, qi, s_begin + i);
    __syncthreads();
  }

  // ---- tile loader: thread handles chunk lc of rows lrs + ps*RPP. Tiles go
  // HBM -> register ring (PF tiles deep) -> LDS double buffer -> MFMA.
  const int lc = tid % CPR, lrs = tid / CPR;
  u32x4_t pre[PF][PASSES];
  uint32_t prevm[PF];
  auto fetch = [&](auto SLOT, int tile) {
    constexpr int slot = decltype(SLOT)::value;
    const int base = s_begin + tile * TR;
    uint32_t vm = 0;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int j = base + lrs + ps * RPP;
      const int code = (j < s_end && j - s_begin < CODE_MAX && (SRC == SRC_SPARSE_DEC || SRC == SRC_SPARSE_PRE) && j < src.top_k)
                           ? lds_code[j - s_begin] : -1;
      const uint8_t* rp = (j < s_end) ? slot_row<SRC, ROWB>(src, qi, j, code, lim0, lim1) : nullptr;
      vm |= (rp != nullptr ? 1u : 0u) << ps;
      pre[slot][ps] = rp ? ld16(rp + lc * 16) : u32x4_t{0, 0, 0, 0};
    }
    prevm[slot] = vm;
  };
  auto stash = [&](auto SLOT, int buf) -> int {
    constexpr int slot = decltype(SLOT)::value;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int r = lrs + ps * RPP;
      float* dst = reinterpret_cast<float*>(&lds_r[buf][r * RPITCH]) + lc * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(pre[slot][ps][e]);
      if (lc == 0) lds_valid[buf][r] = (prevm[slot] >> ps) & 1;
    }
    return prevm[slot] != 0;
  };

  f32x4_t oacc[NTD];
#pragma unroll
  for (int nt = 0; nt < NTD; ++nt) oacc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;  // for `head`, replicated over G

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  static_assert(PF == 2, "ring of two tiles");
  int any_next = 0;
  if (ntiles > 0) {
    fetch(I0{}, 0);
    any_next = stash(I0{}, 0);
    if (ntiles > 1) fetch(I1{}, 1);
    if (ntiles > 2) fetch(I0{}, 2);
    any_next = __syncthreads_or(any_next);
  }
  // one tile: stage tile+1 (ring slot SLOT) into the other LDS buffer, refill
  // the slot with tile+1+PF, compute tile from LDS, one barrier
  auto body = [&](int tile, auto SLOT) {
    const int buf = tile & 1;
    const int any = any_next;
    if (tile + 1 < ntiles) {
      any_next = stash(SLOT, buf ^ 1);
      if (tile + 1 + PF < ntiles) fetch(SLOT, tile + 1 + PF);
    }
    if (any) {
      const uint8_t* R = lds_r[buf];  // tile `tile`
      // ---- S^T[mt] = R(rows mt*16..) Q^T : lane holds rows mt*16 + G*4 + r of `head`
      f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = mt * 16 + l16;
#pragma unroll
        for (int s = 0; s < KSQ; ++s) {
          const float a = reinterpret_cast<const float*>(R + row * RPITCH)[s * 4 + G];
          sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qb[s], sacc[mt], 0, 0, 0);
        }
      }
      // ---- online softmax of `head` over this tile's 32 rows (exp2 domain)
      float sv[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = mt * 16 + G * 4 + r;
          const float v = lds_valid[buf][row] ? sacc[mt][r] * scale_log2 : -INFINITY;
          sv[mt * 4 + r] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      // m_run is the exponent reference (not necessarily the running max): it
      // moves to the tile max only when that exceeds it by RESCALE_SLACK
      const bool move = tmax > m_run + RESCALE_SLACK || (m_run == -INFINITY && tmax != -INFINITY);
      const float m_new = move ? tmax : m_run;
      float alpha = 1.0f, psum = 0.0f;
      float pv[8];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = 0.0f;
      } else {
        if (move) alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_new);
          psum += pv[i];
        }
      }
      psum += shfl_xor(psum, 16);
      psum += shfl_xor(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      // ---- rescale O rows (heads G*4 + r of this wave) when a max moved
      if (__any(alpha != 1.0f)) {
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, G * 4 + r, 64);
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[nt][r] *= ar[r];
      }
      // ---- O += P R; K = 4 rows per step: lane G holds row (j/4)*16 + G*4 + j%4
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = (j >> 2) * 16 + G * 4 + (j & 3);
        const float* rr = reinterpret_cast<const float*>(R + row * RPITCH);
#pragma unroll
        for (int nt = 0; nt < NTD; ++nt)
          oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[j], rr[nt * 16 + l16], oacc[nt], 0, 0, 0);
      }
    }
    if (tile + 1 < ntiles) any_next = __syncthreads_or(any_next);
  };
  for (int t0 = 0; t0 < ntiles; t0 += PF) {
    body(t0, I1{});
    if (t0 + 1 < ntiles) body(t0 + 1, I0{});
  }

  // ---- epilogue: O rows are heads wv*16 + G*4 + r; their (m, l) live in lanes G*4 + r
  float mr[4], lr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mr[r] = __shfl(m_run, G * 4 + r, 64);
    lr[r] = __shfl(l_run, G * 4 + r, 64);
  }
  if (part_o != nullptr) {
    const int64_t pbase = (qi * nsplit + sp) * (int64_t)H;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = wv * 16 + G * 4 + r;
      if (h >= H) continue;
#pragma unroll
      for (int nt = 0; nt < NTD; ++nt) part_o[(pbase + h) * D + nt * 16 + l16] = oacc[nt][r];
    }
    if (G == 0 && head < H) {
      part_ml[(pbase + head) * 2 + 0] = m_run;
      part_ml[(pbase + head) * 2 + 1] = l_run;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = wv * 16 + G * 4 + r;
      if (h >= H) continue;
      const float s2 = sink ? sink[h] * LOG2E_F : -INFINITY;
      const float M = fmaxf(mr[r], s2);
      float fac = 0.0f;
      if (M != -INFINITY) {
        const float a = exp2f(mr[r] - M);
        fac = a / (lr[r] * a + exp2f(s2 - M));
      }
#pragma unroll
      for (int nt = 0; nt < NTD; ++nt) {
        const int64_t o = (qi * H + h) * (int64_t)D + nt * 16 + l16;
        const float v = oacc[nt][r] * fac;
        if (out_dt == DT_BF16)
          reinterpret_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16(v);
        else
          reinterpret_cast<float*>(out)[o] = v;
      }
    }
    if (lse && G == 0 && head < H) {
      const float s2 = sink ? sink[head] * LOG2E_F : -INFINITY;
      const float M = fmaxf(m_run, s2);
      float v = -INFINITY;
      if (M != -INFINITY) v = (M + log2f(l_run * exp2f(m_run - M) + exp2f(s2 - M))) * LN2_F;
      lse[qi * H + head] = v;
    }
  }
}

// Eight consecutive dims of a partial row.
__device__ __forceinline__ void part8(const float* p, float (&v)[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p), b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// Merge split partials in fixed order s = 0..nsplit-1 and add the sink.
// One wave per (query, head); lane l covers the head's dims 8 l .. 8 l + 7.
__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                    const float* __restrict__ sink, int H, int D, int nsplit,
                    void* __restrict__ out, float* __restrict__ lse, int out_dt, QkArgs qk) {
  const int64_t qi = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (h >= H) return;
  const float s2 = sink ? sink[h] * LOG2E_F : -INFINITY;
  const int64_t row0 = qi * nsplit * (int64_t)H + h;  // partial (qi, s, h) at row0 + s*H
  const int d = l * 8;
  const bool dok = d < D;  // D <= 512, a multiple of 8
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  float M = s2, Z = 0.0f;
  constexpr int U1 = 16;
  if (nsplit <= U1) {
    // every partial of the head in one round of loads, then the same merge
    float mv[U1], lv[U1];
    float v[U1][8];
#pragma unroll
    for (int u = 0; u < U1; ++u) {
      const int64_t pb = row0 + (int64_t)u * H;
      const bool in = u < nsplit;
      mv[u] = in ? part_ml[pb * 2] : -INFINITY;
      lv[u] = in ? part_ml[pb * 2 + 1] : 0.0f;
      if (in && dok) {
        part8(part_o + pb * D + d, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U1; ++u) M = fmaxf(M, mv[u]);
    if (M != -INFINITY) {
      Z = exp2f(s2 - M);
#pragma unroll
      for (int u = 0; u < U1; ++u) {
        const float a = exp2f(mv[u] - M);  // 0 for an empty or absent split (m = -inf)
        Z += lv[u] * a;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[u][e] * a;
      }
    }
  } else {
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(row0 + (int64_t)s * H) * 2]);
    if (M != -INFINITY) {
      Z = exp2f(s2 - M);
      for (int s0 = 0; s0 < nsplit; s0 += 4) {
        float v[4][8];
        float a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s = s0 + u;
          a[u] = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
          if (s < nsplit) {
            const int64_t pb = row0 + (int64_t)s * H;
            a[u] = exp2f(part_ml[pb * 2] - M);  // 0 for an empty split (m = -inf)
            Z += part_ml[pb * 2 + 1] * a[u];
            if (dok) part8(part_o + pb * D + d, v[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += v[u][e] * a[u];
      }
    }
  }
  const float inv = (M != -INFINITY) ? 1.0f / Z : 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  if (qk.flags & 2) {
    // the output's inverse rotation, pairs inside the lane's 8 dims; lane
    // i < R/2 forms pair i's angle and the rotating lanes read it (every lane
    // of the wave shuffles)
    float rc, rs;
    rope_lane(qk, qi, rc, rs);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bool rot = dok && d + e >= D - qk.R;
      const int src = rot ? (d + e - (D - qk.R)) >> 1 : 0;
      const float c = __shfl(rc, src, 64), sn = __shfl(rs, src, 64);
      if (rot) {
        const float x0 = acc[e], x1 = acc[e + 1];
        acc[e] = x0 * c + x1 * sn;
        acc[e + 1] = x1 * c - x0 * sn;
      }
    }
  }
  if (dok) {
    const int64_t o = (qi * H + h) * (int64_t)D + d;
    if (out_dt == DT_BF16) {
      const u32x4_t w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                         pack_bf16x2(acc[6], acc[7])};
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + o) = w;
    } else {
      float* op = reinterpret_cast<float*>(out) + o;
      *reinterpret_cast<f32x4_t*>(op) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4_t*>(op + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    }
  }
  if (lse && l == 0) lse[qi * H + h] = (M != -INFINITY) ? (M + log2f(Z)) * LN2_F : -INFINITY;
}

// ----------------------------------------------------------------------------
// host-side launchers
// ----------------------------------------------------------------------------

static RowSrc row_src(const AttnLaunch& a) {
  RowSrc src;
  src.kv_comp = reinterpret_cast<const uint8_t*>(a.kv_comp);
  src.kv_win = reinterpret_cast<const uint8_t*>(a.kv_win);
  src.idx = a.idx;
  src.N_max = a.N_max;
  src.T_tok = a.T_tok;
  src.top_k = a.top_k;
  src.W = a.W;
  src.Tq = a.Tq > 0 ? a.Tq : 1;
  src.Wb = a.Wb > 0 ? a.Wb : a.W;
  return src;
}

static QkArgs qk_args(const AttnLaunch& a) {
  return QkArgs{a.qk_flags, a.qk_gamma, a.qk_eps, a.qk_R, a.qk_flags ? log2((double)a.qk_theta) : 0.0, a.q_pos};
}

static hipError_t launch_combine(const AttnLaunch& a, hipStream_t st) {
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)a.nq, (unsigned)((a.H + 3) / 4)), dim3(256), 0, st,
                     a.part_o, a.part_ml, a.sink, a.H, a.D, a.nsplit, a.out, a.lse, a.out_dt, qk_args(a));
  return hipGetLastError();
}

template <int SRC, bool KV8 = false>
static hipError_t launch_bf16(const AttnLaunch& a, hipStream_t st) {
  if (SRC != SRC_HCA_DEC && a.split_rows > bfk::TAB_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)a.nq, a.nsplit);
  hipLaunchKernelGGL((attn_bf16_kernel<SRC, KV8>), grid, dim3(bfk::NT), 0, st, reinterpret_cast<const uint16_t*>(a.q),
                     row_src(a), a.win_len, a.n_comp, a.q_pos, a.m_rate, a.sink, a.scale * LOG2E_F, a.H, a.slots,
                     a.split_rows, a.nsplit > 1 ? a.part_o : nullptr, a.part_ml, a.out, a.lse, a.out_dt,
                     HcaAppend{reinterpret_cast<const uint16_t*>(a.app_Ca), reinterpret_cast<const uint16_t*>(a.app_Za),
                               a.app_Ba, a.app_n_rows, a.app_tok_begin, a.app_blk, a.app_m, a.app_out},
                     qk_args(a));
  hipError_t e = hipGetLastError();
  phase_mark(PHASE_ATTN, st);
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_combine(a, st);
}

template <int SRC, bool KV8 = false>
static hipError_t launch_pre32(const AttnLaunch& a, hipStream_t st) {
  if (a.nsplit != 1 || (SRC == SRC_SPARSE_PRE && a.slots > prs::TAB_MAX)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_prs_kernel<SRC, KV8>), dim3((unsigned)a.nq), dim3(prs::NT), 0, st,
                     reinterpret_cast<const uint16_t*>(a.q), row_src(a), a.q_pos, a.m_rate, a.sink,
                     a.scale * LOG2E_F, a.H, a.slots, a.out, a.lse, a.out_dt);
  return hipGetLastError();
}

template <int D, int NWAV, int SRC>
static hipError_t launch_f32(const AttnLaunch& a, hipStream_t st) {
  dim3 grid((unsigned)a.nq, a.nsplit);
  hipLaunchKernelGGL((attn_f32_kernel<D, NWAV, SRC>), grid, dim3(64 * NWAV), 0, st,
                     reinterpret_cast<const float*>(a.q), row_src(a), a.win_len, a.n_comp, a.q_pos, a.m_rate, a.sink,
                     a.scale * LOG2E_F, a.H, a.slots, a.split_rows, a.nsplit > 1 ? a.part_o : nullptr, a.part_ml,
                     a.out, a.lse, a.out_dt);
  hipError_t e = hipGetLastError();
  phase_mark(PHASE_ATTN, st);
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_combine(a, st);
}

template <int SRC>
static hipError_t dispatch_src(const AttnLaunch& a, hipStream_t st) {
  if (a.kv_dt == DT_BF16 && a.D == 512 && a.H > 48 && a.H <= 64) {
    if constexpr (SRC == SRC_HCA_PRE) {
      return launch_pre32<SRC>(a, st);
    } else if constexpr (SRC == SRC_SPARSE_PRE) {
      if (a.nsplit == 1) return launch_pre32<SRC>(a, st);
      return launch_bf16<SRC>(a, st);
    } else {
      return launch_bf16<SRC>(a, st);
    }
  }
  if (a.kv_dt == DT_KV_FP8 && a.D == 512 && a.H > 48 && a.H <= 64) {
    if constexpr (SRC == SRC_SPARSE_DEC || SRC == SRC_HCA_DEC) {
      return launch_bf16<SRC, true>(a, st);
    } else {
      if (a.nsplit != 1) return hipErrorInvalidValue;
      return launch_pre32<SRC, true>(a, st);
    }
  }
  if (a.kv_dt == DT_F32 && a.D == 64 && a.H <= 16) return launch_f32<64, 1, SRC>(a, st);
  return hipErrorInvalidValue;
}

hipError_t run_attn(const AttnLaunch& a, hipStream_t st) {
  if (a.nq == 0) return hipSuccess;
  switch (a.src) {
    case 0: return dispatch_src<SRC_SPARSE_DEC>(a, st);
    case 1: return dispatch_src<SRC_HCA_DEC>(a, st);
    case 3: return dispatch_src<SRC_HCA_PRE>(a, st);
    default: return dispatch_src<SRC_SPARSE_PRE>(a, st);
  }
}

}  // namespace csa
