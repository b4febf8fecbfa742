// Shared-KV multi-query attention over rows of D = 512, the decode tile loop
// and its row sources: the device code that the decode kernels (one query per
// workgroup and split) share. What is computed and the design are described
// in attn.hip.
#pragma once
#include "common.h"

namespace csa {

enum { SRC_SPARSE_DEC = 0, SRC_HCA_DEC = 1, SRC_SPARSE_PRE = 2, SRC_HCA_PRE = 3 };

// XOR swizzle of the 16-byte chunk index inside each 256-byte group of a
// tile row (rows are 1 KB, so every row starts in bank group 0). A b128 read
// takes one chunk of 16 consecutive rows; with 64 banks of 4 bytes, row & 15
// puts those 16 chunks in 16 different 16-byte bank groups (measured on
// gfx950: full 256 B/clk, against 150 B/clk for a 3-bit rotation). The
// transpose reads (4 rows x 32 bytes per 16 lanes) run at the rate of that
// instruction with either choice.
__device__ __forceinline__ int swz(int row) { return row & 15; }

// Lazy rescaling of the online softmax: the exponent reference of a head
// only moves when a tile's maximum exceeds it by more than this (log2 units),
// so P <= 2^8 and the O accumulators are rarely touched.
constexpr float RESCALE_SLACK = 8.0f;

struct RowSrc {
  const uint8_t* kv_comp;
  const uint8_t* kv_win;  // window rows (decode) or raw tokens (prefill)
  const int32_t* idx;
  int64_t N_max;
  int64_t T_tok;
  int top_k;
  int W;
  int Tq;  // sparse decode: queries per sequence (query qi is token qi % Tq of sequence qi / Tq)
  int Wb;  // sparse decode: window buffer rows per sequence (W + Tq - 1)
};

// Sparse decode window of query t of a sequence: the buffer's valid rows are
// 0 .. wl-1 (wl = min(win_len, Wb)), its last row the newest token; query t's
// own token is row wl - Tq + t, and its window the (at most) W rows ending
// there. Returns the first row; *cnt gets the row count.
__device__ __forceinline__ int dec_window(const RowSrc& s, const int32_t* __restrict__ win_len, int64_t b, int t,
                                          int* cnt) {
  const int wl = win_len ? min(max(win_len[b], 0), s.Wb) : 0;
  const int hi = wl - s.Tq + t;
  const int lo = max(0, hi - s.W + 1);
  *cnt = max(0, hi - lo + 1);
  return lo;
}

// The memory-resident part of a slot (its top-k index); loaded one tile ahead
// of the row itself so the index -> row dependency never stalls a tile.
template <int SRC>
__device__ __forceinline__ int slot_code(const RowSrc& s, int64_t qi, int j) {
  if ((SRC == SRC_SPARSE_DEC || SRC == SRC_SPARSE_PRE) && j < s.top_k) return s.idx[qi * s.top_k + j];
  return 0;
}

template <int SRC, int ROWB>
__device__ __forceinline__ const uint8_t* slot_row(const RowSrc& s, int64_t qi, int j, int code, int lim0,
                                                   int lim1) {
  // lim0: SPARSE: window length; HCA: visible entries V.  lim1: PRE: position p
  if (SRC == SRC_SPARSE_DEC || SRC == SRC_SPARSE_PRE) {
    if (j < s.top_k) {
      const int id = code;
      if (id < 0 || id >= s.N_max) return nullptr;
      int64_t row = (SRC == SRC_SPARSE_DEC) ? (qi / s.Tq) * s.N_max + id : (int64_t)id;
      return s.kv_comp + row * ROWB;
    }
    int w = j - s.top_k;
    if (SRC == SRC_SPARSE_DEC) {  // lim0: window rows of this query, lim1: its first buffer row
      if (w >= lim0) return nullptr;
      return s.kv_win + ((qi / s.Tq) * s.Wb + lim1 + w) * ROWB;
    }
    int64_t tok = (int64_t)lim1 - s.W + 1 + w;
    if (tok < 0 || tok >= s.T_tok) return nullptr;
    return s.kv_win + tok * ROWB;
  } else if (SRC == SRC_HCA_PRE) {
    // lim0: visible entries V(p); lim1: position p
    if (j < s.N_max) return j < lim0 ? s.kv_comp + (int64_t)j * ROWB : nullptr;
    const int64_t tok = (int64_t)lim1 - s.W + 1 + (j - s.N_max);
    if (tok < 0 || tok >= s.T_tok) return nullptr;
    return s.kv_win + tok * ROWB;
  } else {
    if (j < s.N_max) {
      if (j >= lim0) return nullptr;
      return s.kv_comp + (qi * s.N_max + j) * ROWB;
    }
    int w = j - (int)s.N_max;
    if (w >= lim1) return nullptr;  // HCA: lim1 = window length
    return s.kv_win + (qi * s.W + w) * ROWB;
  }
}

// ----------------------------------------------------------------------------
// bf16 rows of D = 512: eight waves, rows gathered into LDS by DMA
// ----------------------------------------------------------------------------
//
// Wave w owns heads 16*(w%4) .. +15 and the dim half 256*(w/4) .. +255. S^T of
// a 32-row tile is a sum over both dim halves: each wave of a pair (w, w^4)
// computes its half, the pair swaps partials through LDS, and both then hold
// the same S^T (float addition commutes), run the same softmax and each
// accumulates O for its own 256 dims: O (64 VGPRs) and Q (32) stay in
// architectural registers, two waves per SIMD.
//
// Rows reach LDS by global_load_lds_dwordx4: one instruction moves one 1 KB
// row (lane i -> 16-byte chunk i), with no register staging. The row list of
// the workgroup is built once (invalid slots dropped, slot order kept), so a
// row address is one LDS word plus scalar arithmetic. A ring of four 32 KB
// tiles keeps three tiles in flight; waits are explicit vmcnt counts (four
// row loads per wave per tile), and each tile costs two barriers (tile ready,
// S^T partials swapped).

namespace bfk {
constexpr int D = 512, ROWB = 1024, TR = 32, NW = 8, NT = 512, NBUF = 4;
constexpr int TILEB = TR * ROWB;  // 32 KB
constexpr int TAB_MAX = 2048;     // rows of one workgroup for the table-driven sources
}  // namespace bfk


// What a workgroup knows about its query and split: the per-query limits of
// the row sources, where the compressed and window rows live, and the split's
// compacted row list (HCA: two contiguous ranges; sparse: a table in LDS).
struct QRows {
  int lim0, lim1;  // SPARSE_DEC: window length; HCA: V, window length; PRE: -, position; HCA_PRE: V, position
  int s_begin, s_end;
  const uint8_t* comp_base;
  const uint8_t* win_base;
  int n_rows;    // rows after dropping invalid slots
  int len1, w0;  // HCA: rows taken from the compressed range; first window row (HCA_PRE: token)
};

template <int SRC, int ROWB = 1024>
__device__ __forceinline__ QRows query_rows(const RowSrc& src, const int32_t* __restrict__ win_len,
                                            const int32_t* __restrict__ n_comp, const int32_t* __restrict__ q_pos,
                                            int m_rate, int64_t qi, int sp, int slots, int split_rows) {
  QRows r;
  r.lim0 = 0;
  r.lim1 = 0;
  r.w0 = 0;
  if (SRC == SRC_SPARSE_DEC) {
    r.w0 = dec_window(src, win_len, qi / src.Tq, (int)(qi % src.Tq), &r.lim0);
  } else if (SRC == SRC_HCA_DEC) {
    if (n_comp) {
      const int64_t v = min((int64_t)n_comp[qi], ((int64_t)q_pos[qi] + 1) / m_rate);
      r.lim0 = (int)max((int64_t)0, min(v, src.N_max));
    }
    r.lim1 = win_len ? min(max(win_len[qi], 0), src.W) : 0;
  } else if (SRC == SRC_HCA_PRE) {
    r.lim1 = q_pos[qi];
    const int64_t v = min(((int64_t)r.lim1 + 1) / m_rate, src.N_max);
    r.lim0 = (int)max((int64_t)0, v);
  } else {
    r.lim1 = q_pos[qi];
  }
  r.s_begin = sp * split_rows;
  r.s_end = min(slots, r.s_begin + split_rows);
  constexpr bool PRE = SRC == SRC_SPARSE_PRE || SRC == SRC_HCA_PRE;  // one sequence: shared caches
  const int64_t seq = SRC == SRC_SPARSE_DEC ? qi / src.Tq : qi;
  const int64_t wrows = SRC == SRC_SPARSE_DEC ? src.Wb : src.W;
  r.comp_base = src.kv_comp + (PRE ? 0 : seq * src.N_max * ROWB);
  r.win_base = src.kv_win + (PRE ? 0 : seq * wrows * ROWB);
  r.n_rows = r.len1 = 0;
  if (SRC != SRC_SPARSE_DEC) r.w0 = 0;
  if (SRC == SRC_HCA_DEC) {
    // slots [0, N_max) are compressed entries (valid below V), then the window
    r.len1 = max(0, min(r.s_end, r.lim0) - r.s_begin);
    const int a2 = max(r.s_begin, (int)src.N_max), b2 = min(r.s_end, (int)src.N_max + r.lim1);
    r.w0 = a2 - (int)src.N_max;
    r.n_rows = r.len1 + max(0, b2 - a2);
  } else if (SRC == SRC_HCA_PRE) {
    // entries 0 .. V-1, then the window tokens max(0, p-W+1) .. min(p, T_tok-1)
    const int64_t first = max((int64_t)0, (int64_t)r.lim1 - src.W + 1);
    const int64_t last = min((int64_t)r.lim1, src.T_tok - 1);
    r.len1 = r.lim0;
    r.w0 = (int)first;
    r.n_rows = r.len1 + (int)max((int64_t)0, last - first + 1);
  }
  return r;
}

// Row table of a sparse split (all NT threads call it): entry = compressed row
// id, or 0x80000000 | window row; invalid slots dropped, slot order kept (so
// the compressed rows come first), the tail padded to a whole tile of TR with
// the last row (those rows are masked). Returns the row count; the number of
// compressed rows goes to *n_comp when it is given. cnt holds 2 NCH NT/64 ints.
//
// Slots go in groups of NCH chunks of NT: a group's codes are all read before
// any is ranked (one memory round trip per group), and its ranks take one
// exchange of per-(chunk, wave) counts, two barriers per group. A split of one
// group pads its table in the same pass. pre() runs once, right after the
// first group's code loads are issued: loads the caller puts there go out in
// the same memory round trip without the codes waiting behind them.
template <int SRC, int NT, int TR, int NCH, class CodeFn, class PreFn>
__device__ int build_row_table_from(const RowSrc& src, const QRows& r, int64_t qi, int* tab, int* cnt, int* n_comp,
                                    CodeFn code_of, PreFn pre) {
  constexpr int NW = NT / 64, GS = NCH * NT;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ngroups = max(0, r.s_end - r.s_begin + GS - 1) / GS;
  int n_rows = 0, nc = 0;
  // the slots' compressed entries (-1: empty) of group g, at clamped slots
  // and without branches, so the loads are in flight together
  auto load_codes = [&](int g, int (&id)[NCH]) {
    const int base = r.s_begin + g * GS;
    if (src.top_k > 0) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) id[c] = code_of(min(max(base + c * NT + tid, 0), src.top_k - 1));
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) id[c] = -1;
    }
  };
  auto group = [&](int g, const int (&id)[NCH]) {
    const int base = r.s_begin + g * GS;
    int e[NCH];
    bool ok[NCH];
    uint64_t bal[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int j = base + c * NT + tid;
      const int ww = j - src.top_k;  // window slot
      bool okw;
      int row;
      if (SRC == SRC_SPARSE_DEC) {
        okw = ww < r.lim0;
        row = r.w0 + ww;  // this query's window starts at buffer row w0
      } else {
        const int64_t tok = (int64_t)r.lim1 - src.W + 1 + ww;
        okw = tok >= 0 && tok < src.T_tok;
        row = (int)tok;
      }
      const bool is_c = j < src.top_k;
      ok[c] = j < r.s_end && (is_c ? (id[c] >= 0 && id[c] < src.N_max) : okw);
      e[c] = is_c ? id[c] : (int)(0x80000000u | (uint32_t)row);
      // counts of valid slots (and of valid compressed slots) per (chunk,
      // wave) at index c NW + w: the slots' order
      bal[c] = __ballot(ok[c]);
      const uint64_t balc = __ballot(ok[c] && is_c);  // the whole wave votes
      if (l == 0) {
        cnt[c * NW + w] = __popcll(bal[c]);
        cnt[NCH * NW + c * NW + w] = __popcll(balc);
      }
    }
    __syncthreads();
    // rows before each (chunk, this wave): the counts are read together (one
    // LDS round trip) and summed in vector registers. The opaque zero offset
    // keeps them there: read as uniform values they would go to scalar
    // registers one read and one wait at a time.
    int zo = 0;
    asm volatile("" : "+v"(zo));
    int off[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int before = 0, tot = 0;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const int k = cnt[zo + c * NW + v];
        before += v < w ? k : 0;
        tot += k;
        nc += cnt[zo + NCH * NW + c * NW + v];
      }
      off[c] = n_rows + before;
      n_rows += tot;
    }
    const int padded = ngroups == 1 ? (n_rows + TR - 1) / TR * TR : n_rows;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int rank =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[c] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal[c], 0));
      if (ok[c]) {
        tab[off[c] + rank] = e[c];
        // the last row also fills the padding
        if (off[c] + rank == n_rows - 1)
          for (int k = n_rows; k < padded; ++k) tab[k] = e[c];
      }
    }
    __syncthreads();
  };
  // the first group outside the loop, so the waits for its codes count only
  // the loads pre() puts behind them
  int id0[NCH];
  load_codes(0, id0);
  pre();
  if (ngroups > 0) group(0, id0);
  for (int g = 1; g < ngroups; ++g) {
    int id[NCH];
    load_codes(g, id);
    group(g, id);
  }
  if (ngroups > 1) {
    const int padded = (n_rows + TR - 1) / TR * TR;
    if (n_rows > 0 && n_rows + tid < padded) tab[n_rows + tid] = tab[n_rows - 1];
    __syncthreads();
  }
  if (n_comp) *n_comp = __builtin_amdgcn_readfirstlane(nc);
  return __builtin_amdgcn_readfirstlane(n_rows);
}

// The same with the slots' entries read from the top-k output in memory.
template <int SRC, int NT, int TR, int NCH, class PreFn>
__device__ int build_row_table(const RowSrc& src, const QRows& r, int64_t qi, int* tab, int* cnt, int* n_comp,
                               PreFn pre) {
  return build_row_table_from<SRC, NT, TR, NCH>(src, r, qi, tab, cnt, n_comp,
                                           [&](int j) { return src.idx[qi * src.top_k + j]; }, pre);
}

// Address of compacted row c of an HCA split / of a sparse table entry (rows
// of ROWB bytes).
template <int ROWB = 1024>
__device__ __forceinline__ const uint8_t* hca_row(const QRows& r, int c) {
  return c < r.len1 ? r.comp_base + (int64_t)(r.s_begin + c) * ROWB : r.win_base + (int64_t)(r.w0 + c - r.len1) * ROWB;
}
template <int ROWB = 1024>
__device__ __forceinline__ const uint8_t* tab_row(const QRows& r, int e) {
  return e >= 0 ? r.comp_base + (int64_t)e * ROWB : r.win_base + (int64_t)(e & 0x7fffffff) * ROWB;
}

// KV8 rows: dims 0..447 as E4M3 bytes, then the 64 RoPE dims as bf16 (576 B
// in memory). In LDS they sit unswizzled at a 592-byte pitch (148 dwords:
// 16 consecutive rows start in 16 distinct 4-bank groups), the second half
// of a tile 64 bytes further on, so that rows r and r + 16 do not share banks.
template <bool KV8>
struct DecRows {
  static constexpr int SROWB = KV8 ? 576 : bfk::ROWB;            // bytes per row in memory
  static constexpr int NOPE = 448;                               // E4M3 dims of a KV8 row
  static constexpr int PITCH = KV8 ? 592 : bfk::ROWB;            // LDS bytes per row
  static constexpr int TB = KV8 ? bfk::TR * PITCH + 64 : bfk::TILEB;  // LDS bytes per tile
  static __device__ __forceinline__ int lrow(int r) { return KV8 ? r * PITCH + (r >> 4) * 64 : r * bfk::ROWB; }
};

// The tile loop of one workgroup (eight waves): rows rr.n_rows of its
// compacted list (HCA: two contiguous ranges; otherwise the table tab) are
// gathered into the LDS ring and attended by the query held in qb; o, m_ref
// and l_run receive the unnormalised output and the (m, l) partials of the
// lane's head, exponent base 2. ring holds NBUF tiles of DecRows<KV8>::TB
// bytes; xchg is the S^T partial exchange buffer.
template <int SRC, bool KV8>
__device__ __forceinline__ void dec_tiles(const QRows& rr, const int* tab, uint8_t* ring, f32x4_t (*xchg)[2][64],
                                          bf16x8_t (&qb)[8], float scale_log2, f32x4_t (&o)[16], float& m_ref,
                                          float& l_run) {
  using namespace bfk;
  using DR = DecRows<KV8>;
  constexpr int SROWB = DR::SROWB, NOPE = DR::NOPE, TB = DR::TB;
  auto lrow = [](int r) { return DR::lrow(r); };
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = l >> 4, l16 = l & 15;
  const int dh = w >> 2;
  const int n_rows = rr.n_rows;
  const int ntiles = (n_rows + TR - 1) / TR;
  (void)NOPE;
  // ---- row loads: wave w moves rows 4w .. 4w+3 of a tile; the lane offset
  // applies the tile's chunk swizzle on the global side
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = KV8 ? (uint32_t)(l * 16) : (uint32_t)((l ^ swz(4 * w + i)) * 16);
  // a KV8 row is 36 lanes x 16 bytes; the other lanes' LDS slots belong to the next row
  auto row_dma = [&](const uint8_t* rp, int i, uint32_t dst) {
    if (!KV8 || l < SROWB / 16) dma_row(uniform_ptr(rp), voff[i], __builtin_amdgcn_readfirstlane(dst));
  };
  auto issue = [&](int t) {
    const int c0 = t * TR + 4 * w;  // first of this wave's four rows
    const uint32_t dst = ring_lds + (uint32_t)((t & (NBUF - 1)) * TB);
    if (SRC == SRC_HCA_DEC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int c = c0 + i;
        if (c >= n_rows) c = t * TR;  // rows past the end repeat a valid row; they are masked
        row_dma(hca_row<SROWB>(rr, c), i, dst + lrow(4 * w + i));
      }
    } else {
      const u32x4_t e4 = *reinterpret_cast<const u32x4_t*>(&tab[c0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (int)__builtin_amdgcn_readfirstlane(e4[i]);
        row_dma(tab_row<SROWB>(rr, e), i, dst + lrow(4 * w + i));
      }
    }
  };

#pragma unroll
  for (int nt = 0; nt < 16; ++nt) o[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  m_ref = -INFINITY;  // `head`: exponent reference, partial sum of this lane's rows
  l_run = 0.0f;

  // LDS offsets (within a tile, plus 512 dh) of this lane's QK and PV reads
  int qofs[2][4], pofs[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = mt * 16 + l16;
#pragma unroll
    for (int v = 0; v < 4; ++v) qofs[mt][v] = row * ROWB + (((4 * v + G) ^ swz(row)) * 16) + dh * 512;
  }
  {
    const int rowa = G * 4 + (l16 >> 2), rowb = rowa + 16;
    const int c0 = (l16 >> 1) & 1, cb = (l16 & 1) * 8;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      pofs[0][u] = rowa * ROWB + (((2 * u + c0) ^ swz(rowa)) * 16) + cb + dh * 512;
      pofs[1][u] = rowb * ROWB + (((2 * u + c0) ^ swz(rowb)) * 16) + cb + dh * 512;
    }
  }
  // KV8 offsets. S^T operand: row mt*16 + l16 (its E4M3 dims are its bytes).
  // V^T operand of the E4M3 dims (ds_read_b64_tr_b8): within a 16-lane group,
  // lanes 2k and 2k+1 give the addresses of row r_k, columns 0-7 and 8-15 of
  // a 16-dim block, and lane j receives column j of rows r_0 .. r_7; r_k
  // follows P's K order, rows 4G + k and then 16 + 4G + (k-4). The RoPE dims
  // use the 16-bit transposed read (lane: row 4G + l16/4 (+16), four columns).
  int kofs8[2], vofs8, rofs8[2];
  {
    kofs8[0] = lrow(l16);
    kofs8[1] = lrow(16 + l16);
    const int k = l16 >> 1;
    vofs8 = lrow(k < 4 ? 4 * G + k : 16 + 4 * G + (k - 4)) + 8 * (l16 & 1);
    const int rowa = G * 4 + (l16 >> 2);
    rofs8[0] = lrow(rowa) + NOPE + 8 * (l16 & 3);
    rofs8[1] = lrow(rowa + 16) + NOPE + 8 * (l16 & 3);
  }

  // consume Q here: the compiler's wait for its loads lands before the first
  // row load, so its load tracking never waits on rows in flight in the loop
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(qb[s]));
  constexpr int PER = 4;  // row loads per wave per tile
  for (int t = 0; t < ntiles && t < NBUF - 1; ++t) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    const int ahead = min(NBUF - 2, ntiles - 1 - t);  // tiles issued after this one
    if (ahead >= 2)
      vm_barrier<2 * PER>();
    else if (ahead == 1)
      vm_barrier<PER>();
    else
      vm_barrier<0>();
    // the buffer of tile t-1 is free: every wave has passed this barrier
    if (t + NBUF - 1 < ntiles) issue(t + NBUF - 1);
    const uint8_t* R = ring + (t & (NBUF - 1)) * TB;

    // ---- partial S^T over this wave's 256 dims, two 16-row M-tiles
    f32x4_t sa = f32x4_t{0.f, 0.f, 0.f, 0.f}, sb = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (KV8) {
      // dims 256 dh + 32 s + 8 G: E4M3 bytes below 448 (dh = 0, or s < 6),
      // bf16 above (dh = 1, s = 6, 7)
      auto k8 = [&](int mt, int s) {
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(R + kofs8[mt] + 256 * dh + 32 * s + 8 * G);
        return as_bf16x8(u32x4_t{fp8x2_to_bf16x2(v[0], false), fp8x2_to_bf16x2(v[0], true),
                                 fp8x2_to_bf16x2(v[1], false), fp8x2_to_bf16x2(v[1], true)});
      };
      auto kr16 = [&](int mt, int s) {
        return as_bf16x8(*reinterpret_cast<const u32x4_t*>(R + kofs8[mt] + NOPE + 2 * (32 * (s - 6) + 8 * G)));
      };
#pragma unroll
      for (int s = 0; s < 6; ++s) {
        sa = mfma16(k8(0, s), qb[s], sa);
        sb = mfma16(k8(1, s), qb[s], sb);
      }
      if (dh == 0) {
#pragma unroll
        for (int s = 6; s < 8; ++s) {
          sa = mfma16(k8(0, s), qb[s], sa);
          sb = mfma16(k8(1, s), qb[s], sb);
        }
      } else {
#pragma unroll
        for (int s = 6; s < 8; ++s) {
          sa = mfma16(kr16(0, s), qb[s], sa);
          sb = mfma16(kr16(1, s), qb[s], sb);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8_t a0 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(R + qofs[0][s & 3] + (s >> 2) * 256));
        const bf16x8_t a1 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(R + qofs[1][s & 3] + (s >> 2) * 256));
        sa = mfma16(a0, qb[s], sa);
        sb = mfma16(a1, qb[s], sb);
      }
    }
    // ---- swap partials with the other dim half
    xchg[w][0][l] = sa;
    xchg[w][1][l] = sb;
    vm_barrier<63>();
    sa += xchg[w ^ 4][0][l];
    sb += xchg[w ^ 4][1][l];

    // ---- softmax of `head` over this lane's 8 rows (mt*16 + 4G + r), exp2 domain
    const int nvalid = n_rows - t * TR;
    float sv[8];
    float lm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float va = (4 * G + r < nvalid) ? sa[r] * scale_log2 : -INFINITY;
      const float vb = (16 + 4 * G + r < nvalid) ? sb[r] * scale_log2 : -INFINITY;
      sv[r] = va;
      sv[4 + r] = vb;
      lm = fmaxf(lm, fmaxf(va, vb));
    }
    // m_ref only moves when a row exceeds it by RESCALE_SLACK (always on the first tile)
    if (__builtin_expect(__any(lm > m_ref + RESCALE_SLACK), 0)) {
      float tmax = fmaxf(lm, shfl_xor(lm, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float m_new = tmax > m_ref + RESCALE_SLACK ? tmax : m_ref;
      const float alpha = (m_new == m_ref) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
      m_ref = m_new;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, G * 4 + r, 64);  // O rows are heads 16 hg + 4G + r
#pragma unroll
      for (int nt = 0; nt < 16; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[nt][r] *= ar[r];
    }
    const float mr = (m_ref == -INFINITY) ? 0.0f : m_ref;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(sv[i] - mr);
      l_run += pv[i];
    }

    // ---- O += P R over this wave's dims; K order: rows 4G + 0..3, then 16 + 4G + 0..3
    const bf16x8_t pa = as_bf16x8(u32x4_t{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])});
    if constexpr (KV8) {
      // N-tile nt holds dims 256 dh + 16 nt: E4M3 below 448, bf16 for dh = 1, nt >= 12
      auto v8 = [&](int nt) {
        const i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (i32x2_t __attribute__((address_space(3)))*)(R + vofs8 + 256 * dh + 16 * nt));
        return as_bf16x8(u32x4_t{fp8x2_to_bf16x2((uint32_t)r[0], false), fp8x2_to_bf16x2((uint32_t)r[0], true),
                                 fp8x2_to_bf16x2((uint32_t)r[1], false), fp8x2_to_bf16x2((uint32_t)r[1], true)});
      };
      auto v16 = [&](int nt) {
        const int cofs = 2 * 16 * (nt - 12);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4_t __attribute__((address_space(3)))*)(R + rofs8[0] + cofs));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4_t __attribute__((address_space(3)))*)(R + rofs8[1] + cofs));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int nt = 0; nt < 12; ++nt) o[nt] = mfma16(pa, v8(nt), o[nt]);
      if (dh == 0) {
#pragma unroll
        for (int nt = 12; nt < 16; ++nt) o[nt] = mfma16(pa, v8(nt), o[nt]);
      } else {
#pragma unroll
        for (int nt = 12; nt < 16; ++nt) o[nt] = mfma16(pa, v16(nt), o[nt]);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) {
        auto* pa4 = (s16x4_t __attribute__((address_space(3)))*)(R + pofs[0][nt & 7] + (nt >> 3) * 256);
        auto* pb4 = (s16x4_t __attribute__((address_space(3)))*)(R + pofs[1][nt & 7] + (nt >> 3) * 256);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pa4);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pb4);
        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[nt] = mfma16(pa, bv, o[nt]);
      }
    }
  }

}

// The query prologue and output epilogue of a decode step on raw queries
// (DeepSeek V4 脱离 CUDA 全栈国产化, section 二, 其他辅助设计: RMSNorm of the
// queries before the core attention, rotary encoding of the last R dims;
// liduos.com "deepseek-v4-engineering-tradeoffs", 1M Context 的结构与取舍:
// the output takes the inverse rotation). flags: 1 norm, 2 rotation.
struct QkArgs {
  int flags;
  const float* gamma;  // [D] or NULL (ones)
  float eps;
  int R;               // rotated trailing dims, even, R / 2 <= 64
  double log2_theta;
  const int32_t* pos;  // [queries]: the rotation's position
};

// cos and sin of the angle p * theta^(-2i/R) of rotated pair i: the angle
// formed and reduced to [-pi, pi] in double precision (at p = 2^20 the fp32
// product alone would be off by up to 0.06 rad; the double one by ~1e-11),
// then the fp32 sincos of the small remainder
__device__ __forceinline__ void rope_cs(double p, int i, int R, double log2_theta, float& c, float& s) {
  const double a = p * exp2(-2.0 * (double)i / (double)R * log2_theta);
  const double r = a - 6.283185307179586 * rint(a * 0.15915494309189535);
  sincosf((float)r, &s, &c);
}

// This lane's (cos, sin) of pair `lane` (lanes below R / 2), for the lanes
// that rotate a pair to read by a shuffle: each angle formed once per wave.
__device__ __forceinline__ void rope_lane(const QkArgs& qk, int64_t qi, float& c, float& s) {
  const int l = threadIdx.x & 63;
  c = 1.0f;
  s = 0.0f;
  if ((qk.flags & 2) && l < qk.R / 2) rope_cs((double)qk.pos[qi], l, qk.R, qk.log2_theta, c, s);
}

// The prologue on the decode tile loop's query operand: lane (head, G) of
// wave (hg, dh) holds dims 256 dh + 32 s + 8 G .. +7 of its head in qb[s].
// RMSNorm over the head's 512 dims (the waves w and w ^ 4 add their halves
// through `half`, 8 x 16 floats of LDS), then the rotation of the pairs of
// the last R dims (consecutive, inside a lane's 8), in fp32, rounded back to
// bf16 once. All threads of the workgroup call it.
__device__ __forceinline__ void qk_prologue(bf16x8_t (&qb)[8], float* half, const QkArgs& qk, int64_t qi) {
  constexpr int D = 512;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = l >> 4, l16 = l & 15, dh = w >> 2;
  float v[8][8];
#pragma unroll
  for (int s = 0; s < 8; ++s) unpack_bf16x8(__builtin_bit_cast(u32x4_t, qb[s]), v[s]);
  if (qk.flags & 1) {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[s][e] * v[s][e];
    ss += shfl_xor(ss, 16);
    ss += shfl_xor(ss, 32);
    if (G == 0) half[w * 16 + l16] = ss;
    __syncthreads();
    const float tot = half[w * 16 + l16] + half[(w ^ 4) * 16 + l16];
    __syncthreads();  // `half` is free again
    const float r = 1.0f / sqrtf(tot / (float)D + qk.eps);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[s][e] *= r * (qk.gamma ? qk.gamma[dh * 256 + s * 32 + G * 8 + e] : 1.0f);
  }
  if (qk.flags & 2) {
    const int s0 = D - qk.R;  // even: a pair never straddles it
    float cl, sl;
    rope_lane(qk, qi, cl, sl);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (dh * 256 + s * 32 + 32 <= s0) continue;  // uniform: no rotated dim in this chunk
      const int d0 = dh * 256 + s * 32 + G * 8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bool rot = d0 + e >= s0;
        const int src = rot ? (d0 + e - s0) >> 1 : 0;
        const float c = __shfl(cl, src, 64), sn = __shfl(sl, src, 64);
        if (rot) {
          const float x0 = v[s][e], x1 = v[s][e + 1];
          v[s][e] = x0 * c - x1 * sn;
          v[s][e + 1] = x0 * sn + x1 * c;
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qb[s] = as_bf16x8(u32x4_t{pack_bf16x2(v[s][0], v[s][1]), pack_bf16x2(v[s][2], v[s][3]),
                              pack_bf16x2(v[s][4], v[s][5]), pack_bf16x2(v[s][6], v[s][7])});
}

}  // namespace csa
