// Exact top-k selection over indexer scores, for gfx950.
//
// What is computed (DeepSeek V4 脱离 CUDA 全栈国产化, deepseek.csdn.net,
// section 二, CSA step 2: keep the top-k compressed blocks, 512 for Flash and
// 1024 for Pro): for a query row with V visible scores, the K = min(k, V)
// entries with the largest scores; equal scores go to the lower index, so the
// set is unique. Indices are written in ascending order, the row padded with
// -1. Batch invariance (the same page, section 八, on the MegaMoE kernel and
// training stability: a token's result must not depend on its batch) follows
// from the algorithm: the selection is exact, so the output depends on the
// row alone.
//
// Algorithm. Scores become order-preserving uint32 keys; the top 11 bits of
// a key are its digit (sign, exponent, two mantissa bits: four bins per
// binade). A 2048-bin digit histogram of the row names the threshold bin b:
// fewer than K keys have a digit above b, at least K have a digit >= b. The
// candidates -- every key with digit >= b, usually K plus a few hundred --
// are compacted in index order (ballot prefix sums), and an exact radix
// select among them finds the K-th key T and how many keys equal to T are
// kept (the lowest-index ones). A last ordered pass writes the selection.
//
// The histogram is only a hint. The compaction counts the candidates
// exactly; whenever they are fewer than K or too many for the buffer, the
// row is selected exactly from the full score row instead. So a stale,
// partial or garbage histogram can cost time but never changes a result,
// and the workspace's contents on entry never matter.
//
// Workgroups are 256 threads (one wave per SIMD): every instruction of a
// wave-uniform step then costs one issue per SIMD, not four. Rows of up to
// 16384 keys: one workgroup per row holds the keys in registers and finishes
// the row in one launch (topk_row_kernel), with the histogram passed in by
// the prefill indexer or built with LDS atomics. Longer rows are spread over
// 4096-key chunks: topk_filter_kernel compacts each chunk's candidates into a
// per-chunk list, reading the row's histogram that the decode scan
// accumulated (or topk_clear_kernel + topk_hist_kernel built);
// topk_final_kernel gathers the lists in chunk order, selects, writes, and
// clears the row's histogram for the next call. No result depends on the
// order of any atomic operation.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int TK_NT = 256;
constexpr int TK_NW = TK_NT / 64;
constexpr int TK_BINS = 2048;
constexpr int TK_BPL = TK_BINS / TK_NT;    // histogram bins per thread
constexpr int TK_DSHIFT = 21;              // digit = key >> 21 (11 bits)
constexpr int TK_ROW_MAX = 16384;          // keys of a row finished by one workgroup
constexpr int TK_ROW_CAP = 4096;           // candidates of topk_row_kernel (32 KB of LDS)
constexpr int TK_FCH = 4096;               // keys per chunk workgroup: four wave segments of 1024
constexpr int TK_SEG = TK_FCH / TK_NW;     // keys per wave segment
constexpr int TK_WCAP = 512;               // candidates kept per wave segment
constexpr int TK_LDS_MAX = 160 * 1024;     // LDS of a workgroup on gfx950
constexpr uint32_t TK_HINT_CLAMP = (1u << 20) - 1;  // keeps the bin sums inside int32

__device__ __forceinline__ float key_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int below_cnt(uint64_t msk) {  // popcount of the mask's bits below this lane
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
}
// wave exclusive prefix and total of v in 0..7
__device__ __forceinline__ int excl3(int v, int& total) {
  const uint64_t b0 = __ballot(v & 1), b1 = __ballot(v & 2), b2 = __ballot(v & 4);
  total = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
  return below_cnt(b0) + 2 * below_cnt(b1) + 4 * below_cnt(b2);
}

// Given the counts of the TK_BINS bins, find the bin b with (count above b) <
// need <= (count of bins >= b). All threads take part: lane l of wave w holds
// the eight bins below TK_BINS - 512 w - 8 l (one inclusive scan over lanes
// of their sums), the waves' totals meet in tot[0..TK_NW), and the lane
// holding the threshold publishes out[0] = b, out[1] = count above b, out[2] =
// count of b. If no bin qualifies (the counts sum to less than need) out[] is
// left as it was. Ends with a barrier that publishes out[] and frees hist and
// tot.
__device__ __forceinline__ void find_bin_block(const uint32_t* hist, int need, int* tot, int* out) {
  static_assert(TK_BPL == 8, "eight bins per lane");
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int lo = TK_BINS - 8 * (t + 1);  // this lane's lowest bin; its bins are lo .. lo + 7
  const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(hist + lo);
  const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(hist + lo + 4);
  const int own = (int)(c0[0] + c0[1] + c0[2] + c0[3] + c1[0] + c1[1] + c1[2] + c1[3]);
  const int inc = wave_incl_scan_dpp(own);
  if (l == 63) tot[wv] = inc;
  __syncthreads();
  int above = inc - own;  // bins above this lane's, within the wave
#pragma unroll
  for (int u = 0; u < TK_NW; ++u) above += u < wv ? tot[u] : 0;
  if (above < need && need <= above + own) {
    const int c[8] = {(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                      (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
    int a = above, bin = lo, cb = c[0];
    bool found = false;
#pragma unroll
    for (int i = 7; i >= 0; --i) {  // from the top bin down
      if (!found && need <= a + c[i]) {
        found = true;
        bin = lo + i;
        cb = c[i];
      } else if (!found) {
        a += c[i];
      }
    }
    out[0] = bin;
    out[1] = a;
    out[2] = cb;
  }
  __syncthreads();
}

struct TopkArgs {
  const float* scores;     // [rows, N_max]
  const int32_t* q_pos;
  const int32_t* n_comp;
  int64_t Tq, N_max;
  int m, top_k;
  int32_t* out_idx;        // [rows, top_k]
  float* out_score;        // nullable
  uint32_t* hint;          // [rows, TK_BINS] digit histogram; NULL: built by the row kernel
  int clear_hint;          // the hint was accumulated by the scan: clear it once consumed
  uint32_t* ctr;           // [rows] arrival counters of the chunk workgroups, zero on entry
  uint32_t* wkey;          // [rows, nseg, TK_WCAP] candidates per wave segment
  int32_t* widx;
  int32_t* wcnt;           // [rows, nseg]; TK_WCAP + 1 marks an overflowing segment
  int nseg;                // wave segments per row of N_max keys
  int cap;                 // candidates the last workgroup of a row can hold (dynamic LDS)
};

__device__ __forceinline__ int64_t visible_of(const TopkArgs& a, int64_t row) {
  const int64_t b = row / a.Tq;
  const int64_t v = min((int64_t)a.n_comp[b], ((int64_t)a.q_pos[row] + 1) / a.m);
  return max((int64_t)0, min(v, a.N_max));
}

// Where the select and the compaction read keys: the workgroup's LDS cache,
// or a row of scores in memory converted on the fly (positions >= lim read 0).
struct LdsKeys {
  const uint32_t* kc;
  __device__ __forceinline__ u32x4_t load4(int i4) const { return reinterpret_cast<const u32x4_t*>(kc)[i4]; }
  __device__ __forceinline__ uint32_t load1(int i) const { return kc[i]; }
};
struct RowKeys {
  const float* s;
  int lim;
  bool aligned;
  __device__ __forceinline__ u32x4_t load4(int i4) const {
    const int p = 4 * i4;
    if (aligned && p + 3 < lim) {
      const f32x4_t v = reinterpret_cast<const f32x4_t*>(s)[i4];
      return u32x4_t{f32_key(v[0]), f32_key(v[1]), f32_key(v[2]), f32_key(v[3])};
    }
    u32x4_t r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = p + e < lim ? f32_key(s[p + e]) : 0u;
    return r;
  }
  __device__ __forceinline__ uint32_t load1(int i) const { return f32_key(s[i]); }
};

// Exact K-th largest key T of keys [0, n) (0 < K < n) and how many keys equal
// to T belong to the top K (`need`). All threads call it. The digits start
// below the common prefix of the smallest and largest key, so the first
// histogram spreads over the keys' own range.
template <class KS>
__device__ void block_select(const KS& ks, int n, int K, uint32_t* hist, int* red, int* res, uint32_t& T,
                             int& need) {
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  need = K;
  const int n4 = n >> 2;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int i = t; i < n4; i += TK_NT) {
    const u32x4_t k4 = ks.load4(i);
    kmin = min(min(kmin, k4[0]), min(k4[1], min(k4[2], k4[3])));
    kmax = max(max(kmax, k4[0]), max(k4[1], max(k4[2], k4[3])));
  }
  for (int i = 4 * n4 + t; i < n; i += TK_NT) {
    const uint32_t k = ks.load1(i);
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
  kmin = wave_min_u32_dpp(kmin);
  kmax = wave_max_u32_dpp(kmax);
  if (l == 0) {
    red[wv] = (int)kmin;
    red[TK_NW + wv] = (int)kmax;
  }
  for (int i = t; i < TK_BINS; i += TK_NT) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < TK_NW; ++u) {
    kmin = min(kmin, (uint32_t)red[u]);
    kmax = max(kmax, (uint32_t)red[TK_NW + u]);
  }
  if (kmin == kmax) {
    T = kmin;  // all keys equal: the K lowest positions
    __syncthreads();  // every wave has read red[] before the caller reuses it
    return;
  }
  int R = 32 - __builtin_clz(kmin ^ kmax);  // bits below the common prefix
  uint32_t prefix = R >= 32 ? 0u : (kmin >> R);
#pragma unroll 1
  for (int pass = 0; R > 0; ++pass) {
    const int nbits = min(11, R);
    const int shift = R - nbits;
    const uint32_t dmask = (1u << nbits) - 1u;
    uint32_t* h = hist;
    auto add = [&](uint32_t k) {
      if (R >= 32 || (k >> R) == prefix) atomicAdd(&h[(k >> shift) & dmask], 1u);
    };
    for (int i0 = t; i0 < n4; i0 += 4 * TK_NT) {
      u32x4_t k4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) k4[u] = (i0 + u * TK_NT < n4) ? ks.load4(i0 + u * TK_NT) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (i0 + u * TK_NT >= n4) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) add(k4[u][e]);
      }
    }
    for (int i = 4 * n4 + t; i < n; i += TK_NT) add(ks.load1(i));
    __syncthreads();
    find_bin_block(h, need, red, res);
    prefix = (prefix << nbits) | (uint32_t)res[0];
    need -= res[1];
    if (need == res[2] && shift > 0) {
      // every key of the bin is selected: the threshold is just below the
      // bin. Its lower edge exceeds the smallest key (K < n keys lie at or
      // above it), so it is at least 1.
      T = (prefix << shift) - 1u;
      need = 0;
      __syncthreads();  // every wave has read res[] before the caller reuses it
      return;
    }
    R = shift;
    if (R > 0) {
      for (int i = t; i < TK_BINS; i += TK_NT) h[i] = 0;
      __syncthreads();
    }
  }
  T = prefix;  // take all keys > T and the `need` lowest-position keys == T
}

// Ordered compaction of the selection in position order: all keys > T and
// the first `need` keys == T (every key when all == true). emit(pos, key, i)
// receives output slot pos < top_k, the key and its position; slots K..top_k-1
// go to pad(pos). Each wave owns a contiguous segment; a lane handles 4
// consecutive keys per step; index-order prefixes come from ballots of the
// bits of the per-lane counts (0..4).
template <class KS, class Emit, class Pad>
__device__ void block_compact(const KS& ks, int n, int K, bool all, uint32_t T, int need, int top_k, int* red,
                              Emit emit, Pad pad) {
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int seg = ((n + TK_NW - 1) / TK_NW + 255) / 256 * 256;
  const int s_lo = min(n, wv * seg), s_hi = min(n, s_lo + seg);
  int gt = 0, eq = 0;
  if (!all) {
    for (int base = s_lo; base < s_hi; base += 512) {
      u32x4_t k4[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i0 = base + u * 256 + 4 * l;
        k4[u] = i0 < s_hi ? ks.load4(i0 >> 2) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool in = base + u * 256 + 4 * l + e < s_hi;
          gt += in && k4[u][e] > T;
          eq += in && k4[u][e] == T;
        }
    }
    gt = wave_sum_dpp(gt);
    eq = wave_sum_dpp(eq);
  }
  if (l == 0) {
    red[wv] = all ? (s_hi - s_lo) : gt;
    red[TK_NW + wv] = eq;
  }
  __syncthreads();
  int eq_before = 0, sel_before = 0;
  {
    int gs[TK_NW], es[TK_NW];
#pragma unroll
    for (int u = 0; u < TK_NW; ++u) {
      gs[u] = red[u];
      es[u] = red[TK_NW + u];
    }
#pragma unroll
    for (int u = 0; u < TK_NW; ++u) {
      const bool before = u < wv;
      sel_before += before ? gs[u] + (all ? 0 : max(0, min(need - eq_before, es[u]))) : 0;
      eq_before += before ? es[u] : 0;
    }
  }
  int run_sel = 0, run_eq = 0;
  for (int base = s_lo; base < s_hi; base += 256) {
    const int i0 = base + 4 * l;
    const u32x4_t k4 = i0 < s_hi ? ks.load4(i0 >> 2) : u32x4_t{0, 0, 0, 0};
    bool in[4], eqf[4], sel[4];
    int ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      in[e] = i0 + e < s_hi;
      eqf[e] = !all && in[e] && k4[e] == T;
      ne += eqf[e];
    }
    int eq_tot;
    int r = eq_before + run_eq + excl3(ne, eq_tot);
    int ns = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sel[e] = in[e] && (all || k4[e] > T || (eqf[e] && r < need));
      r += eqf[e];
      ns += sel[e];
    }
    int sel_tot;
    int pos = sel_before + run_sel + excl3(ns, sel_tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (sel[e]) {
        if (pos < top_k) emit(pos, k4[e], i0 + e);
        ++pos;
      }
    }
    run_sel += sel_tot;
    run_eq += eq_tot;
  }
  for (int i = K + t; i < top_k; i += TK_NT) pad(i);
  __syncthreads();  // red[] is free again
}

// Keys held in registers by a TK_NT-thread workgroup: KPT per thread. Wave w
// owns positions [lo + w*64*KPT, +64*KPT); in step j (KPT/4 steps) lane l
// holds the four positions base_j + 4 l + e, base_j = lo + w*64*KPT + 256 j.
template <int KPT>
struct RegKeys {
  static_assert(KPT % 4 == 0, "whole 16-byte steps");
  uint32_t k[KPT];
  __device__ __forceinline__ int pos(int lo, int j, int e) const {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    return lo + w * 64 * KPT + 256 * j + 4 * l + e;
  }
  // keys of positions [lo, hi) of src (hi - lo <= TK_NT KPT); others read 0
  // and are never candidates (the callers test positions against hi)
  __device__ __forceinline__ void load(const float* src, int lo, int hi) {
    const bool al = ((reinterpret_cast<uintptr_t>(src + lo)) & 15) == 0;
#pragma unroll
    for (int j = 0; j < KPT / 4; ++j) {
      const int p = pos(lo, j, 0);
      if (al && p + 3 < hi) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + p);
#pragma unroll
        for (int e = 0; e < 4; ++e) k[4 * j + e] = f32_key(v[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) k[4 * j + e] = p + e < hi ? f32_key(src[p + e]) : 0u;
      }
    }
  }
};

// Ordered compaction of the register keys whose position is below hi and
// whose digit is at least b: their (key, position) pairs go to slots
// [0, M) in position order through put(slot, key, pos) (called for slot <
// cap only). Returns M, the exact candidate count (uniform). All threads call
// it; red holds TK_NW ints; ends with a barrier after red is read.
template <int KPT, class Put>
__device__ int reg_compact(const RegKeys<KPT>& rk, int lo, int hi, uint32_t b, int cap, int* red, Put put) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  int pre[KPT / 4];
  int wtot = 0;
#pragma unroll
  for (int j = 0; j < KPT / 4; ++j) {
    int n = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) n += (rk.pos(lo, j, e) < hi) && (rk.k[4 * j + e] >> TK_DSHIFT) >= b;
    int st;
    pre[j] = wtot + excl3(n, st);
    wtot += st;
  }
  if (l == 0) red[w] = wtot;
  __syncthreads();
  int off = 0, M = 0;
#pragma unroll
  for (int u = 0; u < TK_NW; ++u) {
    const int v = red[u];
    off += u < w ? v : 0;
    M += v;
  }
  if (M <= cap) {
#pragma unroll
    for (int j = 0; j < KPT / 4; ++j) {
      int s = off + pre[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = rk.pos(lo, j, e);
        if (p < hi && (rk.k[4 * j + e] >> TK_DSHIFT) >= b) {
          put(s, rk.k[4 * j + e], p);
          ++s;
        }
      }
    }
  }
  __syncthreads();  // red[] is free again; the puts are done
  return M;
}

// The row's visible count is at most the top-k: every visible entry, in order.
__device__ __forceinline__ void emit_all_visible(const TopkArgs& a, int64_t row, int V) {
  const int64_t obase = row * (int64_t)a.top_k;
  const float* src = a.scores + row * a.N_max;
  for (int i = threadIdx.x; i < a.top_k; i += TK_NT) {
    a.out_idx[obase + i] = i < V ? i : -1;
    if (a.out_score) a.out_score[obase + i] = i < V ? src[i] : -INFINITY;
  }
}

template <class KS, class Idx>
__device__ __forceinline__ void write_selection(const TopkArgs& a, int64_t row, const KS& keys, int n, int K, bool all,
                                                uint32_t T, int need, int* red, Idx idx_of) {
  const int64_t obase = row * (int64_t)a.top_k;
  block_compact(
      keys, n, K, all, T, need, a.top_k, red,
      [&](int pos, uint32_t key, int i) {
        a.out_idx[obase + pos] = idx_of(i);
        if (a.out_score) a.out_score[obase + pos] = key_f32(key);
      },
      [&](int i) {
        a.out_idx[obase + i] = -1;
        if (a.out_score) a.out_score[obase + i] = -INFINITY;
      });
}

// Exact selection of the whole row from memory: the path taken when the
// histogram hint does not hold (too few or too many candidates).
__device__ void select_row_from_memory(const TopkArgs& a, int64_t row, int V, int K, uint32_t* hist, int* red,
                                       int* res) {
  const float* src = a.scores + row * a.N_max;
  const RowKeys keys{src, V, (reinterpret_cast<uintptr_t>(src) & 15) == 0};
  uint32_t T = 0;
  int need = 0;
  block_select(keys, V, K, hist, red, res, T, need);
  write_selection(a, row, keys, V, K, false, T, need, red, [](int i) { return (int32_t)i; });
}

// Block sum of one int per thread (uniform result); red holds TK_NW ints.
__device__ __forceinline__ int block_sum(int v, int* red) {
  v = wave_sum_dpp(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int u = 0; u < TK_NW; ++u) s += red[u];
  __syncthreads();
  return s;
}

// The K-th key among M candidates cached in LDS (keys ck, position order),
// the candidates being every key whose digit is at least b, and write the
// row. The threshold lies in digit b when fewer than K candidates have a
// larger digit; the next 11 bits of the keys of digit b then name its
// sub-bin, and (unless the sub-bin is taken whole) the last 10 bits the key
// itself: one or two histogram passes over the candidates. Any inconsistency
// (a hint that did not hold) falls back to a full radix select over the
// candidates, which contain the top K either way.
template <class Idx>
__device__ void select_in_candidates(const TopkArgs& a, int64_t row, const uint32_t* ck, int M, int K, int b,
                                     uint32_t* hist, int* red, int* res, Idx idx_of) {
  const int t = threadIdx.x;
  const LdsKeys keys{ck};
  if (M == K) {
    write_selection(a, row, keys, M, K, true, 0u, 0, red, idx_of);
    return;
  }
  uint32_t T = 0;
  int need = 0;
  bool done = false;
  if (b >= 0) {
    for (int i = t; i < TK_BINS; i += TK_NT) hist[i] = 0;
    __syncthreads();
    int above = 0;
    for (int i = t; i < M; i += TK_NT) {
      const uint32_t k = ck[i];
      const int d = (int)(k >> TK_DSHIFT);
      above += d > b;
      if (d == b) atomicAdd(&hist[(k >> 10) & (TK_BINS - 1)], 1u);
    }
    above = block_sum(above, red);  // its barriers also publish the histogram
    const int need1 = K - above;
    if (need1 > 0) {
      if (t == 0) res[0] = -1;
      __syncthreads();
      find_bin_block(hist, need1, red, res);
      const int s2 = res[0];
      const uint32_t P = ((uint32_t)b << 11) | (uint32_t)max(s2, 0);  // 22-bit key prefix
      if (s2 >= 0 && P > 0) {
        const int need2 = need1 - res[1];
        if (need2 == res[2]) {
          T = (P << 10) - 1u;  // the sub-bin is taken whole
          need = 0;
          done = true;
        } else {
          for (int i = t; i < TK_BINS; i += TK_NT) hist[i] = 0;
          __syncthreads();
          for (int i = t; i < M; i += TK_NT) {
            const uint32_t k = ck[i];
            if ((k >> 10) == P) atomicAdd(&hist[k & 1023u], 1u);
          }
          if (t == 0) res[0] = -1;
          __syncthreads();
          find_bin_block(hist, need2, red, res);
          if (res[0] >= 0) {
            T = (P << 10) | (uint32_t)res[0];
            need = need2 - res[1];
            done = true;
          }
        }
      }
    }
  }
  if (!done) block_select(keys, M, K, hist, red, res, T, need);
  write_selection(a, row, keys, M, K, false, T, need, red, idx_of);
}

// Copy a row's histogram hint into LDS, clamping each bin so that any sum of
// bins stays inside int32 (a clamped bin only weakens the hint).
__device__ __forceinline__ void load_hint(const uint32_t* h, uint32_t* hist) {
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < TK_BPL / 4; ++u) {
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(h)[t + u * TK_NT];
    reinterpret_cast<u32x4_t*>(hist)[t + u * TK_NT] =
        u32x4_t{min(v[0], TK_HINT_CLAMP), min(v[1], TK_HINT_CLAMP), min(v[2], TK_HINT_CLAMP), min(v[3], TK_HINT_CLAMP)};
  }
}
__device__ __forceinline__ void clear_hint(uint32_t* h) {
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < TK_BPL / 4; ++u) reinterpret_cast<u32x4_t*>(h)[t + u * TK_NT] = u32x4_t{0u, 0u, 0u, 0u};
}

// ----------------------------------------------------------------------------
// Rows of up to TK_ROW_MAX keys: one workgroup per row, keys in registers
// ----------------------------------------------------------------------------
template <int KPT>
__global__ void __launch_bounds__(TK_NT) topk_row_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[TK_BINS];
  __shared__ __attribute__((aligned(16))) int red[2 * TK_NW], res[4];
  __shared__ __attribute__((aligned(16))) uint32_t ck[TK_ROW_CAP];
  __shared__ __attribute__((aligned(16))) int32_t ci[TK_ROW_CAP];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int V = (int)visible_of(a, row);
  const int K = min(a.top_k, V);
  uint32_t* h = a.hint ? a.hint + row * TK_BINS : nullptr;
  if (K == V) {
    emit_all_visible(a, row, V);
    if (h && a.clear_hint) clear_hint(h);
    return;
  }
  const float* src = a.scores + row * a.N_max;
  RegKeys<KPT> rk;
  rk.load(src, 0, V);
  // digit histogram of the row (exact), or its hint
  if (h) {
    load_hint(h, hist);
  } else {
    for (int i = t; i < TK_BINS; i += TK_NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (rk.pos(0, j, e) < V) atomicAdd(&hist[rk.k[4 * j + e] >> TK_DSHIFT], 1u);
  }
  if (t == 0) res[0] = -1;
  __syncthreads();
  find_bin_block(hist, K, red, res);
  const int b = res[0];
  int M = -1;
  if (b >= 0)
    M = reg_compact(rk, 0, V, (uint32_t)b, TK_ROW_CAP, red, [&](int s, uint32_t key, int p) {
      ck[s] = key;
      ci[s] = p;
    });
  if (h && a.clear_hint) clear_hint(h);  // consumed: cleared for the next call
  if (M >= K && M <= TK_ROW_CAP)
    select_in_candidates(a, row, ck, M, K, b, hist, red, res, [&](int i) { return ci[i]; });
  else
    select_row_from_memory(a, row, V, K, hist, red, res);
}

// ----------------------------------------------------------------------------
// Longer rows: per-chunk candidates, the row's last workgroup selects
// ----------------------------------------------------------------------------
// Zeroes the hint and the arrival counters of every row (top-k without a
// histogram from the scan).
__global__ void __launch_bounds__(TK_NT) topk_clear_kernel(uint32_t* hint, uint32_t* ctr, int rows) {
  clear_hint(hint + (int64_t)blockIdx.x * TK_BINS);
  if (threadIdx.x == 0) ctr[blockIdx.x] = 0u;
  (void)rows;
}

// Digit histogram of chunk blockIdx.x (16 TK_NT keys) of row blockIdx.y, added
// to the row's histogram (integer atomics: the sums do not depend on order).
__global__ void __launch_bounds__(TK_NT) topk_hist_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[TK_BINS];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int V = (int)visible_of(a, row);
  const int lo = blockIdx.x * (16 * TK_NT);
  if (lo >= V) return;
  const int hi = min(V, lo + 16 * TK_NT);
  for (int i = t; i < TK_BINS; i += TK_NT) hist[i] = 0;
  RegKeys<16> rk;
  rk.load(a.scores + row * a.N_max, lo, hi);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (rk.pos(lo, j, e) < hi) atomicAdd(&hist[rk.k[4 * j + e] >> TK_DSHIFT], 1u);
  __syncthreads();
  uint32_t* g = a.hint + row * TK_BINS;
  for (int i = t; i < TK_BINS; i += TK_NT)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// Chunk blockIdx.x (TK_FCH keys) of row blockIdx.y. Each wave compacts the
// candidates of its 1024-key segment -- keys whose digit is at least the
// threshold bin of the row's histogram hint; every chunk reads the same hint,
// so all agree on the bin -- into its own list, in position order (a ballot
// prefix inside the wave; no workgroup barrier). The workgroup that arrives
// last at the row's counter then gathers every list in segment order and
// selects the row. Rows with K = V are written by chunk 0.
__host__ __device__ constexpr int seg_words(int nseg) { return (nseg + 8 + 3) & ~3; }

// The lists and counts the chunks hand to the row's last workgroup travel by
// device-coherent accesses (relaxed device-scope atomics: the per-XCD L2
// caches are not coherent with each other, and these loads and stores bypass
// them), so the hand-over needs no L2 write-back or invalidation: a chunk
// waits for its own stores to complete before it counts its arrival.
template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(TK_NT) topk_chunk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* hist = smem;                                      // TK_BINS
  int* red = reinterpret_cast<int*>(smem + TK_BINS);          // 2 TK_NW
  int* res = red + 2 * TK_NW;                                 // 4, then the last-arrival flag (+ pad)
  int* off = res + 8;                                         // nseg segment offsets (+ pad)
  uint32_t* ck = reinterpret_cast<uint32_t*>(off + seg_words(a.nseg));  // cap keys
  int32_t* ci = reinterpret_cast<int32_t*>(ck + a.cap);              // and positions
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const int V = (int)visible_of(a, row);
  const int K = min(a.top_k, V);
  uint32_t* h = a.hint + row * TK_BINS;
  if (K == V) {
    if (c == 0) {
      emit_all_visible(a, row, V);
      if (a.clear_hint) clear_hint(h);
    }
    return;
  }
  const int lo = c * TK_FCH;
  if (lo >= V) return;  // chunks past V hold no key and do not arrive
  const int hi = min(V, lo + TK_FCH);
  const int nch = (V + TK_FCH - 1) / TK_FCH;  // chunks that arrive
  RegKeys<TK_FCH / TK_NT> rk;
  rk.load(a.scores + row * a.N_max, lo, hi);
  load_hint(h, hist);
  if (t == 0) res[0] = -1;
  __syncthreads();
  find_bin_block(hist, K, red, res);
  const int b = res[0];
  // this wave's segment: ordered compaction into its list
  {
    constexpr int KPT = TK_FCH / TK_NT;
    const int seg = c * TK_NW + wv;
    const int64_t lb = (row * a.nseg + seg) * (int64_t)TK_WCAP;
    int run = 0;
#pragma unroll
    for (int j = 0; j < KPT / 4; ++j) {
      bool cand[4];
      int n = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cand[e] = b >= 0 && rk.pos(lo, j, e) < hi && (rk.k[4 * j + e] >> TK_DSHIFT) >= (uint32_t)b;
        n += cand[e];
      }
      int st;
      int s = run + excl3(n, st);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (cand[e]) {
          if (s < TK_WCAP) {
            st_dev(&a.wkey[lb + s], rk.k[4 * j + e]);
            st_dev(&a.widx[lb + s], (int32_t)rk.pos(lo, j, e));
          }
          ++s;
        }
      run += st;
    }
    if (l == 0) st_dev(&a.wcnt[row * a.nseg + seg], b < 0 ? TK_WCAP + 1 : min(run, TK_WCAP + 1));
  }
  // arrival: every store of this chunk has completed, then it counts
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (t == 0)
    res[4] = __hip_atomic_fetch_add(&a.ctr[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(nch - 1);
  __syncthreads();
  if (!res[4]) return;
  // ---- last workgroup of the row: segment offsets, gather, select
  const int nseg = (V + TK_SEG - 1) / TK_SEG;
  int M = -1;
  {
    const int32_t* cnt = a.wcnt + row * a.nseg;
    int base = 0, ovf = 0;
    for (int s0 = 0; s0 < nseg; s0 += TK_NT) {
      const int v = s0 + t < nseg ? ld_dev(&cnt[s0 + t]) : 0;
      ovf |= v > TK_WCAP;
      const int vc = min(v, TK_WCAP);
      const int inc = wave_incl_scan_dpp(vc);
      if (l == 63) red[wv] = inc;
      __syncthreads();
      int wb = 0, tot = 0;
#pragma unroll
      for (int u = 0; u < TK_NW; ++u) {
        wb += u < wv ? red[u] : 0;
        tot += red[u];
      }
      if (s0 + t < nseg) off[s0 + t] = base + wb + inc - vc;
      base += tot;
      __syncthreads();
    }
    ovf = block_sum(ovf, red);
    M = ovf ? -1 : base;
  }
  if (M >= K && M <= a.cap) {
    // gather: P threads per segment, each copying every P-th candidate (up to
    // 16 loads in flight per thread)
    const int P = nseg >= TK_NT ? 1 : TK_NT / nseg;
    for (int s0 = 0; s0 < nseg; s0 += TK_NT / P) {
      const int sg = s0 + t / P, sub = t % P;
      if (sg < nseg) {
        const int n = min(ld_dev(&a.wcnt[row * a.nseg + sg]), TK_WCAP), o = off[sg];
        const int64_t lb = (row * a.nseg + sg) * (int64_t)TK_WCAP;
        for (int j0 = sub; j0 < n; j0 += 16 * P) {
          uint32_t kv[16];
          int32_t iv[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int j = j0 + u * P;
            if (j < n) {
              kv[u] = ld_dev(&a.wkey[lb + j]);
              iv[u] = ld_dev(&a.widx[lb + j]);
            }
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int j = j0 + u * P;
            if (j < n) {
              ck[o + j] = kv[u];
              ci[o + j] = iv[u];
            }
          }
        }
      }
    }
    __syncthreads();
    select_in_candidates(a, row, ck, M, K, b, hist, red, res, [&](int i) { return ci[i]; });
  } else {
    select_row_from_memory(a, row, V, K, hist, red, res);
  }
  if (a.clear_hint) clear_hint(h);  // consumed: cleared for the next call
  if (t == 0) a.ctr[row] = 0u;
}

static size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

static bool long_rows(int64_t N_max) { return N_max > TK_ROW_MAX; }
bool topk_long_rows(int64_t N_max) { return long_rows(N_max); }

static int64_t wave_segments(int64_t N_max) { return (N_max + TK_FCH - 1) / TK_FCH * TK_NW; }

// Workspace: hint [rows, TK_BINS] (rows of a histogram-carrying call, or
// long rows) | long rows: ctr [rows] | wcnt [rows, nseg] | wkey, widx [rows,
// nseg, TK_WCAP]
size_t topk_hint_bytes(int64_t rows, int64_t N_max, bool from_scan) {
  return (from_scan || long_rows(N_max)) ? round256((size_t)rows * TK_BINS * 4) : 0;
}

size_t topk_ws_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k, bool from_scan) {
  (void)top_k;
  const int64_t rows = B * Tq;
  if (rows <= 0) return 0;
  size_t n = topk_hint_bytes(rows, N_max, from_scan);
  if (long_rows(N_max)) {
    const int64_t nseg = wave_segments(N_max);
    n += round256((size_t)rows * 4) + round256((size_t)rows * nseg * 4) +
         2 * round256((size_t)rows * nseg * TK_WCAP * 4);
  }
  return n;
}

size_t topk_counter_offset(int64_t rows, int64_t N_max) {
  return long_rows(N_max) ? round256((size_t)rows * TK_BINS * 4) : 0;
}

constexpr int TK_MAX_DEVICES = 64;

hipError_t run_topk(const TopkLaunch& L, hipStream_t st) {
  const int64_t rows = L.B * L.Tq;
  if (rows == 0) return hipSuccess;
  TopkArgs a{};
  a.scores = L.scores;
  a.q_pos = L.q_pos;
  a.n_comp = L.n_comp;
  a.Tq = L.Tq;
  a.N_max = L.N_max;
  a.m = L.m;
  a.top_k = L.top_k;
  a.out_idx = L.idx;
  a.out_score = L.out_score;
  uint8_t* w = reinterpret_cast<uint8_t*>(L.ws);
  const bool from_scan = L.hint_mode != TOPK_HINT_NONE;
  a.clear_hint = L.hint_mode == TOPK_HINT_ACCUMULATED;
  if (!long_rows(L.N_max)) {
    a.hint = from_scan ? reinterpret_cast<uint32_t*>(w) : nullptr;
    const dim3 grid((unsigned)rows);
    if (L.N_max <= 4096)
      hipLaunchKernelGGL(topk_row_kernel<16>, grid, dim3(TK_NT), 0, st, a);
    else
      hipLaunchKernelGGL(topk_row_kernel<64>, grid, dim3(TK_NT), 0, st, a);
    return hipGetLastError();
  }
  const int64_t nseg = wave_segments(L.N_max);
  // candidates the last workgroup of a row can hold: about 8 top-k, at least
  // 4096, at most 16384 and what the LDS leaves beside the segment offsets; a
  // row with more falls back to memory
  const size_t fixed = (size_t)(TK_BINS + 2 * TK_NW + 8 + seg_words((int)nseg)) * 4;
  int cap = (int)std::min<int64_t>(16384, std::max<int64_t>(4096, 8 * (int64_t)L.top_k));
  while (fixed + (size_t)cap * 8 > (size_t)TK_LDS_MAX) cap -= 1024;
  const size_t lds = fixed + (size_t)cap * 8;
  // the LDS opt-in is a per-device function attribute: set once per device
  // (setting it twice is harmless, so concurrent first calls need no lock)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= TK_MAX_DEVICES) return hipErrorInvalidDevice;
  static bool attr_set_dev[TK_MAX_DEVICES] = {};
  if (!attr_set_dev[dev]) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_chunk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       TK_LDS_MAX);
    if (e != hipSuccess) return e;
    attr_set_dev[dev] = true;
  }
  a.hint = reinterpret_cast<uint32_t*>(w);
  w += round256((size_t)rows * TK_BINS * 4);
  a.ctr = reinterpret_cast<uint32_t*>(w);
  w += round256((size_t)rows * 4);
  a.wcnt = reinterpret_cast<int32_t*>(w);
  w += round256((size_t)rows * nseg * 4);
  a.wkey = reinterpret_cast<uint32_t*>(w);
  w += round256((size_t)rows * nseg * TK_WCAP * 4);
  a.widx = reinterpret_cast<int32_t*>(w);
  a.nseg = (int)nseg;
  a.cap = cap;
  if (!from_scan) {
    // no histogram from a scan: build it here (the counters start at zero too)
    a.clear_hint = 0;
    hipLaunchKernelGGL(topk_clear_kernel, dim3((unsigned)rows), dim3(TK_NT), 0, st, a.hint, a.ctr, (int)rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned nh = (unsigned)((L.N_max + 16 * TK_NT - 1) / (16 * TK_NT));
    hipLaunchKernelGGL(topk_hist_kernel, dim3(nh, (unsigned)rows), dim3(TK_NT), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)(nseg / TK_NW), (unsigned)rows), dim3(TK_NT), lds, st, a);
  return hipGetLastError();
}

}  // namespace csa
