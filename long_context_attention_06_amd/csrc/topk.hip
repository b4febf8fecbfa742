// Exact top-k selection over indexer scores, for gfx950.
//
// What is computed (DeepSeek V4 脱离 CUDA 全栈国产化, deepseek.csdn.net,
// section 二, CSA step 2: keep the top-k compressed blocks, 512 for Flash and
// 1024 for Pro): for a query row with V visible scores, the K = min(k, V)
// entries with the largest scores; equal scores go to the lower index, so the
// set is unique. Indices are written in ascending order, the row padded with
// -1. Batch invariance (DeepTech wiki, batch-invariance note) follows from the
// algorithm: selection is exact, so the output depends on the row alone.
//
// Algorithm. A 1024-thread workgroup owns one chunk of up to 32768 keys of a
// row, cached in LDS as order-preserving uint32 keys. A radix select with
// integer LDS histograms finds the exact chunk-local K-th key T: digits of up
// to 11 bits taken below the common prefix of the chunk's smallest and largest
// key (at most three passes); each digit is chosen by one wave that holds the
// bin counts in registers and scans them from the top. The chunk is then compacted in index order (per-wave
// counts, a scan over waves, ballot prefix sums): all keys > T and the
// lowest-index ties == T. A row that fits one chunk is finished in one launch.
// A longer row writes each chunk's top K (key, index) pairs, in index order;
// the union of the chunk winners contains the row's top K (an entry beaten by
// K others inside its chunk is beaten by them in the row, ties included), so
// the next launch selects again among the candidates, and repeats until one
// chunk remains. No cross-workgroup atomics, no memory to clear.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int TK_NT = 1024;
constexpr int TK_NW = TK_NT / 64;
constexpr int TK_BINS = 2048;
constexpr int TK_CHUNK_S = 32768;  // max scores per workgroup (128 KiB of LDS)
constexpr int TK_CHUNK_C = 16384;  // max candidates per workgroup (keys + indices, 128 KiB)
constexpr int TK_CHUNK_MIN = 4096;
constexpr int TK_TARGET_WG = 256;  // workgroups a launch should offer (one per CU)
enum { TK_SCORES = 0, TK_CANDS = 1 };

__device__ __forceinline__ float key_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Given the counts of the TK_BINS bins, find the bin b with (count above b) <
// need <= (count of bins >= b). All threads take part: wave w scans bins
// [TK_BINS - 128 (w+1), TK_BINS - 128 w) from the top, two per lane (one
// inclusive scan over lanes), the waves' totals meet in tot[0..TK_NW), and
// the lane holding the threshold publishes out[0] = b, out[1] = count above b,
// out[2] = count of b. Ends with a barrier that publishes out[] and frees hist
// and tot.
__device__ __forceinline__ void find_bin_block(const uint32_t* hist, int need, int* tot, int* out) {
  static_assert(TK_BINS == 128 * TK_NW, "two bins per lane");
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int hi = TK_BINS - 128 * wv - 2 * l - 1;  // this lane's upper bin; the lower one is hi - 1
  const u32x2_t c2 = *reinterpret_cast<const u32x2_t*>(hist + hi - 1);
  const int chi = (int)c2[1], clo = (int)c2[0], own = chi + clo;
  const int inc = wave_incl_scan_dpp(own);
  if (l == 63) tot[wv] = inc;
  __syncthreads();
  int above = inc - own;  // bins above this lane's, within the wave
#pragma unroll
  for (int q = 0; q < TK_NW / 4; ++q) {
    const u32x4_t t4 = *reinterpret_cast<const u32x4_t*>(tot + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) above += 4 * q + e < wv ? (int)t4[e] : 0;
  }
  if (above < need && need <= above + own) {
    const bool upper = need <= above + chi;
    out[0] = upper ? hi : hi - 1;
    out[1] = upper ? above : above + chi;
    out[2] = upper ? chi : clo;
  }
  __syncthreads();
}

struct TopkArgs {
  const float* scores;     // TK_SCORES: [rows, N_max]
  const uint32_t* ckey;    // TK_CANDS: [rows, n_cand]
  const int32_t* cidx;
  const int32_t* q_pos;
  const int32_t* n_comp;
  int64_t Tq, N_max, n_cand;
  int m, top_k;
  int chunk;               // keys per workgroup at this level
  int32_t* out_idx;        // final: [rows, top_k]
  float* out_score;        // final, nullable
  uint32_t* nkey;          // next level: [rows, nchunk, top_k]
  int32_t* nidx;
  // threshold path: per-row threshold key, per-chunk candidates and counts
  uint32_t* thr;           // [rows]
  uint32_t* fkey;          // [rows, nfch * TK_FCH]
  int32_t* fidx;
  int32_t* fcnt;           // [rows, nfch]
  int nfch;
};

constexpr int TK_FCH = 4096;     // keys per workgroup of the filter
constexpr int TK_SAMPLE = 4096;  // scores sampled per row for the threshold
constexpr int TK_FCH_MAX = 1024; // filter chunks per row the final kernel can gather

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
// histogram spreads over the keys' own range (a fixed top digit puts scores of
// similar magnitude into a few bins, and the LDS atomics of a pass then
// serialise on them).
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
    // four 16-byte reads in flight per thread before their atomics
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
      // another pass: find_bin_block's closing barrier freed the histogram
      // (one buffer keeps the LDS of a 16K-key chunk small enough for two
      // workgroups per CU)
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
    for (int q = 0; q < TK_NW / 4; ++q) {
      const u32x4_t g4 = *reinterpret_cast<const u32x4_t*>(red + 4 * q);
      const u32x4_t e4 = *reinterpret_cast<const u32x4_t*>(red + TK_NW + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gs[4 * q + e] = (int)g4[e];
        es[4 * q + e] = (int)e4[e];
      }
    }
#pragma unroll
    for (int u = 0; u < TK_NW; ++u) {
      const bool before = u < wv;
      sel_before += before ? gs[u] + (all ? 0 : max(0, min(need - eq_before, es[u]))) : 0;
      eq_before += before ? es[u] : 0;
    }
  }
  // popcount of the mask's bits below this lane (v_mbcnt_lo/hi)
  auto below_cnt = [](uint64_t msk) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
  };
  auto excl3 = [&](int v, int& total) {  // wave exclusive prefix and total of v in 0..7
    const uint64_t b0 = __ballot(v & 1), b1 = __ballot(v & 2), b2 = __ballot(v & 4);
    total = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
    return below_cnt(b0) + 2 * below_cnt(b1) + 4 * below_cnt(b2);
  };
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
}

template <int SRC>
__global__ void __launch_bounds__(TK_NT) topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* hist = smem;                                   // TK_BINS
  int* red = reinterpret_cast<int*>(smem + TK_BINS);       // 32
  int* res = red + 32;                                     // 32
  const int CH = a.chunk;
  uint32_t* kc = smem + TK_BINS + 64;                      // CH keys
  int32_t* ic = reinterpret_cast<int32_t*>(kc + CH);       // TK_CANDS: indices

  const int t = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x, nchunk = gridDim.x;
  const int64_t n_row = SRC == TK_SCORES ? visible_of(a, row) : a.n_cand;
  const int64_t lo = (int64_t)c * CH;
  const int n = (int)max((int64_t)0, min(n_row - lo, (int64_t)CH));
  const int top_k = a.top_k;
  const int K = min(top_k, n);
  const bool final_out = nchunk == 1;

  // ---- load the chunk: keys (and candidate indices) into LDS
  if constexpr (SRC == TK_SCORES) {
    const float* src = a.scores + row * a.N_max + lo;
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
      const int n4 = n >> 2;
      const f32x4_t* s4 = reinterpret_cast<const f32x4_t*>(src);
      for (int i0 = t; i0 < n4; i0 += TK_NT * 4) {
        f32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (i0 + u * TK_NT < n4) v[u] = s4[i0 + u * TK_NT];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * TK_NT;
          if (i < n4)
            *reinterpret_cast<u32x4_t*>(kc + 4 * i) =
                u32x4_t{f32_key(v[u][0]), f32_key(v[u][1]), f32_key(v[u][2]), f32_key(v[u][3])};
        }
      }
      for (int i = 4 * n4 + t; i < n; i += TK_NT) kc[i] = f32_key(src[i]);
    } else {
      for (int i = t; i < n; i += TK_NT) kc[i] = f32_key(src[i]);
    }
  } else {
    const uint32_t* ks = a.ckey + row * a.n_cand + lo;
    const int32_t* is = a.cidx + row * a.n_cand + lo;
    if (((reinterpret_cast<uintptr_t>(ks) | reinterpret_cast<uintptr_t>(is)) & 15) == 0) {
      const int n4 = n >> 2;
      for (int i0 = t; i0 < n4; i0 += TK_NT * 2) {
        u32x4_t kv[2], iv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (i0 + u * TK_NT < n4) {
            kv[u] = reinterpret_cast<const u32x4_t*>(ks)[i0 + u * TK_NT];
            iv[u] = reinterpret_cast<const u32x4_t*>(is)[i0 + u * TK_NT];
          }
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (i0 + u * TK_NT < n4) {
            reinterpret_cast<u32x4_t*>(kc)[i0 + u * TK_NT] = kv[u];
            reinterpret_cast<u32x4_t*>(ic)[i0 + u * TK_NT] = iv[u];
          }
      }
      for (int i = 4 * n4 + t; i < n; i += TK_NT) {
        kc[i] = ks[i];
        ic[i] = is[i];
      }
    } else {
      for (int i = t; i < n; i += TK_NT) {
        kc[i] = ks[i];
        ic[i] = is[i];
      }
    }
  }
  __syncthreads();  // publish the key cache

  const LdsKeys keys{kc};
  uint32_t T = 0;
  int need = 0;
  const bool all = K == n;
  if (!all) block_select(keys, n, K, hist, red, res, T, need);
  const int64_t obase = final_out ? row * (int64_t)top_k : (row * nchunk + c) * (int64_t)top_k;
  auto emit = [&](int pos, uint32_t key, int i) {
    const int32_t gi = SRC == TK_SCORES ? (int32_t)(lo + i) : ic[i];
    if (final_out) {
      a.out_idx[obase + pos] = gi;
      if (a.out_score) a.out_score[obase + pos] = key_f32(key);
    } else {
      a.nkey[obase + pos] = key;
      a.nidx[obase + pos] = gi;
    }
  };
  auto pad = [&](int i) {
    if (final_out) {
      a.out_idx[obase + i] = -1;
      if (a.out_score) a.out_score[obase + i] = -INFINITY;
    } else {
      a.nkey[obase + i] = 0u;  // below every finite key: never selected later
      a.nidx[obase + i] = -1;
    }
  };
  block_compact(keys, n, K, all, T, need, top_k, red, emit, pad);
}

// ----------------------------------------------------------------------------
// Threshold path for long rows (one sample select, one filter, one select)
// ----------------------------------------------------------------------------
// 1. topk_threshold_kernel: per row, the exact r-th largest key T_s of an
//    evenly spaced sample of TK_SAMPLE scores, r chosen so that about 2 K of
//    the row's scores lie at or above it. Rows that fit the final kernel take
//    T_s = 0 (every key).
// 2. topk_filter_kernel: per 4096-key chunk, the keys >= T_s with their
//    positions, compacted in position order, and their count.
// 3. topk_filtered_kernel: per row, the chunks' candidates gathered in chunk
//    order (so in position order) and selected exactly. If the sample misled
//    (fewer than K' candidates, or more than fit in LDS), it selects over the
//    whole row read from memory instead. Either way the result is the exact
//    top K'.
__global__ void __launch_bounds__(TK_NT) topk_threshold_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[TK_BINS];
  __shared__ __attribute__((aligned(16))) int red[32], res[32];
  __shared__ __attribute__((aligned(16))) uint32_t kc[TK_SAMPLE];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t V = visible_of(a, row);
  if (V <= TK_CHUNK_C) {
    if (t == 0) a.thr[row] = 0u;
    return;
  }
  const int K = min((int64_t)a.top_k, V);
  const float* src = a.scores + row * a.N_max;
  for (int i = t; i < TK_SAMPLE; i += TK_NT) kc[i] = f32_key(src[(int64_t)i * V / TK_SAMPLE]);
  __syncthreads();
  const int r = (int)min((int64_t)(TK_SAMPLE - 1), (2 * (int64_t)K * TK_SAMPLE + V - 1) / V + 8);
  uint32_t T;
  int need;
  block_select(LdsKeys{kc}, TK_SAMPLE, r, hist, red, res, T, need);
  if (t == 0) a.thr[row] = T;
}

__global__ void __launch_bounds__(TK_NT) topk_filter_kernel(TopkArgs a) {
  __shared__ int wtot[TK_NW];
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const int64_t V = visible_of(a, row);
  const int64_t lo = (int64_t)c * TK_FCH;
  const int n = (int)max((int64_t)0, min(V - lo, (int64_t)TK_FCH));
  const uint32_t thr = a.thr[row];
  const float* src = a.scores + row * a.N_max + lo;
  const int p = 4 * t;
  u32x4_t k4;
  if ((reinterpret_cast<uintptr_t>(src) & 15) == 0 && p + 3 < n) {
    const f32x4_t v = reinterpret_cast<const f32x4_t*>(src)[t];
    k4 = u32x4_t{f32_key(v[0]), f32_key(v[1]), f32_key(v[2]), f32_key(v[3])};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) k4[e] = p + e < n ? f32_key(src[p + e]) : 0u;
  }
  bool sel[4];
  int ns = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sel[e] = p + e < n && k4[e] >= thr;
    ns += sel[e];
  }
  auto below_cnt = [](uint64_t msk) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
  };
  const uint64_t b0 = __ballot(ns & 1), b1 = __ballot(ns & 2), b2 = __ballot(ns & 4);
  const int wsum = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
  int pos = below_cnt(b0) + 2 * below_cnt(b1) + 4 * below_cnt(b2);
  if (l == 0) wtot[wv] = wsum;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int u = 0; u < TK_NW; ++u) {
    const int v = wtot[u];
    pos += u < wv ? v : 0;
    total += v;
  }
  const int64_t obase = row * (int64_t)a.nfch * TK_FCH + lo;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (sel[e]) {
      a.fkey[obase + pos] = k4[e];
      a.fidx[obase + pos] = (int32_t)(lo + p + e);
      ++pos;
    }
  if (t == 0) a.fcnt[row * a.nfch + c] = total;
}

__global__ void __launch_bounds__(TK_NT) topk_filtered_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* hist = smem;                                   // TK_BINS
  int* red = reinterpret_cast<int*>(smem + TK_BINS);       // 32
  int* res = red + 32;                                     // 32
  int* off = res + 32;                                     // TK_FCH_MAX chunk offsets, then the total
  uint32_t* kc = reinterpret_cast<uint32_t*>(off + TK_FCH_MAX + 64);  // TK_CHUNK_C keys
  int32_t* ic = reinterpret_cast<int32_t*>(kc + TK_CHUNK_C);          // and positions
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int64_t row = blockIdx.x;
  const int64_t V = visible_of(a, row);
  const int top_k = a.top_k;
  const int K = (int)min((int64_t)top_k, V);
  const int nfch = a.nfch;
  const int32_t* cnt = a.fcnt + row * nfch;

  // chunk offsets in chunk order (wave 0: a lane sums a contiguous run of chunks)
  if (wv == 0) {
    const int per = (nfch + 63) / 64;
    const int c0 = min(nfch, l * per), c1 = min(nfch, c0 + per);
    int s = 0;
    for (int c = c0; c < c1; ++c) s += cnt[c];
    int run = wave_incl_scan_dpp(s) - s;
    for (int c = c0; c < c1; ++c) {
      off[c] = run;
      run += cnt[c];
    }
    if (l == 63) off[TK_FCH_MAX] = run;
  }
  __syncthreads();
  const int total = off[TK_FCH_MAX];
  const int64_t obase = row * (int64_t)top_k;
  auto emit_to = [&](auto idx_of) {
    return [&, idx_of](int pos, uint32_t key, int i) {
      a.out_idx[obase + pos] = idx_of(i);
      if (a.out_score) a.out_score[obase + pos] = key_f32(key);
    };
  };
  auto pad = [&](int i) {
    a.out_idx[obase + i] = -1;
    if (a.out_score) a.out_score[obase + i] = -INFINITY;
  };
  if (total >= K && total <= TK_CHUNK_C) {
    // gather: wave wv copies chunks wv, wv + 16, ... to their offsets
    const uint32_t* fk = a.fkey + row * (int64_t)nfch * TK_FCH;
    const int32_t* fi = a.fidx + row * (int64_t)nfch * TK_FCH;
    for (int c = wv; c < nfch; c += TK_NW) {
      const int nc = cnt[c], o = off[c];
      for (int j = l; j < nc; j += 64) {
        kc[o + j] = fk[(int64_t)c * TK_FCH + j];
        ic[o + j] = fi[(int64_t)c * TK_FCH + j];
      }
    }
    __syncthreads();
    const LdsKeys keys{kc};
    uint32_t T = 0;
    int need = 0;
    const bool all = K == total;
    if (!all) block_select(keys, total, K, hist, red, res, T, need);
    block_compact(keys, total, K, all, T, need, top_k, red, emit_to([&](int i) { return ic[i]; }), pad);
  } else {
    const float* src = a.scores + row * a.N_max;
    const RowKeys keys{src, (int)V, (reinterpret_cast<uintptr_t>(src) & 15) == 0};
    uint32_t T = 0;
    int need = 0;
    const bool all = K == (int)V;
    if (!all) block_select(keys, (int)V, K, hist, red, res, T, need);
    block_compact(keys, (int)V, K, all, T, need, top_k, red, emit_to([](int i) { return (int32_t)i; }), pad);
  }
}

static int64_t pow2_at_least(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Level plan for rows of length n0: per launch, keys per workgroup (chunk),
// chunks per row and the row length it reads. Chunks are sized so a launch
// offers about one workgroup per CU (a lone workgroup is VALU bound), never
// below 4096 keys or 4*top_k (each level must shrink the rows), never above
// what fits in LDS, and never above the row itself (rounded up to 256 keys):
// LDS is sized by the chunk, and rows of up to 18K keys then leave room for
// two workgroups per CU. Depends on shape arguments only.
static int plan_levels(int64_t rows, int64_t n0, int top_k, int64_t* nch, int64_t* nlen, int64_t* chunk) {
  int lv = 0;
  int64_t n = n0;
  while (true) {
    const int64_t cmax = lv == 0 ? TK_CHUNK_S : TK_CHUNK_C;
    const int64_t want = pow2_at_least((rows * n + TK_TARGET_WG - 1) / TK_TARGET_WG);
    const int64_t ch = std::min({cmax, (n + 255) / 256 * 256,
                                 std::max<int64_t>({want, (int64_t)TK_CHUNK_MIN, pow2_at_least(4 * (int64_t)top_k)})});
    chunk[lv] = ch;
    nch[lv] = std::max<int64_t>(1, (n + ch - 1) / ch);
    nlen[lv] = n;
    ++lv;
    if (nch[lv - 1] == 1 || lv == 12) break;
    n = nch[lv - 1] * top_k;
  }
  return lv;
}

// Long rows (three or more levels) take the threshold path when its final
// kernel can gather every filter chunk. Depends on shape arguments only.
static bool use_threshold_path(int64_t rows, int64_t N_max, int top_k) {
  int64_t nch[12], nlen[12], chunk[12];
  const int lv = plan_levels(rows, N_max, top_k, nch, nlen, chunk);
  const int64_t nfch = (N_max + TK_FCH - 1) / TK_FCH;
  return lv >= 3 && nfch <= TK_FCH_MAX && top_k <= TK_CHUNK_C / 8;
}

static size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// threshold path workspace: thr [rows] | fcnt [rows, nfch] | fkey, fidx [rows, nfch * TK_FCH]
static size_t threshold_ws(int64_t rows, int64_t N_max) {
  const int64_t nfch = (N_max + TK_FCH - 1) / TK_FCH;
  return round256(rows * 4) + round256(rows * nfch * 4) + 2 * round256((size_t)rows * nfch * TK_FCH * 4);
}

size_t topk_ws_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k) {
  if (use_threshold_path(B * Tq, N_max, top_k)) return threshold_ws(B * Tq, N_max);
  int64_t nch[12], nlen[12], chunk[12];
  const int lv = plan_levels(B * Tq, N_max, top_k, nch, nlen, chunk);
  size_t mx = 0;
  for (int i = 0; i + 1 < lv; ++i) mx = std::max(mx, (size_t)(B * Tq) * nch[i] * top_k * 8);
  return mx == 0 ? 0 : 2 * ((mx + 255) & ~size_t(255));
}

constexpr int TK_MAX_DEVICES = 64;

hipError_t run_topk(const TopkLaunch& L, hipStream_t st) {
  const int64_t rows = L.B * L.Tq;
  if (rows == 0) return hipSuccess;
  // the LDS opt-in is a per-device function attribute: set once per device
  // (setting it twice is harmless, so concurrent first calls need no lock)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= TK_MAX_DEVICES) return hipErrorInvalidDevice;
  static bool attr_set_dev[TK_MAX_DEVICES] = {};
  static bool attr_f_dev[TK_MAX_DEVICES] = {};
  bool& attr_set = attr_set_dev[dev];
  const size_t lds_s = (size_t)(TK_BINS + 64 + TK_CHUNK_S) * 4;
  const size_t lds_c = (size_t)(TK_BINS + 64 + 2 * TK_CHUNK_C) * 4;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<TK_SCORES>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_s);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)topk_kernel<TK_CANDS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_c);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (use_threshold_path(rows, L.N_max, L.top_k)) {
    const size_t lds_f = (size_t)(TK_BINS + 64 + TK_FCH_MAX + 64 + 2 * TK_CHUNK_C) * 4;
    bool& attr_f = attr_f_dev[dev];
    if (!attr_f) {
      hipError_t e = hipFuncSetAttribute((const void*)topk_filtered_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_f);
      if (e != hipSuccess) return e;
      attr_f = true;
    }
    const int64_t nfch = (L.N_max + TK_FCH - 1) / TK_FCH;
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
    a.nfch = (int)nfch;
    uint8_t* w = reinterpret_cast<uint8_t*>(L.ws);
    a.thr = reinterpret_cast<uint32_t*>(w);
    w += round256(rows * 4);
    a.fcnt = reinterpret_cast<int32_t*>(w);
    w += round256(rows * nfch * 4);
    a.fkey = reinterpret_cast<uint32_t*>(w);
    w += round256((size_t)rows * nfch * TK_FCH * 4);
    a.fidx = reinterpret_cast<int32_t*>(w);
    hipLaunchKernelGGL(topk_threshold_kernel, dim3((unsigned)rows), dim3(TK_NT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)nfch, (unsigned)rows), dim3(TK_NT), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_filtered_kernel, dim3((unsigned)rows), dim3(TK_NT), lds_f, st, a);
    return hipGetLastError();
  }
  int64_t nch[12], nlen[12], chunk[12];
  const int lv = plan_levels(rows, L.N_max, L.top_k, nch, nlen, chunk);
  size_t half = 0;
  if (lv > 1) half = L.ws_bytes / 2;
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
  for (int i = 0; i < lv; ++i) {
    const bool last = i + 1 == lv;
    uint8_t* cur = reinterpret_cast<uint8_t*>(L.ws) + (i & 1) * half;  // written by level i
    if (!last) {
      const size_t nk = (size_t)rows * nch[i] * L.top_k;
      a.nkey = reinterpret_cast<uint32_t*>(cur);
      a.nidx = reinterpret_cast<int32_t*>(cur + nk * 4);
    }
    dim3 grid((unsigned)nch[i], (unsigned)rows);
    a.chunk = (int)chunk[i];
    if (i == 0) {
      hipLaunchKernelGGL(topk_kernel<TK_SCORES>, grid, dim3(TK_NT), (TK_BINS + 64 + chunk[i]) * 4, st, a);
    } else {
      hipLaunchKernelGGL(topk_kernel<TK_CANDS>, grid, dim3(TK_NT), (TK_BINS + 64 + 2 * chunk[i]) * 4, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!last) {  // the candidates become the next level's input
      a.ckey = a.nkey;
      a.cidx = a.nidx;
      a.n_cand = nch[i] * L.top_k;
    }
  }
  return hipSuccess;
}

}  // namespace csa
