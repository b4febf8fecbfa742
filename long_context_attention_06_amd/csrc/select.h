// Exact selection helpers for gfx950 workgroups of NT threads: the pieces
// the top-k kernels and the fused decode kernel share.
//
// Scores become order-preserving uint32 keys (f32_key). The top 11 bits of a
// key are its digit (sign, exponent, two mantissa bits: four bins per
// binade). A digit histogram names the bin holding the K-th key; the keys of
// that bin and above are the candidates; an exact radix select among them
// finds the K-th key T and how many keys equal to T are kept (the
// lowest-position ones, so equal scores go to the lower index); an ordered
// compaction (ballot prefix sums) writes the selection in position order.
#pragma once
#include "common.h"

namespace csa {
namespace sel {

constexpr int BINS = 2048;
constexpr int DSHIFT = 21;                       // digit = key >> 21 (11 bits)
constexpr uint32_t HINT_CLAMP = (1u << 20) - 1;  // keeps any sum of bins inside int32

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

// Given the counts of the BINS bins, find the bin b with (count above b) <
// need <= (count of bins >= b). All NT threads take part: lane l of wave w
// holds the BINS / NT bins just below BINS - (BINS / NT) (64 w + l) (one
// inclusive scan over lanes of their sums), the waves' totals meet in
// tot[0..NT/64), and the lane holding the threshold publishes out[0] = b,
// out[1] = count above b, out[2] = count of b. If no bin qualifies (the counts
// sum to less than need) out[] is left as it was. Ends with a barrier that
// publishes out[] and frees hist and tot.
template <int NT>
__device__ __forceinline__ void find_bin_block(const uint32_t* hist, int need, int* tot, int* out) {
  constexpr int BPL = BINS / NT, NW = NT / 64;
  static_assert(BPL == 2 || BPL % 4 == 0, "bins per lane");
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int lo = BINS - BPL * (t + 1);  // this lane's lowest bin; its bins are lo .. lo + BPL - 1
  uint32_t c[BPL];
  if constexpr (BPL == 2) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(hist + lo);
    c[0] = v[0];
    c[1] = v[1];
  } else {
#pragma unroll
    for (int q = 0; q < BPL / 4; ++q) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(hist + lo + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) c[4 * q + e] = v[e];
    }
  }
  int own = 0;
#pragma unroll
  for (int i = 0; i < BPL; ++i) own += (int)c[i];
  const int inc = wave_incl_scan_dpp(own);
  if (l == 63) tot[wv] = inc;
  __syncthreads();
  int above = inc - own;  // bins above this lane's, within the wave
#pragma unroll
  for (int u = 0; u < NW; ++u) above += u < wv ? tot[u] : 0;
  if (above < need && need <= above + own) {
    int a = above, bin = lo, cb = (int)c[0];
    bool found = false;
#pragma unroll
    for (int i = BPL - 1; i >= 0; --i) {  // from the top bin down
      if (!found && need <= a + (int)c[i]) {
        found = true;
        bin = lo + i;
        cb = (int)c[i];
      } else if (!found) {
        a += (int)c[i];
      }
    }
    out[0] = bin;
    out[1] = a;
    out[2] = cb;
  }
  __syncthreads();
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
template <int NT, class KS>
__device__ void block_select(const KS& ks, int n, int K, uint32_t* hist, int* red, int* res, uint32_t& T,
                             int& need) {
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  need = K;
  const int n4 = n >> 2;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int i = t; i < n4; i += NT) {
    const u32x4_t k4 = ks.load4(i);
    kmin = min(min(kmin, k4[0]), min(k4[1], min(k4[2], k4[3])));
    kmax = max(max(kmax, k4[0]), max(k4[1], max(k4[2], k4[3])));
  }
  for (int i = 4 * n4 + t; i < n; i += NT) {
    const uint32_t k = ks.load1(i);
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
  kmin = wave_min_u32_dpp(kmin);
  kmax = wave_max_u32_dpp(kmax);
  if (l == 0) {
    red[wv] = (int)kmin;
    red[(NT / 64) + wv] = (int)kmax;
  }
  for (int i = t; i < BINS; i += NT) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < (NT / 64); ++u) {
    kmin = min(kmin, (uint32_t)red[u]);
    kmax = max(kmax, (uint32_t)red[(NT / 64) + u]);
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
    for (int i0 = t; i0 < n4; i0 += 4 * NT) {
      u32x4_t k4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) k4[u] = (i0 + u * NT < n4) ? ks.load4(i0 + u * NT) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (i0 + u * NT >= n4) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) add(k4[u][e]);
      }
    }
    for (int i = 4 * n4 + t; i < n; i += NT) add(ks.load1(i));
    __syncthreads();
    find_bin_block<NT>(h, need, red, res);
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
      for (int i = t; i < BINS; i += NT) h[i] = 0;
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
template <int NT, class KS, class Emit, class Pad>
__device__ void block_compact(const KS& ks, int n, int K, bool all, uint32_t T, int need, int top_k, int* red,
                              Emit emit, Pad pad) {
  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int seg = ((n + (NT / 64) - 1) / (NT / 64) + 255) / 256 * 256;
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
    red[(NT / 64) + wv] = eq;
  }
  __syncthreads();
  int eq_before = 0, sel_before = 0;
  {
    int gs[(NT / 64)], es[(NT / 64)];
#pragma unroll
    for (int u = 0; u < (NT / 64); ++u) {
      gs[u] = red[u];
      es[u] = red[(NT / 64) + u];
    }
#pragma unroll
    for (int u = 0; u < (NT / 64); ++u) {
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
  for (int i = K + t; i < top_k; i += NT) pad(i);
  __syncthreads();  // red[] is free again
}

// Keys held in registers by a NT-thread workgroup: KPT per thread. Wave w
// owns positions [lo + w*64*KPT, +64*KPT); in step j (KPT/4 steps) lane l
// holds the four positions base_j + 4 l + e, base_j = lo + w*64*KPT + 256 j.
template <int NT, int KPT>
struct RegKeys {
  static_assert(KPT % 4 == 0, "whole 16-byte steps");
  uint32_t k[KPT];
  __device__ __forceinline__ int pos(int lo, int j, int e) const {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    return lo + w * 64 * KPT + 256 * j + 4 * l + e;
  }
  // keys of positions [lo, hi) of src (hi - lo <= NT KPT); others read 0
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
// it; red holds (NT / 64) ints; ends with a barrier after red is read.
template <int NT, int KPT, class Put>
__device__ int reg_compact(const RegKeys<NT, KPT>& rk, int lo, int hi, uint32_t b, int cap, int* red, Put put) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  int pre[KPT / 4];
  int wtot = 0;
#pragma unroll
  for (int j = 0; j < KPT / 4; ++j) {
    int n = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) n += (rk.pos(lo, j, e) < hi) && (rk.k[4 * j + e] >> DSHIFT) >= b;
    int st;
    pre[j] = wtot + excl3(n, st);
    wtot += st;
  }
  if (l == 0) red[w] = wtot;
  __syncthreads();
  int off = 0, M = 0;
#pragma unroll
  for (int u = 0; u < (NT / 64); ++u) {
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
        if (p < hi && (rk.k[4 * j + e] >> DSHIFT) >= b) {
          put(s, rk.k[4 * j + e], p);
          ++s;
        }
      }
    }
  }
  __syncthreads();  // red[] is free again; the puts are done
  return M;
}

// Block sum of one int per thread (uniform result); red holds (NT / 64) ints.
template <int NT>
__device__ __forceinline__ int block_sum(int v, int* red) {
  v = wave_sum_dpp(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int u = 0; u < (NT / 64); ++u) s += red[u];
  __syncthreads();
  return s;
}

// Exact threshold among M candidates cached in LDS (keys ck, position order)
// that hold every key whose digit is at least b (M >= K): the K-th key T and
// how many keys equal to T the top K takes (the lowest-position ones). The
// threshold lies in digit b when fewer than K candidates have a larger digit;
// the next 11 bits of the keys of digit b then name its sub-bin, and (unless
// the sub-bin is taken whole) the last 10 bits the key itself: one or two
// histogram passes over the candidates. sub (nullable) holds the counts of
// digit-b keys by their next 11 bits already (summed by the caller's chunks):
// the first pass is skipped. Any inconsistency (a hint that did not hold)
// falls back to a full radix select over the candidates, which contain the
// top K either way. Returns false when all M candidates are taken (M == K).
template <int NT>
__device__ bool refine_threshold(const uint32_t* ck, int M, int K, int b, const uint32_t* sub, uint32_t* hist,
                                 int* red, int* res, uint32_t& T, int& need) {
  const int t = threadIdx.x;
  T = 0u;
  need = 0;
  if (M == K) return false;
  bool done = false;
  if (b >= 0) {
    int cnt_b = 0;
    if (sub) {
#pragma unroll
      for (int u = 0; u < BINS / NT; ++u) {
        const uint32_t v = min(sub[t + u * NT], HINT_CLAMP);
        hist[t + u * NT] = v;
        cnt_b += (int)v;
      }
      cnt_b = block_sum<NT>(cnt_b, red);  // its barriers also publish the histogram
    } else {
      for (int i = t; i < BINS; i += NT) hist[i] = 0;
      __syncthreads();
      for (int i = t; i < M; i += NT) {
        const uint32_t k = ck[i];
        if ((int)(k >> DSHIFT) == b) {
          atomicAdd(&hist[(k >> 10) & (BINS - 1)], 1u);
          ++cnt_b;
        }
      }
      cnt_b = block_sum<NT>(cnt_b, red);
    }
    const int need1 = K - (M - cnt_b);  // the candidates above digit b are all taken
    if (need1 > 0 && need1 <= cnt_b) {
      if (t == 0) res[0] = -1;
      __syncthreads();
      find_bin_block<NT>(hist, need1, red, res);
      const int s2 = res[0];
      const uint32_t P = ((uint32_t)b << 11) | (uint32_t)max(s2, 0);  // 22-bit key prefix
      if (s2 >= 0 && P > 0) {
        const int need2 = need1 - res[1];
        if (need2 == res[2]) {
          T = (P << 10) - 1u;  // the sub-bin is taken whole
          need = 0;
          done = true;
        } else {
          for (int i = t; i < BINS; i += NT) hist[i] = 0;
          __syncthreads();
          for (int i = t; i < M; i += NT) {
            const uint32_t k = ck[i];
            if ((k >> 10) == P) atomicAdd(&hist[k & 1023u], 1u);
          }
          if (t == 0) res[0] = -1;
          __syncthreads();
          find_bin_block<NT>(hist, need2, red, res);
          if (res[0] >= 0) {
            T = (P << 10) | (uint32_t)res[0];
            need = need2 - res[1];
            done = true;
          }
        }
      }
    }
  }
  if (!done) block_select<NT>(LdsKeys{ck}, M, K, hist, red, res, T, need);
  return true;
}

}  // namespace sel
}  // namespace csa
