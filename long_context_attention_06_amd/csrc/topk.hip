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
// Algorithm: one workgroup per row. Scores become order-preserving uint32
// keys. A three-digit radix select (11 + 11 + 10 bits) finds the exact K-th
// key T with integer LDS histograms; each digit is chosen by a block-wide scan
// of bin counts from the top. The row is then compacted in index order: per
// wave segment counts, a scan over waves, and ballot prefix sums, taking all
// keys > T and the lowest-index ties == T. Keys are cached in LDS when the row
// fits, otherwise re-read from global memory each pass.
#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int TK_NT = 512;
constexpr int TK_NW = TK_NT / 64;
constexpr int TK_BINS = 2048;
constexpr int TK_CACHE_MAX = 32768;  // keys cached in LDS (128 KiB)

__device__ __forceinline__ int wave_incl_scan(int v, int l) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (l >= o) v += t;
  }
  return v;
}

// Block-wide exclusive scan (thread order) of one int per thread.
__device__ __forceinline__ int block_excl_scan(int v, int* red) {
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, l);
  if (l == 63) red[wv] = inc;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int u = 0; u < TK_NW; ++u) off += (u < wv) ? red[u] : 0;
  __syncthreads();
  return off + inc - v;
}

// Given counts of nb bins, find the bin b such that the count of bins above b
// is < need <= count of bins >= b. Returns via out[0] = bin, out[1] = count above.
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, int need, int* red, int* out) {
  const int bpt = nb / TK_NT;
  const int t = threadIdx.x;
  // thread t owns bins [nb - (t+1)*bpt, nb - t*bpt), scanned from high to low
  const int hi = nb - t * bpt;
  int loc = 0;
  for (int u = 1; u <= bpt; ++u) loc += (int)hist[hi - u];
  const int above = block_excl_scan(loc, red);
  if (above < need && need <= above + loc) {
    int c = above;
    for (int u = 1; u <= bpt; ++u) {
      const int cnt = (int)hist[hi - u];
      if (need <= c + cnt) {
        out[0] = hi - u;
        out[1] = c;
        break;
      }
      c += cnt;
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(TK_NT)
topk_row_kernel(const float* __restrict__ scores, const int32_t* __restrict__ q_pos,
                const int32_t* __restrict__ n_comp, int64_t Tq, int64_t N_max, int m, int top_k,
                int32_t* __restrict__ idx_out, float* __restrict__ score_out, int cache_cap) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist = smem;                                  // TK_BINS
  int* red = reinterpret_cast<int*>(smem + TK_BINS);      // 32 ints
  int* res = red + 32;                                    // 32 ints
  uint32_t* kc = smem + TK_BINS + 64;                     // key cache (16-byte aligned)

  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int64_t row = blockIdx.x;
  const int64_t b = row / Tq;
  int64_t V64 = min((int64_t)n_comp[b], ((int64_t)q_pos[row] + 1) / m);
  const int V = (int)max((int64_t)0, min(V64, N_max));
  const int K = min(top_k, V);
  const float* srow = scores + row * N_max;
  int32_t* orow = idx_out + row * (int64_t)top_k;
  float* osc = score_out ? score_out + row * (int64_t)top_k : nullptr;

  if (K == V) {  // everything visible is selected
    for (int i = t; i < top_k; i += TK_NT) {
      orow[i] = i < V ? i : -1;
      if (osc) osc[i] = i < V ? srow[i] : -INFINITY;
    }
    return;
  }
  const bool cached = V <= cache_cap;
  if (cached) {
    // 16-byte loads, 8 in flight per thread, when the row is 16-byte aligned
    if ((reinterpret_cast<uintptr_t>(srow) & 15) == 0) {
      const int V4 = V >> 2;
      const f32x4_t* s4 = reinterpret_cast<const f32x4_t*>(srow);
      for (int i0 = t; i0 < V4; i0 += TK_NT * 8) {
        f32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * TK_NT;
          if (i < V4) v[u] = s4[i];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * TK_NT;
          if (i < V4) {
            u32x4_t k4 = {f32_key(v[u][0]), f32_key(v[u][1]), f32_key(v[u][2]), f32_key(v[u][3])};
            *reinterpret_cast<u32x4_t*>(kc + 4 * i) = k4;
          }
        }
      }
      for (int i = 4 * V4 + t; i < V; i += TK_NT) kc[i] = f32_key(srow[i]);
    } else {
      for (int i = t; i < V; i += TK_NT) kc[i] = f32_key(srow[i]);
    }
  }
  // (the first histogram clear below is followed by a barrier)

  uint32_t prefix = 0;
  int need = K;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbits = pass == 2 ? 10 : 11;
    const int nb = 1 << nbits;
    const int hshift = shift + nbits;  // bits above this digit
    for (int i = t; i < nb; i += TK_NT) hist[i] = 0;
    __syncthreads();
    for (int i = t; i < V; i += TK_NT) {
      const uint32_t k = cached ? kc[i] : f32_key(srow[i]);
      const bool in = (pass == 0) || ((k >> hshift) == prefix);
      if (in) atomicAdd(&hist[(k >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(hist, nb, need, red, res);
    prefix = (prefix << nbits) | (uint32_t)res[0];
    need -= res[1];
    __syncthreads();
  }
  const uint32_t T = prefix;  // exact K-th largest key; take `need` ties (>= 1)

  // ---- compaction in index order
  const int seg = ((V + TK_NW - 1) / TK_NW + 63) / 64 * 64;
  const int lo = min(V, wv * seg), hi = min(V, lo + seg);
  int gt = 0, eq = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + l;
    uint32_t k = 0;
    if (i < hi) k = cached ? kc[i] : f32_key(srow[i]);
    gt += __popcll(__ballot(i < hi && k > T));
    eq += __popcll(__ballot(i < hi && k == T));
  }
  if (l == 0) {
    red[wv] = gt;
    red[TK_NW + wv] = eq;
  }
  __syncthreads();
  int eq_before = 0, sel_before = 0;
  for (int u = 0; u < wv; ++u) {
    const int gu = red[u], eu = red[TK_NW + u];
    sel_before += gu + max(0, min(need - eq_before, eu));
    eq_before += eu;
  }
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));
  int run_sel = 0, run_eq = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + l;
    uint32_t k = 0;
    if (i < hi) k = cached ? kc[i] : f32_key(srow[i]);
    const bool is_gt = i < hi && k > T;
    const bool is_eq = i < hi && k == T;
    const uint64_t eqm = __ballot(is_eq);
    const int eq_rank = eq_before + run_eq + __popcll(eqm & below);
    const bool sel = is_gt || (is_eq && eq_rank < need);
    const uint64_t selm = __ballot(sel);
    if (sel) {
      const int pos = sel_before + run_sel + __popcll(selm & below);
      if (pos < top_k) orow[pos] = i;
      if (osc && pos < top_k) osc[pos] = srow[i];
    }
    run_sel += __popcll(selm);
    run_eq += __popcll(eqm);
  }
  for (int i = K + t; i < top_k; i += TK_NT) {
    orow[i] = -1;
    if (osc) osc[i] = -INFINITY;
  }
}

size_t topk_ws_bytes(int64_t, int64_t, int64_t, int) { return 0; }

hipError_t run_topk(const TopkLaunch& a, hipStream_t st) {
  const int64_t rows = a.B * a.Tq;
  if (rows == 0) return hipSuccess;
  const int cache = (int)min(a.N_max, (int64_t)TK_CACHE_MAX);
  const size_t lds = (size_t)(TK_BINS + 64 + cache) * 4;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_row_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)((TK_BINS + 64 + TK_CACHE_MAX) * 4));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)rows), dim3(TK_NT), lds, st, a.scores, a.q_pos, a.n_comp,
                     a.Tq, a.N_max, a.m, a.top_k, a.idx, a.out_score, cache);
  return hipGetLastError();
}

}  // namespace csa
