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

// Given counts of nb bins, find the bin b with (count above b) < need <=
// (count of bins >= b), using wave 0 only: lane l sums the nb/64 bins
// [nb - (l+1)*nb/64, nb - l*nb/64), one shuffle scan over lanes, and the lane
// holding the threshold walks its bins. Result: out[0] = b, out[1] = count
// above b. Ends with a barrier that publishes out[] and frees hist.
__device__ __forceinline__ void find_bin_wave(const uint32_t* hist, int nb, int need, int* out) {
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const int bpl = nb >> 6;  // 32 or 16
    const int lo_bin = nb - (l + 1) * bpl;
    uint32_t v[32];  // this lane's bins, ascending; kept in registers for the walk
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4_t x = (q * 4 < bpl) ? *reinterpret_cast<const u32x4_t*>(hist + lo_bin + q * 4) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) v[q * 4 + e] = x[e];
    }
    int loc = 0;
#pragma unroll
    for (int u = 0; u < 32; ++u) loc += (int)v[u];
    const int inc = wave_incl_scan_dpp(loc);
    const int above = inc - loc;
    if (above < need && need <= inc) {
      int c = above, bin = -1, cab = 0;
#pragma unroll
      for (int u = 31; u >= 0; --u) {  // from the highest bin of the lane down
        const int cnt = (int)v[u];
        if (bin < 0 && u < bpl && need <= c + cnt) {
          bin = lo_bin + u;
          cab = c;
        }
        if (u < bpl) c += cnt;
      }
      out[0] = bin;
      out[1] = cab;
    }
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
};

template <int SRC>
__global__ void __launch_bounds__(TK_NT) topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* hist = smem;                                   // 2 x TK_BINS (alternating passes)
  int* red = reinterpret_cast<int*>(smem + 2 * TK_BINS);   // 32
  int* res = red + 32;                                     // 32
  const int CH = a.chunk;
  uint32_t* kc = smem + 2 * TK_BINS + 64;                  // CH keys
  int32_t* ic = reinterpret_cast<int32_t*>(kc + CH);       // TK_CANDS: indices

  const int t = threadIdx.x, l = t & 63, wv = t >> 6;
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x, nchunk = gridDim.x;
  int64_t n_row;
  if constexpr (SRC == TK_SCORES) {
    const int64_t b = row / a.Tq;
    const int64_t v = min((int64_t)a.n_comp[b], ((int64_t)a.q_pos[row] + 1) / a.m);
    n_row = max((int64_t)0, min(v, a.N_max));
  } else {
    n_row = a.n_cand;
  }
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

  // ---- radix select of the K-th largest key (skipped when everything is kept).
  // The digits start below the common prefix of the chunk's smallest and
  // largest key, so the first histogram spreads over the chunk's own range
  // (a fixed top digit puts scores of similar magnitude into a few bins, and
  // the LDS atomics of a pass then serialise on them).
  uint32_t T = 0;
  int need = 0;
  if (K < n) {
    need = K;
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    {
      const int n4 = n >> 2;
      const u32x4_t* k4p = reinterpret_cast<const u32x4_t*>(kc);
      for (int i = t; i < n4; i += TK_NT) {
        const u32x4_t k4 = k4p[i];
        kmin = min(min(kmin, k4[0]), min(k4[1], min(k4[2], k4[3])));
        kmax = max(max(kmax, k4[0]), max(k4[1], max(k4[2], k4[3])));
      }
      for (int i = 4 * n4 + t; i < n; i += TK_NT) {
        kmin = min(kmin, kc[i]);
        kmax = max(kmax, kc[i]);
      }
    }
    kmin = wave_min_u32_dpp(kmin);
    kmax = wave_max_u32_dpp(kmax);
    if (l == 0) {
      red[wv] = (int)kmin;
      red[TK_NW + wv] = (int)kmax;
    }
    for (int i = t; i < 2 * TK_BINS; i += TK_NT) hist[i] = 0;
    __syncthreads();  // also publishes the key cache
#pragma unroll
    for (int u = 0; u < TK_NW; ++u) {
      kmin = min(kmin, (uint32_t)red[u]);
      kmax = max(kmax, (uint32_t)red[TK_NW + u]);
    }
    if (kmin == kmax) {
      T = kmin;  // all keys equal: the K lowest indices
    } else {
      int R = 32 - __builtin_clz(kmin ^ kmax);  // bits below the common prefix
      uint32_t prefix = R >= 32 ? 0u : (kmin >> R);
#pragma unroll 1
      for (int pass = 0; R > 0; ++pass) {
        const int nbits = min(11, R);
        const int shift = R - nbits;
        const uint32_t dmask = (1u << nbits) - 1u;
        uint32_t* h = hist + (pass & 1) * TK_BINS;
        auto add = [&](uint32_t k) {
          if (R >= 32 || (k >> R) == prefix) atomicAdd(&h[(k >> shift) & dmask], 1u);
        };
        const int n4 = n >> 2;
        const u32x4_t* k4p = reinterpret_cast<const u32x4_t*>(kc);
        // four 16-byte LDS reads in flight per thread before their atomics
        for (int i0 = t; i0 < n4; i0 += 4 * TK_NT) {
          u32x4_t k4[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) k4[u] = (i0 + u * TK_NT < n4) ? k4p[i0 + u * TK_NT] : u32x4_t{0, 0, 0, 0};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (i0 + u * TK_NT >= n4) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) add(k4[u][e]);
          }
        }
        for (int i = 4 * n4 + t; i < n; i += TK_NT) add(kc[i]);
        __syncthreads();
        find_bin_wave(h, TK_BINS, need, res);
        prefix = (prefix << nbits) | (uint32_t)res[0];
        need -= res[1];
        if (pass == 0)  // pass 2 reuses this buffer; nothing reads it during pass 1
          for (int i = t; i < TK_BINS; i += TK_NT) h[i] = 0;
        R = shift;
      }
      T = prefix;  // take all keys > T and the `need` lowest-index keys == T
    }
  } else {
    __syncthreads();  // publish the key cache
  }

  // ---- ordered compaction: each wave owns a contiguous segment; a lane
  // handles 4 consecutive keys per step (one 16-byte LDS read); index-order
  // prefixes come from ballots of the bits of the per-lane counts (0..4)
  const int seg = ((n + TK_NW - 1) / TK_NW + 255) / 256 * 256;
  const int s_lo = min(n, wv * seg), s_hi = min(n, s_lo + seg);
  const bool all = K == n;
  const u32x4_t* kc4 = reinterpret_cast<const u32x4_t*>(kc);
  int gt = 0, eq = 0;
  if (!all) {
    for (int base = s_lo; base < s_hi; base += 512) {
      u32x4_t k4[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i0 = base + u * 256 + 4 * l;
        k4[u] = i0 < s_hi ? kc4[i0 >> 2] : u32x4_t{0, 0, 0, 0};
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
#pragma unroll
  for (int u = 0; u < TK_NW; ++u) {
    const int gu = red[u], eu = red[TK_NW + u];
    if (u < wv) {
      sel_before += gu + (all ? 0 : max(0, min(need - eq_before, eu)));
      eq_before += eu;
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
  const int64_t obase = final_out ? row * (int64_t)top_k : (row * nchunk + c) * (int64_t)top_k;
  for (int base = s_lo; base < s_hi; base += 256) {
    const int i0 = base + 4 * l;
    const u32x4_t k4 = i0 < s_hi ? kc4[i0 >> 2] : u32x4_t{0, 0, 0, 0};
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
        if (pos < top_k) {
          int32_t gi;
          if constexpr (SRC == TK_SCORES) gi = (int32_t)(lo + i0 + e);
          else gi = ic[i0 + e];
          if (final_out) {
            a.out_idx[obase + pos] = gi;
            if (a.out_score) a.out_score[obase + pos] = key_f32(k4[e]);
          } else {
            a.nkey[obase + pos] = k4[e];
            a.nidx[obase + pos] = gi;
          }
        }
        ++pos;
      }
    }
    run_sel += sel_tot;
    run_eq += eq_tot;
  }
  for (int i = K + t; i < top_k; i += TK_NT) {
    if (final_out) {
      a.out_idx[obase + i] = -1;
      if (a.out_score) a.out_score[obase + i] = -INFINITY;
    } else {
      a.nkey[obase + i] = 0u;  // below every finite key: never selected later
      a.nidx[obase + i] = -1;
    }
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
// what fits in LDS. Depends on shape arguments only.
static int plan_levels(int64_t rows, int64_t n0, int top_k, int64_t* nch, int64_t* nlen, int64_t* chunk) {
  int lv = 0;
  int64_t n = n0;
  while (true) {
    const int64_t cmax = lv == 0 ? TK_CHUNK_S : TK_CHUNK_C;
    const int64_t want = pow2_at_least((rows * n + TK_TARGET_WG - 1) / TK_TARGET_WG);
    const int64_t ch = std::min(cmax, std::max<int64_t>({want, (int64_t)TK_CHUNK_MIN, pow2_at_least(4 * (int64_t)top_k)}));
    chunk[lv] = ch;
    nch[lv] = std::max<int64_t>(1, (n + ch - 1) / ch);
    nlen[lv] = n;
    ++lv;
    if (nch[lv - 1] == 1 || lv == 12) break;
    n = nch[lv - 1] * top_k;
  }
  return lv;
}

size_t topk_ws_bytes(int64_t B, int64_t Tq, int64_t N_max, int top_k) {
  int64_t nch[12], nlen[12], chunk[12];
  const int lv = plan_levels(B * Tq, N_max, top_k, nch, nlen, chunk);
  size_t mx = 0;
  for (int i = 0; i + 1 < lv; ++i) mx = std::max(mx, (size_t)(B * Tq) * nch[i] * top_k * 8);
  return mx == 0 ? 0 : 2 * ((mx + 255) & ~size_t(255));
}

hipError_t run_topk(const TopkLaunch& L, hipStream_t st) {
  const int64_t rows = L.B * L.Tq;
  if (rows == 0) return hipSuccess;
  static bool attr_set = false;
  const size_t lds_s = (size_t)(2 * TK_BINS + 64 + TK_CHUNK_S) * 4;
  const size_t lds_c = (size_t)(2 * TK_BINS + 64 + 2 * TK_CHUNK_C) * 4;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<TK_SCORES>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_s);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)topk_kernel<TK_CANDS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_c);
    if (e != hipSuccess) return e;
    attr_set = true;
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
      hipLaunchKernelGGL(topk_kernel<TK_SCORES>, grid, dim3(TK_NT), (2 * TK_BINS + 64 + chunk[i]) * 4, st, a);
    } else {
      hipLaunchKernelGGL(topk_kernel<TK_CANDS>, grid, dim3(TK_NT), (2 * TK_BINS + 64 + 2 * chunk[i]) * 4, st, a);
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
