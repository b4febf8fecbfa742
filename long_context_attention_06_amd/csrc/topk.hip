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

#include "kernels.h"
#include "select.h"

namespace csa {
using namespace sel;

constexpr int TK_NT = 256;
constexpr int TK_NW = TK_NT / 64;
constexpr int TK_BINS = BINS;
constexpr int TK_BPL = TK_BINS / TK_NT;    // histogram bins per thread
constexpr int TK_DSHIFT = DSHIFT;
constexpr int TK_ROW_MAX = 16384;          // keys of a row finished by one workgroup
constexpr int TK_ROW_CAP = 3968;           // candidates of topk_row_kernel (31 KB of LDS: four workgroups per CU)
constexpr int TK_FCH = 4096;               // keys per chunk workgroup: four wave segments of 1024
constexpr int TK_SEG = TK_FCH / TK_NW;     // keys per wave segment
constexpr int TK_WCAP = 512;               // candidates kept per wave segment
constexpr int TK_LDS_MAX = 160 * 1024;     // LDS of a workgroup on gfx950
constexpr uint32_t TK_HINT_CLAMP = HINT_CLAMP;

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
  block_compact<TK_NT>(
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
  block_select<TK_NT>(keys, V, K, hist, red, res, T, need);
  write_selection(a, row, keys, V, K, false, T, need, red, [](int i) { return (int32_t)i; });
}

// Select the row among M candidates cached in LDS (keys ck, position order;
// every key whose digit is at least b) and write it.
template <class Idx>
__device__ void select_in_candidates(const TopkArgs& a, int64_t row, const uint32_t* ck, int M, int K, int b,
                                     uint32_t* hist, int* red, int* res, Idx idx_of) {
  uint32_t T;
  int need;
  const bool some = refine_threshold<TK_NT>(ck, M, K, b, nullptr, hist, red, res, T, need);
  write_selection(a, row, LdsKeys{ck}, M, K, !some, T, need, red, idx_of);
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
__global__ void __launch_bounds__(TK_NT) __attribute__((amdgpu_waves_per_eu(4, 4))) topk_row_kernel(TopkArgs a) {
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
  RegKeys<TK_NT, KPT> rk;
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
  find_bin_block<TK_NT>(hist, K, red, res);
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
  RegKeys<TK_NT, 16> rk;
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
  RegKeys<TK_NT, TK_FCH / TK_NT> rk;
  rk.load(a.scores + row * a.N_max, lo, hi);
  load_hint(h, hist);
  if (t == 0) res[0] = -1;
  __syncthreads();
  find_bin_block<TK_NT>(hist, K, red, res);
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
    ovf = block_sum<TK_NT>(ovf, red);
    M = ovf ? -1 : base;
  }
  if (M >= K && M <= a.cap) {
    // gather: P threads per segment, each copying every P-th candidate (up to
    // 16 loads in flight per thread); a segment's count is the step of the
    // offsets (no second read of the counts)
    const int P = nseg >= TK_NT ? 1 : TK_NT / nseg;
    for (int s0 = 0; s0 < nseg; s0 += TK_NT / P) {
      const int sg = s0 + t / P, sub = t % P;
      if (sg < nseg) {
        const int o = off[sg], n = (sg + 1 < nseg ? off[sg + 1] : M) - o;
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
