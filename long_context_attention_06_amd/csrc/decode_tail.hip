// Fused tail of a CSA decode step for gfx950: the exact top-k of the indexer
// scores, the shared-KV MQA over the selected entries, the window and the
// sink, and the merge of the attention splits, in one launch.
//
// What is computed ("DeepSeek V4 脱离 CUDA 全栈国产化", deepseek.csdn.net,
// section 二, CSA steps 2 and 3; liduos.com "deepseek-v4-engineering-
// tradeoffs", "1M Context 的结构与取舍", for the window and the sink): the
// results of indexer_topk followed by sparse_mqa_decode_multi, bit for bit --
// the selection is exact, the attention splits and their tile loop are those
// of the separate kernels, and the splits merge in the same order with the
// same arithmetic.
//
// Why one launch: with the scores in memory, what remains of a decode step is
// latency -- a top-k whose last chunk to finish selects alone, an attention
// whose splits wait for the top-k's output, a merge that waits for the
// splits. Here the workgroups of a query (all resident at once: the grid is
// at most one workgroup per CU) pass each other their results through
// device-coherent memory and two arrival counters instead of kernel
// boundaries:
//  1. filter: every workgroup compacts the candidates of its chunks of the
//     row (keys whose digit reaches the threshold bin of the histogram the
//     scan accumulated), one list per wave, in position order, and adds the
//     counts of the threshold bin's keys by their next 11 bits;
//  2. arrival 1; each attention workgroup gathers every list and finds the
//     exact K-th key from those counts (select.h), then keeps the slots of
//     its own splits of the selection;
//  3. attention over those slots (attn_core.h), unnormalised partials out;
//  4. arrival 2; every workgroup of the query merges a share of the heads
//     and dims, in split order, and adds the sink.
// The histogram is a hint: when it does not hold, the selection runs over the
// full score row instead (exact, slower).
#include <algorithm>

#include "attn_core.h"
#include "kernels.h"
#include "select.h"

namespace csa {
using namespace sel;

namespace dtl {
constexpr int NT = bfk::NT;            // 512 threads: the attention's eight waves
constexpr int NW = NT / 64;
constexpr int FCH = 4096;              // keys per filter pass (8 per thread)
constexpr int SEG = FCH / NW;          // keys per wave segment
constexpr int WCAP = 256;              // candidates kept per wave segment
constexpr int RING = 128 * 1024;       // the attention's tile ring; the select's scratch before it
constexpr int OFF_B = 8 * 1024;        // ring offsets: histogram at 0, segment offsets, own slots, candidates
constexpr int SEG_MAX = 4096 - 8;      // wave segments per row (rows up to ~2M keys)
constexpr int SEL_B = OFF_B + 4096 * 4;
constexpr int CAND_B = SEL_B + bfk::TAB_MAX * 4;
constexpr int CAP = (RING - CAND_B) / 8;  // candidates a workgroup holds
constexpr int MAX_SPLITS = 16;
constexpr int SPIN = 1 << 22;          // bound of a wait (never reached when all workgroups are resident)
constexpr uint32_t FAILED = 1u << 16;  // added to a query's second counter when a workgroup gave up
constexpr int SC1 = 16;                // buffer cache policy: device-coherent (past the per-XCD caches)
}  // namespace dtl

struct TailArgs {
  // attention
  const uint16_t* q;
  RowSrc src;
  const int32_t* win_len;
  const float* sink;
  float scale_log2;
  int H, slots, split_rows, nsplit;
  float* part_o;  // [nq, nsplit, H, 512]
  float* part_ml;
  void* out;
  float* lse;
  int out_dt;
  // selection
  const float* scores;     // [nq, N_max]
  const int32_t* q_pos;    // [nq]
  const int32_t* n_comp;   // [nq / Tq]
  int m, top_k;
  uint32_t* hint;          // [nq, BINS] digit counts, accumulated by the scan; cleared here
  uint32_t* sync;          // [nq, 2] arrival counters, zero on entry
  uint32_t* sub;           // [nq, BINS] counts of the threshold bin by the next 11 bits, zero on entry
  uint32_t* wkey;          // [nq, nseg, WCAP] candidates per wave segment
  int32_t* widx;
  int32_t* wcnt;           // [nq, nseg]; WCAP + 1 marks an overflowing segment
  int nseg, passes;
  int32_t* out_idx;        // [nq, top_k]
  float* out_score;        // nullable
  // the query prologue and output epilogue (sparse source): RMSNorm of each
  // head's query with qk_gamma, rotation of its last qk_R dims by the query's
  // position, and the inverse rotation of the output; qk_flags 0: none
  int qk_flags;            // 1: norm, 2: rotation
  const float* qk_gamma;   // [D] or NULL (ones)
  float qk_eps;
  int qk_R;
  double qk_log2_theta;
};

// cos and sin of the angle of rotated pair i at position p, formed in double
// precision as the standalone prologue forms it
__device__ __forceinline__ void rope_cs(double p, int i, int R, double log2_theta, float& c, float& s) {
  double sn, cs;
  sincos(p * exp2(-2.0 * (double)i / (double)R * log2_theta), &sn, &cs);
  c = (float)cs;
  s = (float)sn;
}

template <class T>
__device__ __forceinline__ void st_coh(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_coh(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every store of the workgroup has completed, then one arrival is counted.
__device__ __forceinline__ void arrive(uint32_t* ctr) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until the counter reaches target. Bounded: every arrival comes from a
// workgroup of the same launch, and the host launches at most one workgroup
// per CU, so all of them run at once; if the hardware ever held some back,
// the wait gives up and the caller marks its results invalid (NaN, index -1)
// instead of hanging. Returns the counter's value (uniform).
__device__ __forceinline__ uint32_t wait_for(const uint32_t* ctr, uint32_t target, int* slot) {
  if (threadIdx.x == 0) {
    uint32_t v = ld_coh(ctr);
    for (int it = 0; it < dtl::SPIN && v < target; ++it) {
      __builtin_amdgcn_s_sleep(1);
      v = ld_coh(ctr);
    }
    *slot = (int)v;
  }
  __syncthreads();
  return (uint32_t)*slot;
}

template <bool KV8>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
csa_decode_tail_kernel(TailArgs a) {
  using namespace bfk;
  constexpr int TB = DecRows<KV8>::TB;
  static_assert(NBUF * TB <= dtl::RING, "tile ring");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[dtl::RING];
  __shared__ __attribute__((aligned(16))) f32x4_t xchg[NW][2][64];
  __shared__ __attribute__((aligned(16))) int tab[TAB_MAX];
  __shared__ __attribute__((aligned(16))) int red[2 * NW], res[8], cnt[2 * NW], nrow[dtl::MAX_SPLITS];
  uint32_t* hist = reinterpret_cast<uint32_t*>(ring);
  int* off = reinterpret_cast<int*>(ring + dtl::OFF_B);
  int* mysel = reinterpret_cast<int*>(ring + dtl::SEL_B);
  uint32_t* ck = reinterpret_cast<uint32_t*>(ring + dtl::CAND_B);
  int32_t* ci = reinterpret_cast<int32_t*>(ck + dtl::CAP);

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = l >> 4, l16 = l & 15;
  const int hg = w & 3, dh = w >> 2;
  const int head = hg * 16 + l16;
  const int c = blockIdx.x, P = gridDim.x;
  const int64_t qi = blockIdx.y;
  const int H = a.H, SR = a.split_rows, nsplit = a.nsplit, top_k = a.top_k;
  const int nmine = c < nsplit ? (nsplit - 1 - c) / P + 1 : 0;  // splits c, c + P, ... of this workgroup

  // ---- the query (attention workgroups): its loads overlap the filter
  bf16x8_t qb[8];
  if (nmine > 0) {
    const bool hok = head < H;
    const uint16_t* qp = a.q + (qi * H + (hok ? head : 0)) * (int64_t)D + dh * 256 + G * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[s] = as_bf16x8(hok ? ld16(qp + s * 32) : u32x4_t{0, 0, 0, 0});
  }

  // ---- 1. filter
  const int64_t Tq = a.src.Tq;
  int V = (int)min((int64_t)a.n_comp[qi / Tq], ((int64_t)a.q_pos[qi] + 1) / a.m);
  V = (int)max((int64_t)0, min((int64_t)V, a.src.N_max));
  const int K = min(top_k, V);
  const float* srow = a.scores + qi * a.src.N_max;
  int b = -1;
  if (K < V) {
    const uint32_t* h = a.hint + qi * BINS;
#pragma unroll
    for (int u = 0; u < BINS / dtl::NT; ++u) hist[tid + u * dtl::NT] = min(h[tid + u * dtl::NT], HINT_CLAMP);
    if (tid == 0) res[0] = -1;
    __syncthreads();
    find_bin_block<dtl::NT>(hist, K, red, res);
    b = res[0];
    for (int ps = 0; ps < a.passes; ++ps) {
      const int chunk = c * a.passes + ps;
      const int lo = chunk * dtl::FCH;
      if (lo >= V) break;
      const int hi = min(V, lo + dtl::FCH);
      RegKeys<dtl::NT, dtl::FCH / dtl::NT> rk;
      rk.load(srow, lo, hi);
      constexpr int KPT = dtl::FCH / dtl::NT;
      const int seg = chunk * dtl::NW + w;
      const int64_t lb = (qi * a.nseg + seg) * (int64_t)dtl::WCAP;
      int run = 0;
#pragma unroll
      for (int j = 0; j < KPT / 4; ++j) {
        bool cand[4];
        int n = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cand[e] = b >= 0 && rk.pos(lo, j, e) < hi && (int)(rk.k[4 * j + e] >> DSHIFT) >= b;
          n += cand[e];
        }
        int st;
        int s = run + excl3(n, st);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (cand[e]) {
            const uint32_t k = rk.k[4 * j + e];
            if (s < dtl::WCAP) {
              st_coh(&a.wkey[lb + s], k);
              st_coh(&a.widx[lb + s], (int32_t)rk.pos(lo, j, e));
            }
            if ((int)(k >> DSHIFT) == b)
              __hip_atomic_fetch_add(&a.sub[qi * BINS + ((k >> 10) & (BINS - 1))], 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
            ++s;
          }
        run += st;
      }
      if (l == 0) st_coh(&a.wcnt[qi * a.nseg + seg], b < 0 ? dtl::WCAP + 1 : min(run, dtl::WCAP + 1));
    }
  }
  arrive(&a.sync[qi * 2]);

  // ---- the query prologue (while the other workgroups filter): RMSNorm over
  // the head's 512 dims (a wave holds 256 of them: the pair w, w ^ 4 adds its
  // halves through LDS), then the rotation of the last R dims (pairs of
  // consecutive dims inside a lane's 8), in fp32, rounded back to bf16
  if (a.qk_flags && nmine > 0) {
    float v[8][8];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) unpack_bf16x8(__builtin_bit_cast(u32x4_t, qb[s2]), v[s2]);
    if (a.qk_flags & 1) {
      float ss = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[s2][e] * v[s2][e];
      ss += shfl_xor(ss, 16);
      ss += shfl_xor(ss, 32);
      float* half = reinterpret_cast<float*>(xchg);  // free until the tile loop
      if (G == 0) half[w * 16 + l16] = ss;
      __syncthreads();
      const float tot = half[w * 16 + l16] + half[(w ^ 4) * 16 + l16];
      const float r = 1.0f / sqrtf(tot / (float)D + a.qk_eps);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = dh * 256 + s2 * 32 + G * 8 + e;
          v[s2][e] *= r * (a.qk_gamma ? a.qk_gamma[d] : 1.0f);
        }
    }
    if (a.qk_flags & 2) {
      // lane i < R/2 forms pair i's angle once; the lanes that rotate it
      // read it by a shuffle (all lanes shuffle; s0 is even, so a pair never
      // straddles it)
      const int s0 = D - a.qk_R;
      float cl = 1.0f, sl = 0.0f;
      if (l < a.qk_R / 2) rope_cs((double)a.q_pos[qi], l, a.qk_R, a.qk_log2_theta, cl, sl);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        if (dh * 256 + s2 * 32 + 32 <= s0) continue;  // uniform: no rotated dim in this chunk
        const int d0 = dh * 256 + s2 * 32 + G * 8;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bool rot = d0 + e >= s0;
          const int src = rot ? (d0 + e - s0) >> 1 : 0;
          const float c2 = __shfl(cl, src, 64), sn = __shfl(sl, src, 64);
          if (rot) {
            const float x0 = v[s2][e], x1 = v[s2][e + 1];
            v[s2][e] = x0 * c2 - x1 * sn;
            v[s2][e + 1] = x0 * sn + x1 * c2;
          }
        }
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      qb[s2] = as_bf16x8(u32x4_t{pack_bf16x2(v[s2][0], v[s2][1]), pack_bf16x2(v[s2][2], v[s2][3]),
                                 pack_bf16x2(v[s2][4], v[s2][5]), pack_bf16x2(v[s2][6], v[s2][7])});
  }

  // ---- 2. selection (attention workgroups): the slots of this workgroup's splits
  if (nmine > 0) {
    const bool ok = wait_for(&a.sync[qi * 2], (uint32_t)P, &res[6]) >= (uint32_t)P;  // every list is in
    if (!ok) {
      // give up on this query (see wait_for): invalid indices, and the merge writes NaN
      for (int pos = tid; pos < top_k; pos += dtl::NT)
        if ((pos / SR) % P == c) a.out_idx[qi * top_k + pos] = -1;
      if (tid == 0) __hip_atomic_fetch_add(&a.sync[qi * 2 + 1], dtl::FAILED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      goto merge;
    }
    if (c == 0) {
      uint32_t* h = a.hint + qi * BINS;
#pragma unroll
      for (int u = 0; u < BINS / dtl::NT; ++u) h[tid + u * dtl::NT] = 0u;
    }
    // slot pos -> this workgroup's own slot index, or -1
    auto mine = [&](int pos) {
      const int sp = pos / SR;
      return sp % P == c ? (sp / P) * SR + pos % SR : -1;
    };
    auto take = [&](int pos, int idx, float score) {
      const int m = mine(pos);
      if (m < 0) return;
      mysel[m] = idx;
      a.out_idx[qi * top_k + pos] = idx;
      if (a.out_score) a.out_score[qi * top_k + pos] = score;
    };
    if (K == V) {
      for (int pos = tid; pos < top_k; pos += dtl::NT) take(pos, pos < V ? pos : -1, pos < V ? srow[pos] : -INFINITY);
    } else {
      const int nsr = (V + dtl::SEG - 1) / dtl::SEG;
      // the threshold bin's counts by the next 11 bits: loaded beside the
      // segment counts (one round trip for both)
      uint32_t subv[BINS / dtl::NT];
#pragma unroll
      for (int u = 0; u < BINS / dtl::NT; ++u) subv[u] = ld_coh(&a.sub[qi * BINS + tid + u * dtl::NT]);
      int M = -1;
      if (b >= 0 && nsr <= dtl::SEG_MAX) {
        const int32_t* cntp = a.wcnt + qi * a.nseg;
        int base = 0, ovf = 0;
        for (int s0 = 0; s0 < nsr; s0 += dtl::NT) {
          const int v = s0 + tid < nsr ? ld_coh(&cntp[s0 + tid]) : 0;
          ovf |= v > dtl::WCAP;
          const int vc = min(v, dtl::WCAP);
          const int inc = wave_incl_scan_dpp(vc);
          if (l == 63) red[w] = inc;
          __syncthreads();
          int wb = 0, tot = 0;
#pragma unroll
          for (int u = 0; u < NW; ++u) {
            wb += u < w ? red[u] : 0;
            tot += red[u];
          }
          if (s0 + tid < nsr) off[s0 + tid] = base + wb + inc - vc;
          base += tot;
          __syncthreads();
        }
        if (tid == 0) off[nsr] = base;
        ovf = block_sum<dtl::NT>(ovf, red);
        M = ovf ? -1 : base;
      }
      if (M >= K && M <= dtl::CAP) {
        // gather: Pt threads per segment, each copying every Pt-th candidate
        const int Pt = nsr >= dtl::NT ? 1 : dtl::NT / nsr;
        for (int s0 = 0; s0 < nsr; s0 += dtl::NT / Pt) {
          const int sg = s0 + tid / Pt, sub = tid % Pt;
          if (sg < nsr) {
            const int o = off[sg], n = off[sg + 1] - o;
            const int64_t lb = (qi * a.nseg + sg) * (int64_t)dtl::WCAP;
            for (int j0 = sub; j0 < n; j0 += 8 * Pt) {
              uint32_t kv[8];
              int32_t iv[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const int j = j0 + u * Pt;
                if (j < n) {
                  kv[u] = ld_coh(&a.wkey[lb + j]);
                  iv[u] = ld_coh(&a.widx[lb + j]);
                }
              }
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const int j = j0 + u * Pt;
                if (j < n) {
                  ck[o + j] = kv[u];
                  ci[o + j] = iv[u];
                }
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < BINS / dtl::NT; ++u) hist[tid + u * dtl::NT] = subv[u];
        __syncthreads();
        uint32_t T;
        int need;
        const bool some = refine_threshold<dtl::NT>(ck, M, K, b, hist, hist, red, res, T, need);
        block_compact<dtl::NT>(
            LdsKeys{ck}, M, K, !some, T, need, top_k, red,
            [&](int pos, uint32_t key, int i) { take(pos, ci[i], key_f32(key)); },
            [&](int pos) { take(pos, -1, -INFINITY); });
      } else {
        // the hint did not hold: the whole row, from memory
        const RowKeys keys{srow, V, (reinterpret_cast<uintptr_t>(srow) & 15) == 0};
        uint32_t T = 0;
        int need = 0;
        block_select<dtl::NT>(keys, V, K, hist, red, res, T, need);
        block_compact<dtl::NT>(
            keys, V, K, false, T, need, top_k, red, [&](int pos, uint32_t key, int i) { take(pos, i, key_f32(key)); },
            [&](int pos) { take(pos, -1, -INFINITY); });
      }
    }
    __syncthreads();  // mysel is complete

    // ---- row tables of every own split (the select's scratch is in the
    // ring, which the tiles then take over)
    for (int k = 0; k < nmine; ++k) {
      const int sp = c + k * P;
      const QRows rq = query_rows<SRC_SPARSE_DEC, DecRows<KV8>::SROWB>(a.src, a.win_len, nullptr, nullptr, 1, qi,
                                                                         sp, a.slots, SR);
      const int n = build_row_table_from<SRC_SPARSE_DEC, dtl::NT, TR>(
          a.src, rq, qi, tab + k * SR, cnt, nullptr, [&](int j) { return mysel[k * SR + (j - sp * SR)]; });
      if (tid == 0) nrow[k] = n;
    }
    __syncthreads();
  }

  // ---- 3. attention over the own splits in turn
  if (nmine > 0) {
#pragma unroll 1
    for (int k = 0; k < nmine; ++k) {
      const int sp = c + k * P;
      QRows rq = query_rows<SRC_SPARSE_DEC, DecRows<KV8>::SROWB>(a.src, a.win_len, nullptr, nullptr, 1, qi, sp,
                                                                   a.slots, SR);
      rq.n_rows = nrow[k];
      f32x4_t o[16];
      float m_ref, l_run;
      dec_tiles<SRC_SPARSE_DEC, KV8>(rq, tab + k * SR, ring, xchg, qb, a.scale_log2, o, m_ref, l_run);
      // ---- partials (unnormalised, exponent base 2), device-coherent
      l_run += shfl_xor(l_run, 16);
      l_run += shfl_xor(l_run, 32);
      int dbase = dh * 256 + l16;
      // opaque to the compiler: the stores' addresses are formed here, not
      // hoisted out of the loop over splits (64 of them would not fit in
      // registers beside the tile loop's)
      asm volatile("" : "+v"(dbase));
      if (nsplit > 1) {
        const int64_t pbase = (qi * nsplit + sp) * (int64_t)H;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = hg * 16 + G * 4 + r;
          if (h >= H) continue;
#pragma unroll
          for (int nt = 0; nt < 16; ++nt) st_coh(&a.part_o[(pbase + h) * D + dbase + nt * 16], o[nt][r]);
        }
        if (dh == 0 && G == 0 && head < H) {
          st_coh(&a.part_ml[(pbase + head) * 2 + 0], m_ref);
          st_coh(&a.part_ml[(pbase + head) * 2 + 1], l_run);
        }
      } else {
        float rope_c = 1.0f, rope_s = 0.0f;
        if ((a.qk_flags & 2) && l < a.qk_R / 2) rope_cs((double)a.q_pos[qi], l, a.qk_R, a.qk_log2_theta, rope_c, rope_s);
        // one split: normalise here, as the separate kernel does
        float mrr[4], lrr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mrr[r] = __shfl(m_ref, G * 4 + r, 64);
          lrr[r] = __shfl(l_run, G * 4 + r, 64);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = hg * 16 + G * 4 + r;
          if (h >= H) continue;
          const float s2 = a.sink ? a.sink[h] * LOG2E_F : -INFINITY;
          const float Mx = fmaxf(mrr[r], s2);
          float fac = 0.0f;
          if (Mx != -INFINITY) {
            const float e = exp2f(mrr[r] - Mx);
            fac = e / (lrr[r] * e + exp2f(s2 - Mx));
          }
#pragma unroll
          for (int nt = 0; nt < 16; ++nt) {
            const int64_t oo = (qi * H + h) * (int64_t)D + dbase + nt * 16;
            float v = o[nt][r] * fac;
            if ((a.qk_flags & 2) && dh * 256 + nt * 16 + 16 > D - a.qk_R) {
              // the inverse rotation: the pair's other dim is in the lane next
              // door; lane i < R/2 formed pair i's angle (rope_l)
              const int d = dbase + nt * 16, s0 = D - a.qk_R;
              const float other = shfl_xor(v, 1);
              const int src = d >= s0 ? (d - s0) >> 1 : 0;
              const float c2 = __shfl(rope_c, src, 64), sn = __shfl(rope_s, src, 64);
              if (d >= s0) v = (l16 & 1) ? v * c2 - other * sn : v * c2 + other * sn;
            }
            if (a.out_dt == DT_BF16)
              reinterpret_cast<uint16_t*>(a.out)[oo] = (uint16_t)f32_to_bf16(v);
            else
              reinterpret_cast<float*>(a.out)[oo] = v;
          }
        }
        if (a.lse && dh == 0 && G == 0 && head < H) {
          const float s2 = a.sink ? a.sink[head] * LOG2E_F : -INFINITY;
          const float Mx = fmaxf(m_ref, s2);
          float v = -INFINITY;
          if (Mx != -INFINITY) v = (Mx + log2f(l_run * exp2f(m_ref - Mx) + exp2f(s2 - Mx))) * LN2_F;
          a.lse[qi * H + head] = v;
        }
      }
      __syncthreads();  // the ring is free for the next split
    }
  }
merge:
  if (nsplit == 1) return;

  // ---- 4. merge: one wave per head (its 512 dims, eight per lane), every
  // split's partial in one round of device-coherent loads, then the same
  // arithmetic in split order as the separate merge kernel
  {
    arrive(&a.sync[qi * 2 + 1]);
    const uint32_t got = wait_for(&a.sync[qi * 2 + 1], (uint32_t)P, &res[7]);
    const bool ok = got >= (uint32_t)P && got < dtl::FAILED;
    constexpr int U1 = dtl::MAX_SPLITS;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        a.part_o + qi * nsplit * (int64_t)H * D, (short)0, (int)(nsplit * H * D * 4), BUF_RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        a.part_ml + qi * nsplit * (int64_t)H * 2, (short)0, (int)(nsplit * H * 2 * 4), BUF_RSRC_WORD3);
    const int d = l * 8;  // this lane's eight dims
    float rope_c = 1.0f, rope_s = 0.0f;
    if ((a.qk_flags & 2) && l < a.qk_R / 2 && c * NW < H)
      rope_cs((double)a.q_pos[qi], l, a.qk_R, a.qk_log2_theta, rope_c, rope_s);
    for (int h = c * NW + w; h < H; h += P * NW) {
      const float s2 = a.sink ? a.sink[h] * LOG2E_F : -INFINITY;
      float mv[U1], lv[U1];
      float v[U1][8];
#pragma unroll
      for (int u = 0; u < U1; ++u) {
        const bool in = u < nsplit;
        const int pb = u * H + h;  // partial (qi, u, h)
        if (in) {
          const u32x2_t ml =
              __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rm, pb * 8, 0, dtl::SC1));
          mv[u] = __uint_as_float(ml[0]);
          lv[u] = __uint_as_float(ml[1]);
#pragma unroll
          for (int hv = 0; hv < 2; ++hv) {
            const f32x4_t r = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, (pb * D + d + 4 * hv) * 4, 0, dtl::SC1));
#pragma unroll
            for (int i = 0; i < 4; ++i) v[u][4 * hv + i] = r[i];
          }
        } else {
          mv[u] = -INFINITY;
          lv[u] = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
        }
      }
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
      float Mx = s2, Z = 0.0f;
#pragma unroll
      for (int u = 0; u < U1; ++u) Mx = fmaxf(Mx, mv[u]);
      if (Mx != -INFINITY) {
        Z = exp2f(s2 - Mx);
#pragma unroll
        for (int u = 0; u < U1; ++u) {
          const float e = exp2f(mv[u] - Mx);  // 0 for an empty or absent split (m = -inf)
          Z += lv[u] * e;
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += v[u][q] * e;
        }
      }
      const float inv = ok ? ((Mx != -INFINITY) ? 1.0f / Z : 0.0f) : __builtin_nanf("");
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] *= inv;
      if (a.qk_flags & 2) {
        // the output's inverse rotation, pairs inside the lane's 8 dims (all
        // lanes shuffle; lane i < R/2 formed pair i's angle before the loop)
#pragma unroll
        for (int q = 0; q < 8; q += 2) {
          const bool rot = d + q >= D - a.qk_R;
          const int src = rot ? (d + q - (D - a.qk_R)) >> 1 : 0;
          const float c2 = __shfl(rope_c, src, 64), sn = __shfl(rope_s, src, 64);
          if (rot) {
            const float x0 = acc[q], x1 = acc[q + 1];
            acc[q] = x0 * c2 + x1 * sn;
            acc[q + 1] = x1 * c2 - x0 * sn;
          }
        }
      }
      const int64_t oo = (qi * H + h) * (int64_t)D + d;
      if (a.out_dt == DT_BF16) {
        const u32x4_t wv = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                            pack_bf16x2(acc[6], acc[7])};
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(a.out) + oo) = wv;
      } else {
        float* op = reinterpret_cast<float*>(a.out) + oo;
        *reinterpret_cast<f32x4_t*>(op) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4_t*>(op + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
      }
      if (a.lse && l == 0)
        a.lse[qi * H + h] = !ok ? __builtin_nanf("") : (Mx != -INFINITY) ? (Mx + log2f(Z)) * LN2_F : -INFINITY;
    }
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
constexpr int DT_MAX_DEVICES = 64;

static size_t r256(size_t x) { return (x + 255) & ~size_t(255); }

// Workgroups per query and filter passes, or false when the fused launch
// does not apply (then the caller runs the separate kernels).
static bool tail_plan(int64_t nq, int64_t N_max, int top_k, int split_rows, int nsplit, int* P_out,
                      int* passes_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= DT_MAX_DEVICES) return false;
  static int resident_dev[DT_MAX_DEVICES] = {};
  int& resident = resident_dev[dev];
  if (resident == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, csa_decode_tail_kernel<false>, dtl::NT, 0) != hipSuccess)
      return false;
    int per8 = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per8, csa_decode_tail_kernel<true>, dtl::NT, 0) != hipSuccess)
      return false;
    // one workgroup per CU (the LDS allows no second), so the grid may not
    // exceed the CU count: then every workgroup of it runs at once
    resident = std::max(1, std::min({per, per8, 1}) * cus);
  }
  if (nq <= 0 || nq > resident || nsplit > dtl::MAX_SPLITS || top_k > 4096) return false;
  const int64_t chunks = std::max<int64_t>(1, (N_max + dtl::FCH - 1) / dtl::FCH);
  const int64_t P = std::min<int64_t>(chunks, resident / nq);
  if (P < 1) return false;
  const int64_t passes = (chunks + P - 1) / P;
  const int64_t nmine = (nsplit + P - 1) / P;
  if (nmine * split_rows > bfk::TAB_MAX || nmine > dtl::MAX_SPLITS) return false;
  *P_out = (int)P;
  *passes_out = (int)passes;
  return true;
}

bool decode_tail_applies(int64_t nq, int64_t N_max, int top_k, int slots, int split_rows, int nsplit, int kv_dt) {
  int P = 0, passes = 0;
  (void)slots;
  return (kv_dt == DT_BF16 || kv_dt == DT_KV_FP8) && tail_plan(nq, N_max, top_k, split_rows, nsplit, &P, &passes);
}

size_t decode_tail_ws_bytes(int64_t nq, int64_t N_max, int top_k, int H, int D, int slots, int split_rows,
                            int nsplit) {
  (void)top_k;
  const int64_t nseg = std::max<int64_t>(1, (N_max + dtl::FCH - 1) / dtl::FCH) * dtl::NW + dtl::NW;
  return r256((size_t)nq * 2 * 4) + r256((size_t)nq * BINS * 4) + r256((size_t)nq * nseg * 4) +
         2 * r256((size_t)nq * nseg * dtl::WCAP * 4) + r256((size_t)nq * nsplit * H * D * 4) +
         r256((size_t)nq * nsplit * H * 2 * 4) + (size_t)0 * (slots + split_rows);
}

size_t decode_tail_zero_bytes(int64_t nq) { return r256((size_t)nq * 2 * 4) + (size_t)nq * BINS * 4; }

hipError_t run_decode_tail(const DecodeTailLaunch& L, hipStream_t st, bool* launched) {
  *launched = false;
  int P = 0, passes = 0;
  if (!tail_plan(L.nq, L.N_max, L.top_k, L.split_rows, L.nsplit, &P, &passes)) return hipSuccess;
  if (L.kv_dt != DT_BF16 && L.kv_dt != DT_KV_FP8) return hipSuccess;
  TailArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(L.q);
  a.src.kv_comp = reinterpret_cast<const uint8_t*>(L.kv_comp);
  a.src.kv_win = reinterpret_cast<const uint8_t*>(L.kv_win);
  a.src.idx = nullptr;
  a.src.N_max = L.N_max;
  a.src.T_tok = 0;
  a.src.top_k = L.top_k;
  a.src.W = L.W;
  a.src.Tq = L.Tq;
  a.src.Wb = L.W + L.Tq - 1;
  a.win_len = L.W > 0 ? L.win_len : nullptr;
  a.sink = L.sink;
  a.scale_log2 = L.scale * LOG2E_F;
  a.H = L.H;
  a.slots = L.slots;
  a.split_rows = L.split_rows;
  a.nsplit = L.nsplit;
  a.out = L.out;
  a.lse = L.lse;
  a.out_dt = L.out_dt;
  a.scores = L.scores;
  a.q_pos = L.q_pos;
  a.n_comp = L.n_comp;
  a.m = L.m;
  a.top_k = L.top_k;
  a.hint = L.hint;
  a.out_idx = L.out_idx;
  a.out_score = L.out_score;
  a.qk_flags = L.qk_flags;
  a.qk_gamma = L.qk_gamma;
  a.qk_eps = L.qk_eps;
  a.qk_R = L.qk_R;
  a.qk_log2_theta = L.qk_flags ? log2((double)L.qk_theta) : 0.0;
  const int64_t nseg = std::max<int64_t>(1, (L.N_max + dtl::FCH - 1) / dtl::FCH) * dtl::NW + dtl::NW;
  uint8_t* w = reinterpret_cast<uint8_t*>(L.ws);
  a.sync = reinterpret_cast<uint32_t*>(w);
  w += r256((size_t)L.nq * 2 * 4);
  a.sub = reinterpret_cast<uint32_t*>(w);
  w += r256((size_t)L.nq * BINS * 4);
  a.wcnt = reinterpret_cast<int32_t*>(w);
  w += r256((size_t)L.nq * nseg * 4);
  a.wkey = reinterpret_cast<uint32_t*>(w);
  w += r256((size_t)L.nq * nseg * dtl::WCAP * 4);
  a.widx = reinterpret_cast<int32_t*>(w);
  w += r256((size_t)L.nq * nseg * dtl::WCAP * 4);
  a.part_o = reinterpret_cast<float*>(w);
  w += r256((size_t)L.nq * L.nsplit * L.H * 512 * 4);
  a.part_ml = reinterpret_cast<float*>(w);
  a.nseg = (int)nseg;
  a.passes = passes;
  const dim3 grid((unsigned)P, (unsigned)L.nq);
  if (L.kv_dt == DT_KV_FP8)
    hipLaunchKernelGGL(csa_decode_tail_kernel<true>, grid, dim3(dtl::NT), 0, st, a);
  else
    hipLaunchKernelGGL(csa_decode_tail_kernel<false>, grid, dim3(dtl::NT), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) *launched = true;
  return e;
}

}  // namespace csa
