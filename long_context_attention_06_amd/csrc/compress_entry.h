// Device code of the compression (entry i of a sequence as the softmax(Z+B)-
// weighted sum of its block, plus the overlap branch over block i-1): DeepSeek
// V4 脱离 CUDA 全栈国产化 (deepseek.csdn.net), section 二, CSA step 1, the CComp_i
// equation. Shared by the compression kernels and by the decode scan, whose
// launch can carry a decode step's compression as extra workgroups.
#pragma once
#include "common.h"

namespace csa {

// Arguments of one compression launch (validated by the caller).
struct CompressArgs {
  const void *Ca, *Cb, *Za, *Zb;
  const float *Ba, *Bb;
  void* out;
  int64_t B, n_rows, tok_begin, blk_begin, nblk, out_cap;
  int d, m;
  int overlap, joint;
};

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t off, float* f) {
  if constexpr (DT == DT_BF16) {
    unpack_bf16x8(ld16(reinterpret_cast<const uint16_t*>(base) + off), f);
  } else {
    const float* p = reinterpret_cast<const float*>(base) + off;
    f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = a[e];
      f[4 + e] = b[e];
    }
  }
}

// fp32 -> OCP E4M3 (FN) code, round to nearest even, saturating at +-448
// (the format has no infinity): 3 mantissa bits kept from the binary32 bit
// pattern, the exponent rebiased from 127 to 7; below 2^-6 the grid is the
// subnormal step 2^-9 (a rounded multiple of 8 is the smallest normal).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t ua = __float_as_uint(a);
    const uint32_t lsb = (ua >> 20) & 1u;
    code = ((ua + 0x7ffffu + lsb) >> 20) - (120u << 3);
  }
  return code | sign;
}

// Stores 8 channels c0 .. c0+7 of one entry. Mixed-precision KV rows (d - 64
// E4M3 bytes, then the 64 RoPE channels as bf16: d + 64 bytes) take E4M3 or
// bf16 by the channels' side of d - 64 (a multiple of 8).
template <int OUT_DT>
__device__ __forceinline__ void store8(void* out, int64_t row, int d, int c0, const float* res) {
  if constexpr (OUT_DT == DT_BF16) {
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(res[2 * e], res[2 * e + 1]);
    st16(reinterpret_cast<uint16_t*>(out) + row * d + c0, v);
  } else if constexpr (OUT_DT == DT_KV_FP8) {
    uint8_t* orow = reinterpret_cast<uint8_t*>(out) + row * (int64_t)(d + 64);
    const int nope = d - 64;
    if (c0 < nope) {
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        w[h] = f32_to_e4m3(res[4 * h]) | (f32_to_e4m3(res[4 * h + 1]) << 8) | (f32_to_e4m3(res[4 * h + 2]) << 16) |
               (f32_to_e4m3(res[4 * h + 3]) << 24);
      *reinterpret_cast<u32x2_t*>(orow + c0) = u32x2_t{w[0], w[1]};
    } else {
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(res[2 * e], res[2 * e + 1]);
      *reinterpret_cast<u32x4_t*>(orow + nope + 2 * (c0 - nope)) = v;
    }
  } else {
    float* p = reinterpret_cast<float*>(out) + row * d + c0;
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{res[0], res[1], res[2], res[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{res[4], res[5], res[6], res[7]};
  }
}

struct SoftAcc {
  float mx[8], sm[8], acc[8];
  __device__ void init() {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mx[e] = -INFINITY;
      sm[e] = 0.f;
      acc[e] = 0.f;
    }
  }
  // feed up to 4 tokens at once: z2 in the exp2 domain
  template <int NTOK>
  __device__ void feed(const float (*z2)[8], const float (*c)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float gm = z2[0][e];
#pragma unroll
      for (int t = 1; t < NTOK; ++t) gm = fmaxf(gm, z2[t][e]);
      const float nm = fmaxf(mx[e], gm);
      const float a = exp2f(mx[e] - nm);  // 0 on the first group
      float s = sm[e] * a, v = acc[e] * a;
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        const float p = exp2f(z2[t][e] - nm);
        s += p;
        v += p * c[t][e];
      }
      mx[e] = nm;
      sm[e] = s;
      acc[e] = v;
    }
  }
};

template <int IN_DT>
__device__ __forceinline__ void feed_block(SoftAcc& S, const void* Cx, const void* Zx, const float* Bx, int64_t row0,
                                           int d, int m, int c0) {
  // rows row0 .. row0+m-1 of [*, d] tensors; bias rows 0..m-1
  int j = 0;
  for (; j + 4 <= m; j += 4) {
    float z[4][8], c[4][8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      load8<IN_DT>(Zx, (row0 + j + t) * d + c0, z[t]);
      load8<IN_DT>(Cx, (row0 + j + t) * d + c0, c[t]);
      const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(Bx + (int64_t)(j + t) * d + c0);
      const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(Bx + (int64_t)(j + t) * d + c0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[t][e] = (z[t][e] + b0[e]) * LOG2E_F;
        z[t][4 + e] = (z[t][4 + e] + b1[e]) * LOG2E_F;
      }
    }
    S.feed<4>(z, c);
  }
  for (; j < m; ++j) {
    float z[1][8], c[1][8];
    load8<IN_DT>(Zx, (row0 + j) * d + c0, z[0]);
    load8<IN_DT>(Cx, (row0 + j) * d + c0, c[0]);
    const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(Bx + (int64_t)j * d + c0);
    const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(Bx + (int64_t)j * d + c0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[0][e] = (z[0][e] + b0[e]) * LOG2E_F;
      z[0][4 + e] = (z[0][4 + e] + b1[e]) * LOG2E_F;
    }
    S.feed<1>(z, c);
  }
}

// Raw inputs of four tokens of one block (8 channels each), loaded before
// any arithmetic so that the loads of several blocks overlap.
template <int IN_DT>
struct Raw4 {
  float z[4][8], c[4][8], b[4][8];
  __device__ void load(const void* Cx, const void* Zx, const float* Bx, int64_t row0, int j, int d, int c0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      load8<IN_DT>(Zx, (row0 + j + t) * d + c0, z[t]);
      load8<IN_DT>(Cx, (row0 + j + t) * d + c0, c[t]);
      const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(Bx + (int64_t)(j + t) * d + c0);
      const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(Bx + (int64_t)(j + t) * d + c0 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        b[t][e] = b0[e];
        b[t][4 + e] = b1[e];
      }
    }
  }
  __device__ void feed(SoftAcc& S) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) z[t][e] = (z[t][e] + b[t][e]) * LOG2E_F;
    S.feed<4>(z, c);
  }
};

struct CompressLaunch;
CompressArgs compress_args(const CompressLaunch& a);  // host: the launch's kernel arguments

// One thread computes 8 channels of one entry: thread gid < B * nblk * d/8.
template <int IN_DT, int OUT_DT>
__device__ __forceinline__ void compress_entry(const CompressArgs& a, int64_t gid) {
  const void *Ca = a.Ca, *Cb = a.Cb, *Za = a.Za, *Zb = a.Zb;
  const float *Ba = a.Ba, *Bb = a.Bb;
  const int64_t n_rows = a.n_rows, tok_begin = a.tok_begin, blk_begin = a.blk_begin, nblk = a.nblk;
  const int d = a.d, m = a.m;
  const bool overlap = a.overlap, joint = a.joint;
  const int groups = d / 8;
  const int64_t total = a.B * nblk * groups;
  if (gid >= total) return;
  const int cg = (int)(gid % groups);
  const int64_t t = gid / groups;
  const int64_t i = blk_begin + t % nblk;
  const int64_t b = t / nblk;
  const int c0 = cg * 8;

  SoftAcc A, Bs;
  A.init();
  const int64_t rowa = b * n_rows + (m * i - tok_begin);
  float res[8];
  const bool has_b = overlap && i >= 1;
  if (m == 4) {
    // one group per block: both blocks' loads go out before any arithmetic.
    // Without a previous block (no overlap branch, where Cb, Zb, Bb may be
    // null, or block 0) the second load repeats block i of Ca, Za, Ba, unused.
    Raw4<IN_DT> ra, rb;
    ra.load(Ca, Za, Ba, rowa, 0, d, c0);
    rb.load(has_b ? Cb : Ca, has_b ? Zb : Za, has_b ? Bb : Ba, has_b ? rowa - m : rowa, 0, d, c0);
    ra.feed(A);
    if (has_b && joint) {
      rb.feed(A);
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = A.acc[e] / A.sm[e];
    } else if (has_b) {
      Bs.init();
      rb.feed(Bs);
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = A.acc[e] / A.sm[e] + Bs.acc[e] / Bs.sm[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = A.acc[e] / A.sm[e];
    }
  } else if (has_b) {
    feed_block<IN_DT>(A, Ca, Za, Ba, rowa, d, m, c0);
    const int64_t rowb = b * n_rows + (m * (i - 1) - tok_begin);
    if (joint) {
      feed_block<IN_DT>(A, Cb, Zb, Bb, rowb, d, m, c0);
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = A.acc[e] / A.sm[e];
    } else {
      Bs.init();
      feed_block<IN_DT>(Bs, Cb, Zb, Bb, rowb, d, m, c0);
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = A.acc[e] / A.sm[e] + Bs.acc[e] / Bs.sm[e];
    }
  } else {
    feed_block<IN_DT>(A, Ca, Za, Ba, rowa, d, m, c0);
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] = A.acc[e] / A.sm[e];
  }
  store8<OUT_DT>(a.out, b * a.out_cap + i, d, c0, res);
}


// One single-branch entry (no overlap term), computed by a whole workgroup of
// NT threads: thread (slice sl, channel group g) runs the online softmax of
// its 8 channels over tokens sl * 4 + 4 * SL * k .. +3 of the block (SL =
// NT / (d / 8) slices), and the slices' (max, sum, weighted sum) merge in
// slice order through `scratch` (3 * SL * d floats of LDS). Entry row orow of
// out gets it. Used where a decode step's append rides in the attention's
// launch.
template <int IN_DT, int OUT_DT, int NT>
__device__ void block_entry_wg(const void* Ca, const void* Za, const float* Ba, int64_t row0, int d, int m,
                               void* out, int64_t orow, float* scratch) {
  const int groups = d / 8;
  const int SL = NT / groups;  // d = 512: 8 slices
  const int tid = threadIdx.x;
  const int g = tid % groups, sl = tid / groups;
  const int c0 = g * 8;
  SoftAcc A;
  A.init();
  if (sl < SL) {
    for (int j0 = sl * 4; j0 < m; j0 += SL * 4) {
      float z[4][8], c[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = min(j0 + u, m - 1);  // a repeated token is masked below
        load8<IN_DT>(Za, (row0 + j) * d + c0, z[u]);
        load8<IN_DT>(Ca, (row0 + j) * d + c0, c[u]);
        const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(Ba + (int64_t)j * d + c0);
        const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(Ba + (int64_t)j * d + c0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[u][e] = j0 + u < m ? (z[u][e] + b0[e]) * LOG2E_F : -INFINITY;
          z[u][4 + e] = j0 + u < m ? (z[u][4 + e] + b1[e]) * LOG2E_F : -INFINITY;
        }
      }
      A.feed<4>(z, c);  // token j0 < m is in the group: its maximum is finite
    }
    float* pm = scratch;
    float* ps = scratch + SL * d;
    float* pa = scratch + 2 * SL * d;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pm[sl * d + c0 + e] = A.mx[e];
      ps[sl * d + c0 + e] = A.sm[e];
      pa[sl * d + c0 + e] = A.acc[e];
    }
  }
  __syncthreads();
  if (tid < groups) {
    float res[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = c0 + e;
      float mx = -INFINITY;
      for (int q = 0; q < SL; ++q) mx = fmaxf(mx, scratch[q * d + ch]);
      float sm = 0.f, acc = 0.f;
      for (int q = 0; q < SL; ++q) {
        const float v = scratch[q * d + ch];
        const float a = v == -INFINITY ? 0.f : exp2f(v - mx);
        sm += scratch[(SL + q) * d + ch] * a;
        acc += scratch[(2 * SL + q) * d + ch] * a;
      }
      res[e] = acc / sm;
    }
    store8<OUT_DT>(out, orow, d, c0, res);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the entry is written before the barrier releases readers
  __syncthreads();
}

}  // namespace csa
