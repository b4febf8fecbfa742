// QK RMSNorm and partial rotary position encoding for gfx950.
//
// DeepSeek V4 脱离 CUDA 全栈国产化 (deepseek.csdn.net), section 二, 其他辅助设计:
// queries and keys are RMS-normalised before the core attention, and rotary
// position encoding is applied to the last 64 dims only. liduos.com
// "deepseek-v4-engineering-tradeoffs", 1M Context 的结构与取舍: because each
// row serves as both key and value, the attention output takes the inverse
// rotation. One op covers the three: RMSNorm, then a rotation by the
// position (the query/key prologue), or the inverse rotation (the output
// epilogue).
//
// One wave per row of D <= 512 values, 8 consecutive values per lane: the
// row's sum of squares is a wave reduction; the rotated pairs are
// (D-R+2i, D-R+2i+1), which never straddle a lane's 8 values. Angles
// p * theta^(-2i/R) are formed and reduced in double precision (in fp32 the
// product alone is off by up to 0.06 rad at p = 2^20), one pair per lane, and
// reach the lanes that rotate by a shuffle; the rotation itself runs in fp32.
#include "common.h"
#include "kernels.h"

namespace csa {

template <int DT>
__global__ void __launch_bounds__(256)
norm_rope_kernel(const void* __restrict__ x, void* __restrict__ out, const float* __restrict__ gamma,
                 const int32_t* __restrict__ pos, int64_t rows, int H, int D, int R, float eps, double log2_theta,
                 int flags) {
  const int l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int c0 = 8 * l;
  const bool live = c0 < D;
  const int64_t base = row * D + c0;
  float v[8];
  if (DT == DT_BF16) {
    const u32x4_t u = live ? ld16(reinterpret_cast<const uint16_t*>(x) + base) : u32x4_t{0, 0, 0, 0};
    unpack_bf16x8(u, v);
  } else {
    const float* p = reinterpret_cast<const float*>(x) + base;
    const f32x4_t a = live ? *reinterpret_cast<const f32x4_t*>(p) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const f32x4_t b = live ? *reinterpret_cast<const f32x4_t*>(p + 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
  if (flags & NR_NORM) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= r * (gamma && live ? gamma[c0 + e] : 1.0f);
  }
  const int s0 = D - R;  // first rotated dim
  if (flags & (NR_ROPE | NR_ROPE_INV)) {
    // pair i's angle, one pair per lane in rounds of 64 (R/2 pairs), handed
    // to the lane that holds the pair by a lane shuffle
    const double p = (double)pos[row / H] * ((flags & NR_ROPE_INV) ? -1.0 : 1.0);
    for (int base = 0; base < R / 2; base += 64) {
      float cs_l = 1.0f, sn_l = 0.0f;
      if (base + l < R / 2) {
        double sn, cs;
        sincos(p * exp2(-2.0 * (double)(base + l) / (double)R * log2_theta), &sn, &cs);
        cs_l = (float)cs;
        sn_l = (float)sn;
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int i = (c0 + e - s0) >> 1;  // this lane's pair (negative: not rotated)
        const bool mine = live && c0 + e >= s0 && i >= base && i < base + 64;
        const int src = mine ? i - base : l;
        const float c = __shfl(cs_l, src, 64), s = __shfl(sn_l, src, 64);
        if (mine) {
          const float a = v[e], b = v[e + 1];
          v[e] = a * c - b * s;
          v[e + 1] = a * s + b * c;
        }
      }
    }
  }
  if (!live) return;
  if (DT == DT_BF16) {
    u32x4_t u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    st16(reinterpret_cast<uint16_t*>(out) + base, u);
  } else {
    float* p = reinterpret_cast<float*>(out) + base;
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

hipError_t run_norm_rope(const NormRopeLaunch& a, hipStream_t st) {
  const int64_t rows = a.T * a.H;
  if (rows == 0) return hipSuccess;
  const int64_t grid = (rows + 3) / 4;
  const double l2t = log2((double)a.theta);
  if (a.dt == DT_BF16)
    hipLaunchKernelGGL(norm_rope_kernel<DT_BF16>, dim3((unsigned)grid), dim3(256), 0, st, a.x, a.out, a.gamma,
                       a.pos, rows, a.H, a.D, a.R, a.eps, l2t, a.flags);
  else
    hipLaunchKernelGGL(norm_rope_kernel<DT_F32>, dim3((unsigned)grid), dim3(256), 0, st, a.x, a.out, a.gamma, a.pos,
                       rows, a.H, a.D, a.R, a.eps, l2t, a.flags);
  return hipGetLastError();
}

}  // namespace csa
