// Device-side helpers shared by the gfx950 kernels: vector types, bf16 and
// fp8 conversions, MFMA wrappers, wave shuffles.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

// dtype tags (match the ABI codes)
enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round-to-nearest-even fp32 -> bf16 bits; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Unpack 8 bf16 held in a 16-byte vector to fp32.
__device__ __forceinline__ void unpack_bf16x8(u32x4_t v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// 4 OCP E4M3 codes (one dword) -> 4 bf16 (two dwords), exact: every E4M3
// value is a bf16 value. The hardware converter goes through fp32; dropping
// the low 16 bits of those fp32 values loses nothing (3 mantissa bits).
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t codes) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
  u32x2_t r;
  r[0] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
  r[1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
  return r;
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Order-preserving map fp32 -> uint32 (larger float <=> larger key); -0 and
// +0 share one key. NaN maps above +inf (positive NaN) or below -inf.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
