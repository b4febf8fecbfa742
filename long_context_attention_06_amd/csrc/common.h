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
typedef int i32x2_t __attribute__((ext_vector_type(2)));

#define LOG2E_F 1.4426950408889634f
#define LN2_F 0.6931471805599453f

// dtype tags (match the ABI codes)
enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP4 = 3, DT_KV_FP8 = 4 };

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (v_cvt_pk_bf16_f32 on gfx950); NaN
// stays NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
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

// 2 OCP E4M3 codes (the low or high 16 bits of a dword) -> 2 bf16 in one
// instruction (gfx950 scaled convert, scale 1.0), exact.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t codes, bool high) {
  return __builtin_bit_cast(uint32_t, high ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false));
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

// Cross-lane steps on DPP (data-parallel primitives, GFX9 encoding): a VALU
// operand modifier, so no LDS round trip as with ds_bpermute-based shuffles.
// Rows are groups of 16 lanes.
template <int CTRL, int ROW_MASK = 0xf, bool BOUND_ZERO = false>
__device__ __forceinline__ int dpp_mov(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, BOUND_ZERO);
}
enum : int { DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118,
             DPP_ROW_ROR1 = 0x121, DPP_ROW_ROR2 = 0x122, DPP_ROW_ROR4 = 0x124, DPP_ROW_ROR8 = 0x128,
             DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143 };

// Inclusive prefix sum over the 64 lanes: Hillis-Steele within each row, then
// the rows' totals carried by row broadcasts.
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += dpp_mov<DPP_ROW_SHR1, 0xf, true>(0, v);
  v += dpp_mov<DPP_ROW_SHR2, 0xf, true>(0, v);
  v += dpp_mov<DPP_ROW_SHR4, 0xf, true>(0, v);
  v += dpp_mov<DPP_ROW_SHR8, 0xf, true>(0, v);
  v += dpp_mov<DPP_ROW_BCAST15, 0xa>(0, v);
  v += dpp_mov<DPP_ROW_BCAST31, 0xc>(0, v);
  return v;
}

// Sum over the four 16-lane rows of a wave, per column: lane l gets
// x[l%16] + x[l%16 + 16] + x[l%16 + 32] + x[l%16 + 48]. gfx950's permlane
// swaps exchange rows as plain VALU operations (no LDS round trip).
__device__ __forceinline__ float sum_rows16(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Wave-wide reductions, result uniform (rotations within rows, then the four
// rows' values read as scalars).
__device__ __forceinline__ int wave_sum_dpp(int v) {
  v += dpp_mov<DPP_ROW_ROR8>(v, v);
  v += dpp_mov<DPP_ROW_ROR4>(v, v);
  v += dpp_mov<DPP_ROW_ROR2>(v, v);
  v += dpp_mov<DPP_ROW_ROR1>(v, v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ uint32_t wave_min_u32_dpp(uint32_t v) {
  v = min(v, (uint32_t)dpp_mov<DPP_ROW_ROR8>((int)v, (int)v));
  v = min(v, (uint32_t)dpp_mov<DPP_ROW_ROR4>((int)v, (int)v));
  v = min(v, (uint32_t)dpp_mov<DPP_ROW_ROR2>((int)v, (int)v));
  v = min(v, (uint32_t)dpp_mov<DPP_ROW_ROR1>((int)v, (int)v));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  v = max(v, (uint32_t)dpp_mov<DPP_ROW_ROR8>((int)v, (int)v));
  v = max(v, (uint32_t)dpp_mov<DPP_ROW_ROR4>((int)v, (int)v));
  v = max(v, (uint32_t)dpp_mov<DPP_ROW_ROR2>((int)v, (int)v));
  v = max(v, (uint32_t)dpp_mov<DPP_ROW_ROR1>((int)v, (int)v));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// max(0, x) in one integer max on the bit pattern: negative floats (and -0)
// are negative integers; positive values pass unchanged.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ---- HBM -> LDS without registers (global_load_lds, issued from inline asm so
// the compiler's own load tracking never waits on it; the caller waits with
// explicit vmcnt counts). Vector memory stores also count in vmcnt and may
// complete out of order with loads: a loop that relies on these counts issues
// no stores while loads are in flight.
//
// 16 bytes per lane: lane i copies bytes base+voff .. +15 to lds_addr + 16 i.
__device__ __forceinline__ void dma_row(const uint8_t* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}
// 4 bytes per lane: lane i copies bytes base+voff .. +3 to lds_addr + 4 i.
__device__ __forceinline__ void dma_dword(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}
// Wait until at most N vector memory operations of this wave are in flight
// and every LDS access of this wave is done, then join the workgroup.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const T*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
// Third dword of a raw (untyped) buffer descriptor on gfx9: 32-bit data format.
constexpr int BUF_RSRC_WORD3 = 0x00020000;
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Order-preserving map fp32 -> uint32 (larger float <=> larger key); -0 and
// +0 share one key. NaN maps above +inf (positive NaN) or below -inf.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
