// CSA / HCA KV compression for gfx950.
//
// Computes the compression equation of DeepSeek V4 脱离 CUDA 全栈国产化
// (deepseek.csdn.net, section 二, CSA step 1, the CComp_i equation): entry i
// of a sequence is, per channel, a softmax-weighted sum of the m candidate
// values of block i (logits Z_a plus the positional bias B_a) plus, with the
// overlap branch, a second softmax-weighted sum over block i-1 (Z_b + B_b,
// C_b). Tokens after the last complete block form no entry (m.lqnn.cn
// "Deepseek-V4 技术报告里最值得复现的三个改动", section 5).
//
// The op is a pure HBM stream: every input element is read once. One thread
// owns 8 consecutive channels of one entry, so a wave reads whole 1 KiB rows
// with 16-byte loads. The softmax runs online over the block in groups of
// four tokens (one rescale per group), in fp32 and the exp2 domain.
#include "common.h"
#include "kernels.h"

namespace csa {

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

template <int IN_DT, int OUT_DT>
__global__ void __launch_bounds__(256)
compress_kernel(const void* __restrict__ Ca, const void* __restrict__ Cb, const void* __restrict__ Za,
                const void* __restrict__ Zb, const float* __restrict__ Ba, const float* __restrict__ Bb,
                void* __restrict__ out, int64_t B, int64_t n_rows, int64_t tok_begin, int64_t blk_begin,
                int64_t nblk, int64_t out_cap, int d, int m, int overlap, int joint) {
  const int groups = d / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = B * nblk * groups;
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
  store8<OUT_DT>(out, b * out_cap + i, d, c0, res);
}

// Single-branch compression with long blocks (HCA, m' = 128): a thread per
// 8 channels would walk all m tokens one group after another, so a decode
// step (one block per sequence) would wait for m/4 dependent load rounds.
// Here 16 threads split a block's tokens, 8 each, with all their loads issued
// before any arithmetic; each keeps an online-softmax partial (max, sum,
// weighted sum) per channel, and the 16 partials of a channel are merged
// through LDS in slice order. A workgroup covers 16 channel groups (128
// channels) of one block; lanes run along the channels, so a wave reads 256
// contiguous bytes of four token rows.
constexpr int CS_TOK = 8;    // tokens per slice
constexpr int CS_SL = 16;    // slices per workgroup pass
constexpr int CS_CG = 16;    // channel groups per workgroup

template <int IN_DT, int OUT_DT>
__global__ void __launch_bounds__(256)
compress_split_kernel(const void* __restrict__ Ca, const void* __restrict__ Za, const float* __restrict__ Ba,
                      void* __restrict__ out, int64_t n_rows, int64_t tok_begin, int64_t blk_begin, int64_t nblk,
                      int64_t out_cap, int d, int m) {
  __shared__ float part[3][CS_SL][CS_CG * 8];  // max, sum, weighted sum (exp2 domain)
  const int groups = d / 8;
  const int cgb = (groups + CS_CG - 1) / CS_CG;  // workgroups per block
  const int cgl = threadIdx.x % CS_CG, sl = threadIdx.x / CS_CG;
  const int cg = (int)(blockIdx.x % cgb) * CS_CG + cgl;
  const int64_t t = blockIdx.x / cgb;
  const int64_t i = blk_begin + t % nblk;
  const int64_t b = t / nblk;
  const bool live = cg < groups;
  const int c0 = live ? cg * 8 : 0;
  const int64_t row0 = b * n_rows + (m * i - tok_begin);

  SoftAcc A;
  A.init();
  // slices sl, sl + 16, ... of the block; tokens past m are dropped
  for (int j0 = sl * CS_TOK; j0 < m; j0 += CS_SL * CS_TOK) {
    float z[CS_TOK][8], c[CS_TOK][8];
#pragma unroll
    for (int u = 0; u < CS_TOK; ++u) {
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
    A.feed<4>(z, c);
    A.feed<4>(z + 4, c + 4);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    part[0][sl][cgl * 8 + e] = A.mx[e];
    part[1][sl][cgl * 8 + e] = A.sm[e];
    part[2][sl][cgl * 8 + e] = A.acc[e];
  }
  __syncthreads();
  // merge: thread cgl2 < 16 takes the 8 channels of its channel group
  if (threadIdx.x >= CS_CG) return;
  const int cgl2 = threadIdx.x;
  const int cg2 = (int)(blockIdx.x % cgb) * CS_CG + cgl2;
  if (cg2 >= groups) return;
  float res[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int ch = cgl2 * 8 + e;
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < CS_SL; ++q) mx = fmaxf(mx, part[0][q][ch]);
    float sm = 0.f, acc = 0.f;
#pragma unroll
    for (int q = 0; q < CS_SL; ++q) {
      const float a = part[0][q][ch] == -INFINITY ? 0.f : exp2f(part[0][q][ch] - mx);
      sm += part[1][q][ch] * a;
      acc += part[2][q][ch] * a;
    }
    res[e] = acc / sm;
  }
  store8<OUT_DT>(out, b * out_cap + i, d, cg2 * 8, res);
}

template <int IN_DT, int OUT_DT>
static hipError_t launch(const CompressLaunch& a, hipStream_t st) {
  const int64_t nblk = a.blk_end - a.blk_begin;
  if (!a.overlap && a.m >= 2 * CS_TOK) {
    const int64_t grid = a.B * nblk * ((a.d / 8 + CS_CG - 1) / CS_CG);
    hipLaunchKernelGGL((compress_split_kernel<IN_DT, OUT_DT>), dim3((unsigned)grid), dim3(256), 0, st, a.Ca, a.Za,
                       a.Ba, a.out, a.n_rows, a.tok_begin, a.blk_begin, nblk, a.out_cap, a.d, a.m);
    return hipGetLastError();
  }
  const int64_t total = a.B * nblk * (a.d / 8);
  // few entries (a decode step): 64-thread groups reach more CUs
  const int nt = total < 256 * 256 ? 64 : 256;
  const int64_t grid = (total + nt - 1) / nt;
  hipLaunchKernelGGL((compress_kernel<IN_DT, OUT_DT>), dim3((unsigned)grid), dim3(nt), 0, st, a.Ca, a.Cb, a.Za,
                     a.Zb, a.Ba, a.Bb, a.out, a.B, a.n_rows, a.tok_begin, a.blk_begin, nblk, a.out_cap, a.d, a.m,
                     (int)a.overlap, (int)a.joint);
  return hipGetLastError();
}

hipError_t run_compress(const CompressLaunch& a, hipStream_t st) {
  if (a.B == 0 || a.blk_end <= a.blk_begin) return hipSuccess;
  if (a.out_dt == DT_KV_FP8)
    return a.in_dt == DT_BF16 ? launch<DT_BF16, DT_KV_FP8>(a, st) : launch<DT_F32, DT_KV_FP8>(a, st);
  if (a.in_dt == DT_BF16 && a.out_dt == DT_BF16) return launch<DT_BF16, DT_BF16>(a, st);
  if (a.in_dt == DT_BF16 && a.out_dt == DT_F32) return launch<DT_BF16, DT_F32>(a, st);
  if (a.in_dt == DT_F32 && a.out_dt == DT_BF16) return launch<DT_F32, DT_BF16>(a, st);
  return launch<DT_F32, DT_F32>(a, st);
}

}  // namespace csa
