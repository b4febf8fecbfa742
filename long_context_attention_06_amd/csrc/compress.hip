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
#include "compress_entry.h"
#include "kernels.h"

namespace csa {

template <int IN_DT, int OUT_DT>
__global__ void __launch_bounds__(256) compress_kernel(CompressArgs a) {
  compress_entry<IN_DT, OUT_DT>(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
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
constexpr int CS_CG = 16;    // channel groups per workgroup
// With few blocks (a decode step's append: one block per sequence) the
// workgroups cover 4 channel groups and 64 slices of 2 tokens instead, so a
// step of 16 sequences offers 256 workgroups rather than 64.
constexpr int CS_TOK_FEW = 2, CS_CG_FEW = 4;

template <int IN_DT, int OUT_DT, int CG, int TOK>
__global__ void __launch_bounds__(256)
compress_split_kernel(const void* __restrict__ Ca, const void* __restrict__ Za, const float* __restrict__ Ba,
                      void* __restrict__ out, int64_t n_rows, int64_t tok_begin, int64_t blk_begin, int64_t nblk,
                      int64_t out_cap, int d, int m) {
  constexpr int SL = 256 / CG;  // slices per workgroup pass
  __shared__ float part[3][SL][CG * 8];  // max, sum, weighted sum (exp2 domain)
  __shared__ float merged[CG * 8];
  const int groups = d / 8;
  const int cgb = (groups + CG - 1) / CG;  // workgroups per block
  const int cgl = threadIdx.x % CG, sl = threadIdx.x / CG;
  const int cg = (int)(blockIdx.x % cgb) * CG + cgl;
  const int64_t t = blockIdx.x / cgb;
  const int64_t i = blk_begin + t % nblk;
  const int64_t b = t / nblk;
  const bool live = cg < groups;
  const int c0 = live ? cg * 8 : 0;
  const int64_t row0 = b * n_rows + (m * i - tok_begin);

  SoftAcc A;
  A.init();
  // slices sl, sl + SL, ... of the block; tokens past m are dropped
  for (int j0 = sl * TOK; j0 < m; j0 += SL * TOK) {
    float z[TOK][8], c[TOK][8];
#pragma unroll
    for (int u = 0; u < TOK; ++u) {
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
    // the first group holds token j0 < m, so its maximum is finite
    if constexpr (TOK >= 4) {
#pragma unroll
      for (int g = 0; g < TOK; g += 4) A.feed<4>(z + g, c + g);
    } else {
      A.feed<TOK>(z, c);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    part[0][sl][cgl * 8 + e] = A.mx[e];
    part[1][sl][cgl * 8 + e] = A.sm[e];
    part[2][sl][cgl * 8 + e] = A.acc[e];
  }
  __syncthreads();
  // merge: one thread per channel over the slices, in slice order
  if (threadIdx.x < CG * 8) {
    const int ch = threadIdx.x;
    float mx = -INFINITY;
    for (int q = 0; q < SL; ++q) mx = fmaxf(mx, part[0][q][ch]);
    float sm = 0.f, acc = 0.f;
    for (int q = 0; q < SL; ++q) {
      const float a = part[0][q][ch] == -INFINITY ? 0.f : exp2f(part[0][q][ch] - mx);
      sm += part[1][q][ch] * a;
      acc += part[2][q][ch] * a;
    }
    merged[ch] = acc / sm;
  }
  __syncthreads();
  if (threadIdx.x >= CG) return;
  const int cg2 = (int)(blockIdx.x % cgb) * CG + (int)threadIdx.x;
  if (cg2 >= groups) return;
  float res[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) res[e] = merged[threadIdx.x * 8 + e];
  store8<OUT_DT>(out, b * out_cap + i, d, cg2 * 8, res);
}

CompressArgs compress_args(const CompressLaunch& a) {
  return CompressArgs{a.Ca, a.Cb, a.Za, a.Zb, a.Ba, a.Bb, a.out, a.B, a.n_rows, a.tok_begin, a.blk_begin,
                      a.blk_end - a.blk_begin, a.out_cap, a.d, a.m, (int)a.overlap, (int)a.joint};
}

template <int IN_DT, int OUT_DT>
static hipError_t launch(const CompressLaunch& a, hipStream_t st) {
  const int64_t nblk = a.blk_end - a.blk_begin;
  if (!a.overlap && a.m >= 2 * CS_TOK) {
    const int64_t grid = a.B * nblk * ((a.d / 8 + CS_CG - 1) / CS_CG);
    if (grid < 256 && a.m >= 64) {
      const int64_t gf = a.B * nblk * ((a.d / 8 + CS_CG_FEW - 1) / CS_CG_FEW);
      hipLaunchKernelGGL((compress_split_kernel<IN_DT, OUT_DT, CS_CG_FEW, CS_TOK_FEW>), dim3((unsigned)gf), dim3(256),
                         0, st, a.Ca, a.Za, a.Ba, a.out, a.n_rows, a.tok_begin, a.blk_begin, nblk, a.out_cap, a.d,
                         a.m);
    } else {
      hipLaunchKernelGGL((compress_split_kernel<IN_DT, OUT_DT, CS_CG, CS_TOK>), dim3((unsigned)grid), dim3(256), 0,
                         st, a.Ca, a.Za, a.Ba, a.out, a.n_rows, a.tok_begin, a.blk_begin, nblk, a.out_cap, a.d, a.m);
    }
    return hipGetLastError();
  }
  const int64_t total = a.B * nblk * (a.d / 8);
  // few entries (a decode step): 64-thread groups reach more CUs
  const int nt = total < 256 * 256 ? 64 : 256;
  const int64_t grid = (total + nt - 1) / nt;
  hipLaunchKernelGGL((compress_kernel<IN_DT, OUT_DT>), dim3((unsigned)grid), dim3(nt), 0, st, compress_args(a));
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
