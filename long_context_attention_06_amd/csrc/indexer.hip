// Lightning-indexer scores for gfx950.
//
// What is computed (DeepSeek V4 脱离 CUDA 全栈国产化, deepseek.csdn.net,
// section 二, CSA step 2; 64 indexer heads of dim 128 per m.lqnn.cn
// "Deepseek-V4 技术报告里最值得复现的三个改动", section 3): for a query with
// indexer vectors q_h (h < 64) and head weights w_h, every visible compressed
// entry i with key k_i gets  s_i = sum_h w_h * max(0, sigma_i <q_h, k_i>),
// sigma_i being the per-entry scale of FP8 keys (1 otherwise).
//
// Design: the scan over keys is the dominant HBM stream of CSA decode. It is
// a [64 heads x 128] x [128 x entries] contraction, run on
// v_mfma_f32_32x32x16_bf16 with heads as M (two 32-row tiles) and entries as
// N (32 per column block). The query operand stays in registers for the whole
// workgroup. Each lane reads 128 contiguous bytes of one key row (bf16) or 64
// (FP8, decoded exactly to bf16 in registers; the scale is applied after the
// head sum since it is positive). The epilogue never leaves registers: a lane
// holds 16 heads of one entry per tile, applies ReLU and w, sums, and one
// cross-half shuffle completes the 64-head sum. K dims are visited in a
// permuted order (lane half g covers dims g*64..g*64+63), identical for q and
// k, which leaves the dot products unchanged.
#include "common.h"
#include "kernels.h"

namespace csa {

// bf16 / fp8 keys, 64 heads x 128 dims.  Grid: (tile groups, rows).
// A workgroup (4 waves) walks entry tiles of 256 (64 per wave) of one query row.
template <int KDT>
__global__ void __launch_bounds__(256)
idx_scan_bf16_kernel(const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                     const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale,
                     const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_comp, int64_t Tq,
                     int64_t N_max, int m, float* __restrict__ scores) {
  constexpr int H = 64, DI = 128, KS = 8;  // k-steps of 16
  constexpr int KROW = (KDT == DT_FP8) ? DI : DI * 2;  // bytes per key row
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = l >> 5, l32 = l & 31;
  const int64_t row = blockIdx.y;
  const int64_t b = row / Tq;
  int64_t V = min((int64_t)n_comp[b], ((int64_t)q_pos[row] + 1) / m);
  V = max((int64_t)0, min(V, N_max));
  const int64_t ntiles = (V + 255) / 256;
  if ((int64_t)blockIdx.x >= ntiles) return;

  // query operand: A[m = head][k], lane (head mt*32+l32, half g) holds dims g*64 + s*8 + 0..7
  bf16x8_t qa[2][KS];
  float wr[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const uint16_t* qp = q_idx + (row * H + mt * 32 + l32) * DI + g * 64;
#pragma unroll
    for (int s = 0; s < KS; ++s) qa[mt][s] = as_bf16x8(ld16(qp + s * 8));
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[mt][r] = w[row * H + mt * 32 + (r >> 2) * 8 + g * 4 + (r & 3)];
  }
  const uint8_t* kb = k_idx + b * N_max * KROW;
  float* srow = scores + row * N_max;

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int64_t e = tile * 256 + wv * 64 + cb * 32 + l32;
      const bool ok = e < V;
      bf16x8_t kbv[KS];
      if constexpr (KDT == DT_FP8) {
        const uint8_t* kp = kb + (ok ? e : 0) * KROW + g * 64;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4_t v = ok ? ld16(kp + c * 16) : u32x4_t{0, 0, 0, 0};
          u32x2_t a0 = fp8x4_to_bf16x4(v[0]), a1 = fp8x4_to_bf16x4(v[1]);
          u32x2_t a2 = fp8x4_to_bf16x4(v[2]), a3 = fp8x4_to_bf16x4(v[3]);
          kbv[2 * c] = as_bf16x8(u32x4_t{a0[0], a0[1], a1[0], a1[1]});
          kbv[2 * c + 1] = as_bf16x8(u32x4_t{a2[0], a2[1], a3[0], a3[1]});
        }
      } else {
        const uint8_t* kp = kb + (ok ? e : 0) * KROW + g * 128;
#pragma unroll
        for (int s = 0; s < KS; ++s) kbv[s] = as_bf16x8(ok ? ld16(kp + s * 16) : u32x4_t{0, 0, 0, 0});
      }
      float part = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16_t acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma32(qa[mt][s], kbv[s], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) part += wr[mt][r] * fmaxf(acc[r], 0.0f);
      }
      part += shfl_xor(part, 32);
      if (g == 0 && ok) {
        if constexpr (KDT == DT_FP8) part *= k_scale[b * N_max + e];
        srow[e] = part;
      }
    }
  }
}

// fp32 keys and queries, up to 32 heads (tiny shapes): v_mfma_f32_32x32x2f32,
// heads padded to 32 with zero rows. D_I = 32.
__global__ void __launch_bounds__(256)
idx_scan_f32_kernel(const float* __restrict__ q_idx, const float* __restrict__ w, const float* __restrict__ k_idx,
                    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_comp, int64_t Tq,
                    int64_t N_max, int m, int H, float* __restrict__ scores) {
  constexpr int DI = 32, KS = DI / 2;
  const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = l >> 5, l32 = l & 31;
  const int64_t row = blockIdx.y;
  const int64_t b = row / Tq;
  int64_t V = min((int64_t)n_comp[b], ((int64_t)q_pos[row] + 1) / m);
  V = max((int64_t)0, min(V, N_max));
  const int64_t ntiles = (V + 127) / 128;
  if ((int64_t)blockIdx.x >= ntiles) return;

  float qa[KS];
  const bool hok = l32 < H;
#pragma unroll
  for (int s = 0; s < KS; ++s) qa[s] = hok ? q_idx[(row * H + l32) * DI + g * (DI / 2) + s] : 0.0f;
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int h = (r >> 2) * 8 + g * 4 + (r & 3);
    wr[r] = h < H ? w[row * H + h] : 0.0f;
  }
  float* srow = scores + row * N_max;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t e = tile * 128 + wv * 32 + l32;
    const bool ok = e < V;
    const float* kp = k_idx + (b * N_max + (ok ? e : 0)) * DI + g * (DI / 2);
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(qa[s], ok ? kp[s] : 0.0f, acc);
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.0f);
    part += shfl_xor(part, 32);
    if (g == 0 && ok) srow[e] = part;
  }
}

hipError_t run_indexer(const IndexerLaunch& a, hipStream_t st) {
  const int64_t rows = a.B * a.Tq;
  if (rows == 0 || a.N_max == 0) return hipSuccess;
  if (a.H_I == 64 && a.D_I == 128 && a.q_dt == DT_BF16) {
    const int64_t ntiles = (a.N_max + 255) / 256;
    // enough workgroups per row to fill the chip, each walking a few tiles
    int64_t per_row = (2048 + rows - 1) / rows;
    per_row = max((int64_t)1, min(ntiles, per_row));
    dim3 grid((unsigned)per_row, (unsigned)rows);
    if (a.k_dt == DT_FP8)
      hipLaunchKernelGGL((idx_scan_bf16_kernel<DT_FP8>), grid, dim3(256), 0, st,
                         reinterpret_cast<const uint16_t*>(a.q_idx), a.w, reinterpret_cast<const uint8_t*>(a.k_idx),
                         a.k_scale, a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores);
    else
      hipLaunchKernelGGL((idx_scan_bf16_kernel<DT_BF16>), grid, dim3(256), 0, st,
                         reinterpret_cast<const uint16_t*>(a.q_idx), a.w, reinterpret_cast<const uint8_t*>(a.k_idx),
                         a.k_scale, a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores);
    return hipGetLastError();
  }
  // f32, D_I = 32, H_I <= 32
  const int64_t ntiles = (a.N_max + 127) / 128;
  int64_t per_row = (2048 + rows - 1) / rows;
  per_row = max((int64_t)1, min(ntiles, per_row));
  dim3 grid((unsigned)per_row, (unsigned)rows);
  hipLaunchKernelGGL(idx_scan_f32_kernel, grid, dim3(256), 0, st, reinterpret_cast<const float*>(a.q_idx), a.w,
                     reinterpret_cast<const float*>(a.k_idx), a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.H_I,
                     a.scores);
  return hipGetLastError();
}

}  // namespace csa
