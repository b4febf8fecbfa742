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
// v_mfma_f32_16x16x32_bf16 (or, for the FP4 QK path, the scaled FP4 MFMA)
// with heads as M (four 16-row tiles) and entries as N (16 per wave). The
// query operand stays in registers for the whole workgroup. Decode scans
// load the key operands straight from HBM into a register ring (no LDS tile,
// no barrier per tile); FP8 and FP4 keys are widened exactly to bf16 in
// registers, the FP8 scale applied after the head sum (it is positive). The
// prefill scan shares each key tile of LDS among eight query rows. The
// epilogue never leaves registers: a lane holds 16 heads of one entry per
// tile, applies ReLU and w, sums, and two cross-lane shuffles complete the
// 64-head sum. K dims are visited in a permuted order (lane group G covers
// dims G*32..G*32+31), identical for q and k, which leaves the dot products
// unchanged.
#include <type_traits>

#include "common.h"
#include "compress_entry.h"
#include "kernels.h"

namespace csa {

#ifndef IDX_BF16_TE
#define IDX_BF16_TE 64
#endif

// The scans also count, per query row, the scores by digit: the top 11 bits
// of the order-preserving key (sign, exponent, two mantissa bits). The top-k
// uses the counts to find the bin holding its threshold without a pass of its
// own; it checks the counts against the scores, so they are a hint only.
constexpr int DIG_BINS = 2048;
constexpr int DIG_SHIFT = 21;

// Workgroup (0, 0) of a scan zeroes the top-k's arrival counters (the scan
// runs first in the call, so they are zero when the top-k starts).
__device__ __forceinline__ void zero_counters(uint32_t* zero, int64_t n) {
  if (zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) zero[i] = 0u;
}

// XOR swizzle of the 16-byte chunk index of key row r in a prefill LDS tile.
// The operand reads take one chunk of each of 16 consecutive rows; with 64
// banks of 4 bytes those 16 chunks must fall in 16 different 16-byte bank
// groups.
// fp8 rows are 128 bytes (odd rows start in group 8): chunk ^ ((r >> 1) & 7).
// MXFP4 rows are 64 bytes (four rows per 256 bytes): chunk ^ ((r >> 2) & 3).
// bf16 rows (256 bytes, every row starts in group 0) serve the prefill
// kernel's 32x32 operand reads: a 16-byte access is served in passes of the
// 16 lanes that agree in lane bits 2 and 4, which there are eight rows (low
// bits 0, 1, 3 varying) times two chunk halves, and in the tile stores two
// rows (bit 1 varying) times eight chunks (bit 2 fixed). Row bits (2, 0, 1, 3)
// as the chunk's bits (0, 1, 2, 3) keep the 16 lanes of a pass in 16 groups
// in both.
template <int KDT>
__device__ __forceinline__ int kswz(int r) {
  return KDT == DT_FP8 ? ((r >> 1) & 7)
         : KDT == DT_MXFP4 ? ((r >> 2) & 3)
                           : (((r >> 2) & 1) | ((r & 1) << 1) | ((r & 2) << 1) | (r & 8));
}

// 8 OCP MXFP4 codes (one dword, element 2j in the low nibble of byte j) ->
// 8 bf16, times the block scale 2^(E - 127): gfx950's scaled convert takes two
// codes per instruction and applies the scale's exponent exactly (every E2M1
// value times a power of two in bf16 range is a bf16 value).
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t codes, float scale) {
  return as_bf16x8(u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3))});
}

// One OCP MXFP4 block (Microscaling Formats v1.0: 32 values, one E8M0 scale)
// from 32 bf16 values: x[j] holds values 8j .. 8j + 7, value 8j + 2c + h in
// half h of dword c. The shared exponent is floor(log2 amax) - 2 (2 being the
// largest E2M1 exponent), which for a bf16 amax is its exponent field minus
// 2, kept in 1..254 (127 for an all-zero block). Each value times
// 2^(127 - E) (exact: a power of two) is rounded half-to-even on the E2M1
// grid -- spacing 0.5 below 2, 1 below 4, 2 above, so round-half-even of the
// value over its spacing -- and saturated at 6 (code 7); a value that rounds
// to zero keeps no sign. Codes are packed as MXFP4 stores them: value 8j + i
// in bits 4i .. 4i + 3 of codes[j]. Returns the scale byte.
__device__ __forceinline__ int mxfp4_quant_block(const u32x4_t (&x)[4], u32x4_t& codes) {
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) amax = max(amax, max(x[j][c] & 0x7fffu, (x[j][c] >> 16) & 0x7fffu));
  const int E = amax == 0 ? 127 : min(max((int)(amax >> 7) - 2, 1), 254);
  // 2^(127 - E) has the fp32 exponent field 254 - E, in 2..253 for every
  // finite amax (a finite bf16's field is at most 254, so E <= 252)
  const float inv = __uint_as_float((uint32_t)(254 - E) << 23);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t d = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t bits = h ? (x[j][c] & 0xffff0000u) : (x[j][c] << 16);
        const float a = fabsf(__uint_as_float(bits)) * inv;
        const float sp = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
        const int off = a < 2.0f ? 0 : (a < 4.0f ? 2 : 4);
        const uint32_t n = (uint32_t)min((int)__builtin_rintf(a * sp) + off, 7);
        d |= (n | ((bits >> 28) & (n ? 8u : 0u))) << (8 * c + 4 * h);
      }
    codes[j] = d;
  }
  return E;
}

// S[16 heads x 16 entries] of one 128-dim FP4 x FP4 product with E8M0 block
// scales on gfx950's scaled MFMA (format 4 = E2M1 for both operands). Lane
// (group G, column l16) gives, for row l16 of each operand, the 32 codes of
// dims 32G .. 32G + 31 (four dwords, the MXFP4 packing) and that block's
// scale byte; the result has the layout of v_mfma_f32_16x16x32_bf16.
__device__ __forceinline__ f32x4_t mfma_fp4(const u32x4_t& a, int sa, const u32x4_t& b, int sb) {
  typedef int v8i_t __attribute__((ext_vector_type(8)));
  const v8i_t av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const v8i_t bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, sa, 0, sb);
}

// bf16 keys, 64 heads x 128 dims.  Grid: (workgroups per row, rows).
// A workgroup walks tiles of TE = 64 entries of one query row with a stride
// of gridDim.x tiles; wave w owns entries 16 w .. 16 w + 15 of each tile and
// loads its MFMA operands straight from memory: for k-step s (dims 32 s ..
// 32 s + 31) lane (group G, entry l16) takes the 16 bytes of dims 32 s + 8 G
// .. + 7, so each load instruction reads 64 contiguous bytes of 16 key rows.
// The waves never wait for each other (no LDS tile, no barrier per tile).
// Two tiles per wave are in flight (a register ring) while one is computed;
// heads are four 16-row M tiles of v_mfma_f32_16x16x32_bf16. With NQ = 2 a
// workgroup serves two query rows of one sequence (a step with a drafted
// token): each key tile is loaded once for both queries' 2 x 64 heads.
// With CO != 0 the grid's rows past scan_y are a decode step's compression
// (bf16 in, output dtype CO): it has no dependence on the scan, so its few
// workgroups run beside the scan's instead of in a launch of their own.
template <int NQ, int CO>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
idx_scan_bf16_kernel(const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                     const uint8_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos,
                     const int32_t* __restrict__ n_comp, int64_t Tq, int64_t N_max, int m,
                     float* __restrict__ scores, CompressArgs ca, unsigned scan_y, uint32_t* __restrict__ hint,
                     uint32_t* __restrict__ zero, int64_t zero_n) {
  if constexpr (CO != 0) {
    if (blockIdx.y >= scan_y) {
      compress_entry<DT_BF16, CO>(ca, ((int64_t)(blockIdx.y - scan_y) * gridDim.x + blockIdx.x) * 256 + threadIdx.x);
      return;
    }
  }
  constexpr int H = 64, DI = 128, KS = 4;               // k-steps of 32
  constexpr int KROW = DI * 2;                          // bytes per key row
  constexpr int TE = IDX_BF16_TE;                       // entries per tile (16 per wave)
  static_assert(TE == 64, "one 16-entry N tile per wave");
  __shared__ __attribute__((aligned(16))) float lds_w[NQ * H];
  __shared__ __attribute__((aligned(16))) uint32_t lds_h[NQ * DIG_BINS];  // digit histogram per query row

  const int tid = threadIdx.x;
  const int l = tid & 63, wv = tid >> 6;
  const int G = l >> 4, l16 = l & 15;  // k-group (8 dims of each k-step) and entry of the MFMA operands
  const int64_t row0 = (int64_t)blockIdx.y * NQ;  // first query row of this workgroup (Tq % NQ == 0)
  const int64_t b = row0 / Tq;
  const uint8_t* kb = k_idx + b * N_max * KROW + G * 16;

  u32x4_t rg[3][KS];
  // register ring slots are compile-time indices (a runtime index would move
  // the ring to scratch memory). Every lane loads (the entry clamped to
  // lim - 1, lim >= 1): predicated loads would leave the number in flight
  // path-dependent and the compiler would then wait for all of them each tile.
  // Entries at or past lim are computed but never stored. lim is N_max for the
  // first two tiles, which go out before the row's visible count V is known,
  // and V after.
  auto load = [&](auto SLOT, int64_t tile, int64_t lim) {
    constexpr int slot = decltype(SLOT)::value;
    const int64_t e = min(tile * TE + wv * 16 + l16, lim - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s) rg[slot][s] = ld16(kb + e * KROW + s * 64);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  load(I0{}, blockIdx.x, N_max);
  load(I1{}, blockIdx.x + gridDim.x, N_max);

  int64_t Vq[NQ], V = 0;  // visible entries of each query; the tiles cover the largest
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    Vq[j] = max((int64_t)0, min(min((int64_t)n_comp[b], ((int64_t)q_pos[row0 + j] + 1) / m), N_max));
    V = max(V, Vq[j]);
  }
  const int64_t ntiles = (V + TE - 1) / TE;
  if ((int64_t)blockIdx.x >= ntiles) {
    zero_counters(zero, zero_n);
    return;
  }
  const int64_t nmine = (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;  // tiles of this workgroup

  // query operand A[m = head][k]: lane (head mt*16 + l16, group G) holds dims
  // 32 s + 8 G .. + 7 for k-step s
  bf16x8_t qa[NQ][4][KS];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint16_t* qp = q_idx + ((row0 + j) * H + mt * 16 + l16) * DI + G * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s) qa[j][mt][s] = as_bf16x8(ld16(qp + s * 32));
    }
  if (tid < NQ * H) lds_w[tid] = w[row0 * H + tid];
  if (hint)
    for (int i = tid; i < NQ * DIG_BINS; i += 256) lds_h[i] = 0u;
  // wait for the query and the weights here, on every lane: left pending into
  // the loop, these loads would make each tile wait for all loads in flight
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qa[j][mt][s]));
  __syncthreads();
  f32x4_t wr[NQ][4];  // weights of heads mt*16 + G*4 + 0..3 (accumulator rows of this lane)
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) wr[j][mt] = *reinterpret_cast<const f32x4_t*>(&lds_w[j * H + mt * 16 + G * 4]);
  // scores go out through a buffer descriptor of each row's V entries: the
  // hardware drops stores past its end, so the store needs no branch (a
  // branch would again make the count of memory operations in flight unknown)
  __amdgpu_buffer_rsrc_t srow[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
    srow[j] = __builtin_amdgcn_make_buffer_rsrc(scores + (row0 + j) * N_max, (short)0, (int)(Vq[j] * 4),
                                                BUF_RSRC_WORD3);

  // tile it is in slot it % 3; the load of tile it + 2 goes to the slot the
  // previous tile used, so no register is both read and refilled in one step
  auto body = [&](int64_t it, auto SLOT, auto NEXT) {
    constexpr int slot = decltype(SLOT)::value;
    const int64_t tile = blockIdx.x + it * gridDim.x;
    load(NEXT, blockIdx.x + (it + 2) * gridDim.x, V);  // past the last tile: clamped, unused
    const int e = (int)(tile * TE) + wv * 16 + l16;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float part = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma16(qa[j][mt][s], as_bf16x8(rg[slot][s]), acc);
        // accumulator row r of this lane is head mt*16 + G*4 + r
#pragma unroll
        for (int r = 0; r < 4; ++r) part += wr[j][mt][r] * relu_bits(acc[r]);
      }
      part = sum_rows16(part);
      // lanes of groups 1..3 hold the same sums: their offset is past the end
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part), srow[j], G == 0 ? e * 4 : (int)(Vq[j] * 4), 0,
                                            0);
      if (hint && G == 0 && e < Vq[j]) atomicAdd(&lds_h[j * DIG_BINS + (f32_key(part) >> DIG_SHIFT)], 1u);
    }
  };
  // whole triples and unconditional loads keep the count of memory operations
  // in flight the same on every path, so each tile waits for its own loads
  // only; trailing tiles past the row are computed past V and dropped
  for (int64_t it = 0; it < nmine; it += 3) {
    body(it, I0{}, I2{});
    body(it + 1, I1{}, I0{});
    body(it + 2, I2{}, I1{});
  }
  zero_counters(zero, zero_n);
  if (hint) {
    __syncthreads();
    for (int i = tid; i < NQ * DIG_BINS; i += 256) {
      const uint32_t v = lds_h[i];
      if (v) atomicAdd(&hint[(row0 + i / DIG_BINS) * DIG_BINS + (i % DIG_BINS)], v);
    }
  }
}

// Decode scan of low-precision keys (E4M3 with a per-entry fp32 scale, or
// MXFP4), 64 heads x 128 dims. Grid: (workgroups per row, rows); one query
// row per workgroup. As in the bf16 scan the waves load their MFMA operands
// straight from memory and never wait for each other: a workgroup tile is
// 64 NT entries, wave w owns entries 16 NT w .. 16 NT w + 16 NT - 1 of it as
// NT 16-entry N tiles, and for N tile n lane (group G, entry l16) loads the
// codes of dims 32 G .. 32 G + 31 of its entry (E4M3: 32 bytes, so one load
// instruction reads two 1 KB halves of 16 consecutive 128-byte rows; MXFP4:
// block G, 16 bytes, 1 KB of 16 consecutive 64-byte rows) and the entry's
// scale word. A three-slot register ring keeps two tiles in flight.
//   bf16 query (QF4 false): codes are widened exactly to bf16 (two per
//   scaled convert) in the k order of the query operand (k-step s takes dims
//   32 G + 8 s .. + 7, a permutation applied to both sides), and a tile's
//   16 entries x 64 heads are 4 x 4 v_mfma_f32_16x16x32_bf16; the E4M3 scale
//   multiplies the head-weighted sum (it is positive).
//   FP4 query (QF4, MXFP4 keys: the FP4 QK path): the query is quantised
//   once per workgroup (thread t makes block t % 4 of head t / 4,
//   mxfp4_quant_block; the codes reach the operand lanes through 4 KB of
//   LDS) and each N tile is four scaled FP4 MFMAs (v_mfma_scale_f32_16x16x128
//   _f8f6f4, one per 16-head M tile over all 128 dims) with the key block's
//   scale byte; no code is widened.
template <int KDT, bool QF4, int CO>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
idx_scan_reg_kernel(const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                    const uint8_t* __restrict__ k_idx, const uint32_t* __restrict__ k_scale,
                    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_comp, int64_t Tq,
                    int64_t N_max, int m, float* __restrict__ scores, CompressArgs ca, unsigned scan_y,
                    uint32_t* __restrict__ hint, uint32_t* __restrict__ zero, int64_t zero_n) {
  static_assert(KDT == DT_FP8 || KDT == DT_MXFP4, "low-precision keys");
  static_assert(!QF4 || KDT == DT_MXFP4, "the FP4 query goes with MXFP4 keys");
  if constexpr (CO != 0) {
    if (blockIdx.y >= scan_y) {
      compress_entry<DT_BF16, CO>(ca, ((int64_t)(blockIdx.y - scan_y) * gridDim.x + blockIdx.x) * 256 + threadIdx.x);
      return;
    }
  }
  constexpr bool MX = KDT == DT_MXFP4;
  constexpr int H = 64, DI = 128, KS = 4;  // k-steps of 32 (bf16 query)
  constexpr int KROW = MX ? DI / 2 : DI;   // code bytes per key row
  constexpr int CPL = MX ? 1 : 2;          // 16-byte code chunks per lane and N tile
  constexpr int NT = MX ? 4 : 2;           // N tiles per wave and tile (4 KB of codes per wave)
  constexpr int TE = 64 * NT;              // entries per workgroup tile
  __shared__ __attribute__((aligned(16))) u32x4_t lds_qc[QF4 ? H * 4 : 1];  // FP4 query: block g of head h at [4 h + g]
  __shared__ __attribute__((aligned(16))) int lds_qs[QF4 ? H * 4 : 1];      // and its scale byte
  __shared__ __attribute__((aligned(16))) uint32_t lds_h[DIG_BINS];

  const int tid = threadIdx.x;
  const int l = tid & 63, wv = tid >> 6;
  const int G = l >> 4, l16 = l & 15;
  const int64_t row = blockIdx.y;
  const int64_t b = row / Tq;
  const uint8_t* kb = k_idx + b * N_max * KROW + G * (16 * CPL);
  const uint32_t* ksw = k_scale + b * N_max;

  u32x4_t rc[3][NT][CPL];  // ring: the lane's codes of entry (tile, wave, n, l16)
  uint32_t rs[3][NT];      // and that entry's scale word
  // unconditional loads, the entry clamped to lim - 1 (lim >= 1), as in the
  // bf16 scan: the number of loads in flight is the same on every path
  auto load = [&](auto SLOT, int64_t tile, int64_t lim) {
    constexpr int slot = decltype(SLOT)::value;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int64_t e = min(tile * TE + wv * (16 * NT) + n * 16 + l16, lim - 1);
#pragma unroll
      for (int c = 0; c < CPL; ++c) rc[slot][n][c] = ld16(kb + e * KROW + c * 16);
      rs[slot][n] = ksw[e];
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  load(I0{}, blockIdx.x, N_max);
  load(I1{}, blockIdx.x + gridDim.x, N_max);

  const int64_t V = max((int64_t)0, min(min((int64_t)n_comp[b], ((int64_t)q_pos[row] + 1) / m), N_max));
  const int64_t ntiles = (V + TE - 1) / TE;
  if ((int64_t)blockIdx.x >= ntiles) {
    zero_counters(zero, zero_n);
    return;
  }
  const int64_t nmine = (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;

  bf16x8_t qa[QF4 ? 1 : 4][KS];  // bf16 query: lane (head mt*16 + l16, group G) holds dims 32 G + 8 s .. + 7
  u32x4_t qc[4];                 // FP4 query: block G of head mt*16 + l16, and its scale byte
  int qsb[4];
  if constexpr (QF4) {
    const int h = tid >> 2, g = tid & 3;  // thread t: block g (dims 32 g .. 32 g + 31) of head h
    const uint16_t* qp = q_idx + (row * H + h) * DI + g * 32;
    u32x4_t xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[j] = ld16(qp + j * 8);
    u32x4_t c;
    lds_qs[tid] = mxfp4_quant_block(xv, c);
    lds_qc[tid] = c;
  } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint16_t* qp = q_idx + (row * H + mt * 16 + l16) * DI + G * 32;
#pragma unroll
      for (int s = 0; s < KS; ++s) qa[mt][s] = as_bf16x8(ld16(qp + s * 8));
    }
  }
  f32x4_t wr[4];  // weights of heads mt*16 + G*4 + 0..3 (the accumulator rows of this lane)
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[mt][r] = w[row * H + mt * 16 + G * 4 + r];
  if (hint)
    for (int i = tid; i < DIG_BINS; i += 256) lds_h[i] = 0u;
  __syncthreads();
  if constexpr (QF4) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      qc[mt] = lds_qc[(mt * 16 + l16) * 4 + G];
      qsb[mt] = lds_qs[(mt * 16 + l16) * 4 + G];
    }
  } else {
    // the query's loads complete here, not inside the loop
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qa[mt][s]));
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) asm volatile("" ::"v"(wr[mt]));
  const __amdgpu_buffer_rsrc_t srow =
      __builtin_amdgcn_make_buffer_rsrc(scores + row * N_max, (short)0, (int)(V * 4), BUF_RSRC_WORD3);

  auto body = [&](int64_t it, auto SLOT, auto NEXT) {
    constexpr int slot = decltype(SLOT)::value;
    const int64_t tile = blockIdx.x + it * gridDim.x;
    load(NEXT, blockIdx.x + (it + 2) * gridDim.x, V);  // past the last tile: clamped, unused
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = (int)(tile * TE) + wv * (16 * NT) + n * 16 + l16;
      float part = 0.0f;
      if constexpr (QF4) {
        const int kscale = (int)((rs[slot][n] >> (8 * G)) & 0xffu);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4_t acc = mfma_fp4(qc[mt], qsb[mt], rc[slot][n][0], kscale);
#pragma unroll
          for (int r = 0; r < 4; ++r) part += wr[mt][r] * relu_bits(acc[r]);
        }
      } else {
        bf16x8_t kbv[KS];
        if constexpr (MX) {
          // block G's E8M0 byte as the fp32 2^(E - 127), applied in the convert
          const float sc = __uint_as_float(((rs[slot][n] >> (8 * G)) & 0xffu) << 23);
#pragma unroll
          for (int s = 0; s < KS; ++s) kbv[s] = fp4x8_to_bf16x8(rc[slot][n][0][s], sc);
        } else {
          // k-step s: bytes 8 s .. 8 s + 7 of the lane's 32, i.e. chunk s / 2, half s % 2
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const u32x4_t v = rc[slot][n][c];
            u32x4_t lo, hi;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              lo[2 * q] = fp8x2_to_bf16x2(v[q], false);
              lo[2 * q + 1] = fp8x2_to_bf16x2(v[q], true);
              hi[2 * q] = fp8x2_to_bf16x2(v[2 + q], false);
              hi[2 * q + 1] = fp8x2_to_bf16x2(v[2 + q], true);
            }
            kbv[2 * c] = as_bf16x8(lo);
            kbv[2 * c + 1] = as_bf16x8(hi);
          }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) acc = mfma16(qa[mt][s], kbv[s], acc);
          // accumulator row r of this lane is head mt*16 + G*4 + r
#pragma unroll
          for (int r = 0; r < 4; ++r) part += wr[mt][r] * relu_bits(acc[r]);
        }
      }
      part = sum_rows16(part);
      // E4M3: sigma_i scales the head-weighted sum (ReLU commutes with a
      // positive scale); MXFP4 scales are inside the products
      if constexpr (!MX) part *= __uint_as_float(rs[slot][n]);
      // lanes of groups 1..3 hold the same sums: their offset is past the end
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part), srow, G == 0 ? e * 4 : (int)(V * 4), 0, 0);
      if (hint && G == 0 && e < V) atomicAdd(&lds_h[f32_key(part) >> DIG_SHIFT], 1u);
    }
  };
  for (int64_t it = 0; it < nmine; it += 3) {
    body(it, I0{}, I2{});
    body(it + 1, I1{}, I0{});
    body(it + 2, I2{}, I1{});
  }
  zero_counters(zero, zero_n);
  if (hint) {
    __syncthreads();
    uint32_t* gh = hint + row * DIG_BINS;
    for (int i = tid; i < DIG_BINS; i += 256) {
      const uint32_t v = lds_h[i];
      if (v) atomicAdd(&gh[i], v);
    }
  }
}

// Prefill: many queries of one sequence. A workgroup of 8 waves owns 8
// consecutive query rows (wave w <-> row 8*blockIdx.x + w); each 64-entry key
// tile is loaded once (coalesced, XOR-swizzled LDS, double-buffered) and used
// by all 8 waves, so HBM/L2 key traffic drops 8x against the row kernel. Per
// wave and tile: 4 M-tiles (heads) x 4 N-tiles (entries) x 4 k-steps of
// v_mfma_f32_16x16x32_bf16. The workgroup walks tiles up to the largest
// visible count of its rows; entries a row cannot see are not written.
template <int KDT>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
idx_prefill_kernel(const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                   const uint8_t* __restrict__ k_idx, const uint32_t* __restrict__ k_scale,
                   const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_comp, int64_t Tq,
                   int64_t N_max, int m, float* __restrict__ scores, uint32_t* __restrict__ hint,
                   uint32_t* __restrict__ zero, int64_t zero_n) {
  constexpr int H = 64, DI = 128, KS = 4, QB = 8;
  constexpr bool MX = KDT == DT_MXFP4;
  constexpr int KROW = (KDT == DT_FP8) ? DI : MX ? DI / 2 : DI * 2;
  constexpr int TE = 64;
  constexpr int TB = TE * KROW;
  constexpr int NT = 64 * QB;
  constexpr int LPT = (TB + NT * 16 - 1) / (NT * 16);  // 16-byte loads per thread per tile
  static_assert(TB % (NT * 16) == 0 || TB < NT * 16, "tile load mapping");
  // bf16 keys: a DMA ring of four tiles; E4M3 / MXFP4: two register-staged tiles
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k[KDT == DT_BF16 ? 4 : 2][TB];
  __shared__ __attribute__((aligned(16))) uint32_t lds_ks[2][MX ? TE : 1];  // MXFP4: four E8M0 bytes per entry
  __shared__ __attribute__((aligned(16))) float lds_w[QB][H];
  // each wave's row: digit histogram, two 16-bit counts per word (the wave
  // sees its whole row, so the counts are exact unless one wraps)
  __shared__ __attribute__((aligned(16))) uint32_t lds_h[QB][DIG_BINS / 2];

  const int tid = threadIdx.x;
  const int l = tid & 63, wv = tid >> 6;
  const int G = l >> 4, l16 = l & 15;
  const int64_t b = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * QB + wv;  // this wave's query inside sequence b
  const bool qok = t < Tq;
  const int64_t row = b * Tq + (qok ? t : 0);
  int64_t Vq = 0;
  if (qok) {
    Vq = min((int64_t)n_comp[b], ((int64_t)q_pos[row] + 1) / m);
    Vq = max((int64_t)0, min(Vq, N_max));
  }
  // largest visible count over the workgroup's rows (rows are not assumed sorted)
  __shared__ int64_t lds_vmax[QB];
  if (l == 0) lds_vmax[wv] = Vq;
  if (tid < H * QB) {
    const int qq = tid / H, h = tid % H;
    const int64_t tq = (int64_t)blockIdx.x * QB + qq;
    lds_w[qq][h] = tq < Tq ? w[(b * Tq + tq) * H + h] : 0.0f;
  }
  __syncthreads();
  int64_t Vmax = 0;
#pragma unroll
  for (int i = 0; i < QB; ++i) Vmax = max(Vmax, lds_vmax[i]);
  const int64_t ntiles = (Vmax + TE - 1) / TE;
  zero_counters(zero, zero_n);
  if (ntiles == 0) return;  // no row of this workgroup sees an entry: the top-k never reads their counts
  if (hint)
    for (int i = l; i < DIG_BINS / 2; i += 64) lds_h[wv][i] = 0u;

  // bf16 keys run v_mfma_f32_32x32x16_bf16: heads are two 32-row M blocks,
  // entries two 32-column N blocks, dims eight k-steps of 16. Lane (h, l32)
  // with h = l / 32 holds A = head 32 mb + l32, dims 16 ks + 8 h .. +7, and
  // B = entry 32 nb + l32, the same dims; its output holds entry 32 nb + l32
  // for heads 32 mb + 8 (r / 4) + 4 h + r % 4 (r < 16).
  constexpr bool M32 = KDT == DT_BF16;
  const int h2 = l >> 5, l32 = l & 31;
  // this lane's head weights, read once (16x16 form: heads 16 mt + 4 G + r;
  // 32x32 form: heads 32 mb + 8 q + 4 h + r, quartet 4 mb + q)
  f32x4_t wq[M32 ? 8 : 4];
#pragma unroll
  for (int i = 0; i < (M32 ? 8 : 4); ++i)
    wq[i] = *reinterpret_cast<const f32x4_t*>(&lds_w[wv][M32 ? (i >> 2) * 32 + (i & 3) * 8 + 4 * h2 : i * 16 + G * 4]);
  // query operand, 16 registers of 16 bytes in either form (16x16: [mt][s],
  // head 16 mt + l16, dims 32 G + 8 s; 32x32: [2 mb + ks / 4][ks % 4], head
  // 32 mb + l32, dims 16 ks + 8 h)
  bf16x8_t qa[4][KS];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* qp = M32 ? q_idx + (row * H + (mt >> 1) * 32 + l32) * DI + (mt & 1) * 64 + h2 * 8
                             : q_idx + (row * H + mt * 16 + l16) * DI + G * 32;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qa[mt][s] = as_bf16x8(qok ? ld16(qp + (M32 ? s * 16 : s * 8)) : u32x4_t{0, 0, 0, 0});
  }
  const uint8_t* kb = k_idx + b * N_max * KROW;
  float* srow = scores + row * N_max;

  u32x4_t rg[2][LPT];
  uint32_t rs[2] = {0u, 0u};  // MXFP4: the scale dword of entry tid of the tile
  auto load = [&](auto SLOT, int64_t tile) {
    constexpr int slot = decltype(SLOT)::value;
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int o = (j * NT + tid) * 16;
      const int64_t e = tile * TE + o / KROW;
      rg[slot][j] = (o < TB && e < Vmax) ? ld16(kb + e * KROW + (o % KROW)) : u32x4_t{0, 0, 0, 0};
    }
    if constexpr (MX) {
      const int64_t e = tile * TE + tid;
      rs[slot] = (tid < TE && e < Vmax) ? k_scale[b * N_max + e] : 0u;
    }
  };
  auto stash = [&](auto SLOT) {
    constexpr int slot = decltype(SLOT)::value;
    if constexpr (MX) {
      if (tid < TE) lds_ks[slot][tid] = rs[slot];
    }
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int o = (j * NT + tid) * 16;
      if (o >= TB) continue;
      const int r = o / KROW, c = (o % KROW) / 16;
      *reinterpret_cast<u32x4_t*>(&lds_k[slot][r * KROW + ((c ^ kswz<KDT>(r)) * 16)]) = rg[slot][j];
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // 32x32 form: accumulators [mb][nb]; N block 1 carries into the next tile
  f32x16_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][1][r] = 0.0f;
  auto compute32 = [&](int64_t tile, const uint8_t* kt) {
    {
      // Half-tile software pipeline: the products of entries 0-31 (N block 0)
      // run beside the head sums of the previous tile's entries 32-63, the
      // products of entries 32-63 beside the head sums of entries 0-31. All
      // waves compute every tile (a row that does not see an entry stores
      // nothing for it), so the products and the sums form one straight-line
      // region the scheduler can interleave.
      // qa[2 mb + ks / 4][ks % 4] holds dims 16 ks + 8 h .. +7 of head 32 mb + l32
      auto kread = [&](int nb, int ks) {
        const int el = nb * 32 + l32;
        return as_bf16x8(
            *reinterpret_cast<const u32x4_t*>(&kt[el * KROW + (((2 * ks + h2) ^ kswz<KDT>(el)) * 16)]));
      };
      // head sum of N block nb, eight of its 32 (head, value) pairs per step
      auto hsum_part = [&](int nb, int q, float& part) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mb = q >> 2, r = (q & 3) * 4 + i;
          part += wq[4 * mb + (r >> 2)][r & 3] * relu_bits(acc[mb][nb][r]);
        }
      };
      float pprev = 0.0f, pcur = 0.0f;
      bf16x8_t kb = kread(0, 0);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][0][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t kn = kread(ks < 7 ? 0 : 1, ks < 7 ? ks + 1 : 0);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[mb][0] = mfma32(qa[2 * mb + (ks >> 2)][ks & 3], kb, acc[mb][0]);
        hsum_part(1, ks, pprev);  // the previous tile's N block 1
        kb = kn;
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][1][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8_t kn = kb;
        if (ks < 7) kn = kread(1, ks + 1);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[mb][1] = mfma32(qa[2 * mb + (ks >> 2)][ks & 3], kb, acc[mb][1]);
        hsum_part(0, ks, pcur);  // this tile's N block 0
        kb = kn;
      }
      // the other 32 heads of an entry sit in lane l ^ 32: both halves get the
      // same sum (float addition commutes)
      {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(pprev), __float_as_uint(pprev), false, false);
        pprev = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(pcur), __float_as_uint(pcur), false, false);
        pcur = __uint_as_float(c[0]) + __uint_as_float(c[1]);
      }
      // lanes 0-31 store this tile's entries 0-31, lanes 32-63 the previous
      // tile's entries 32-63: one store and one count instruction
      const float v = h2 == 0 ? pcur : pprev;
      const int64_t e = h2 == 0 ? tile * TE + l32 : (tile - 1) * TE + 32 + l32;
      if (qok && e >= 0 && e < Vq && (h2 == 0 || tile > 0)) {
        srow[e] = v;
        if (hint) {
          const uint32_t d = f32_key(v) >> DIG_SHIFT;
          atomicAdd(&lds_h[wv][d >> 1], 1u << ((d & 1u) << 4));
        }
      }
    }
  };
  auto body = [&](int64_t tile, auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    stash(BUF);
    if (tile + 2 < ntiles) load(BUF, tile + 2);
    __syncthreads();
    if constexpr (M32) {
      compute32(tile, lds_k[buf]);
    } else if (qok && tile * TE < Vq) {
      float part[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int el = nt * 16 + l16;
        const uint8_t* kr = &lds_k[buf][el * KROW];
        const int sw = kswz<KDT>(el);
        bf16x8_t kbv[KS];
        if constexpr (MX) {
          // block G of the entry: one chunk, scaled by its E8M0 byte
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(kr + ((G ^ sw) * 16));
          const float sc = __uint_as_float(((lds_ks[buf][el] >> (8 * G)) & 0xffu) << 23);
#pragma unroll
          for (int s = 0; s < KS; ++s) kbv[s] = fp4x8_to_bf16x8(v[s], sc);
        } else if constexpr (KDT == DT_FP8) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(kr + (((G * 2 + c) ^ sw) * 16));
            u32x4_t lo, hi;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              lo[2 * q] = fp8x2_to_bf16x2(v[q], false);
              lo[2 * q + 1] = fp8x2_to_bf16x2(v[q], true);
              hi[2 * q] = fp8x2_to_bf16x2(v[2 + q], false);
              hi[2 * q + 1] = fp8x2_to_bf16x2(v[2 + q], true);
            }
            kbv[2 * c] = as_bf16x8(lo);
            kbv[2 * c + 1] = as_bf16x8(hi);
          }
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s)
            kbv[s] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kr + (((G * 4 + s) ^ sw) * 16)));
        }
        // the four head tiles' chains interleaved, each product three
        // products after the one it accumulates onto
        f32x4_t acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma16(qa[mt][s], kbv[s], acc[mt]);
        part[nt] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) part[nt] += wq[mt][r] * relu_bits(acc[mt][r]);
      }
      // every lane group holds the four 16-entry sums: lane (G, l16) takes
      // entry 16 G + l16, so one store covers the tile's 64 scores (256
      // contiguous bytes) and one count instruction their digits
      float v4[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) v4[nt] = sum_rows16(part[nt]);
      const float v = G == 0 ? v4[0] : G == 1 ? v4[1] : G == 2 ? v4[2] : v4[3];
      const int64_t e = tile * TE + G * 16 + l16;
      if (e < Vq) {
        const float sc = KDT == DT_FP8 ? v * __uint_as_float(k_scale[b * N_max + e]) : v;
        srow[e] = sc;
        if (hint) {
          const uint32_t d = f32_key(sc) >> DIG_SHIFT;
          atomicAdd(&lds_h[wv][d >> 1], 1u << ((d & 1u) << 4));
        }
      }
    }
  };
  if constexpr (M32) {
    // bf16 keys: tiles reach LDS by DMA (global_load_lds, one 1 KB piece =
    // four rows per instruction, two per wave and tile; lane i takes row
    // 4 j + i / 16 and fetches the chunk that lands in slot i % 16, i.e. chunk
    // (i % 16) ^ kswz(row)), four buffers, two tiles per barrier: at a barrier
    // every wave's loads of the next two tiles have landed and every wave is
    // done with the two tiles before, whose buffers then take the two after.
    // Entries past the workgroup's largest visible count load entry Vmax - 1.
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    auto issue_tile = [&](int64_t tile) {
      const uint32_t dst = (uint32_t)(uintptr_t)&lds_k[tile & 3][0];
      const uint8_t* base = kb + tile * TE * KROW;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 2 * wvu + u;
        const int r = 4 * j + (l >> 4);
        const int64_t e = min(tile * TE + r, Vmax - 1);
        const uint32_t voff = (uint32_t)((e - tile * TE) * KROW + (((l & 15) ^ kswz<KDT>(r)) * 16));
        dma_row(uniform_ptr(base), voff, __builtin_amdgcn_readfirstlane(dst + (uint32_t)(j * 1024)));
      }
    };
    issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    for (int64_t t0 = 0; t0 < ntiles; t0 += 2) {
      vm_barrier<0>();
      if (t0 + 2 < ntiles) issue_tile(t0 + 2);
      if (t0 + 3 < ntiles) issue_tile(t0 + 3);
      compute32(t0, lds_k[t0 & 3]);
      if (t0 + 1 < ntiles) compute32(t0 + 1, lds_k[(t0 + 1) & 3]);
    }
  } else {
    load(I0{}, 0);
    if (ntiles > 1) load(I1{}, 1);
    for (int64_t it = 0; it < ntiles; it += 2) {
      body(it, I0{});
      if (it + 1 < ntiles) body(it + 1, I1{});
    }
  }
  if constexpr (M32) {
    // the last tile's entries 32-63
    float pl = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pl += wq[4 * mb + (r >> 2)][r & 3] * relu_bits(acc[mb][1][r]);
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(pl), __float_as_uint(pl), false, false);
    pl = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const int64_t e = (ntiles - 1) * TE + 32 + l32;
    if (qok && h2 == 1 && e < Vq) {
      srow[e] = pl;
      if (hint) {
        const uint32_t d = f32_key(pl) >> DIG_SHIFT;
        atomicAdd(&lds_h[wv][d >> 1], 1u << ((d & 1u) << 4));
      }
    }
  }
  if (hint && qok) {  // the row's whole histogram, unpacked (the wave's own LDS: no barrier needed)
    uint32_t* g = hint + row * DIG_BINS;
    for (int i = l; i < DIG_BINS / 2; i += 64) {
      const uint32_t v = lds_h[wv][i];
      *reinterpret_cast<u32x2_t*>(g + 2 * i) = u32x2_t{v & 0xffffu, v >> 16};
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
    for (int r = 0; r < 16; ++r) part += wr[r] * relu_bits(acc[r]);
    part += shfl_xor(part, 32);
    if (g == 0 && ok) srow[e] = part;
  }
}

int indexer_hint_mode(const IndexerLaunch& a) {
  if (a.q_dt == DT_BF16_MXFP4) return TOPK_HINT_ACCUMULATED;  // the row scan, whatever Tq
  if (!(a.H_I == 64 && a.D_I == 128 && a.q_dt == DT_BF16)) return TOPK_HINT_NONE;  // the tiny fp32 scan counts nothing
  return a.Tq >= 8 ? TOPK_HINT_WRITTEN : TOPK_HINT_ACCUMULATED;
}

// Workgroups per row of the low-precision row scan: a few per CU in total,
// each walking a strided run of its row's tiles.
static int64_t lp_per_row(const IndexerLaunch& a, int64_t rows) {
  const int64_t te = a.k_dt == DT_FP8 ? 128 : 256;
  const int64_t ntiles = (a.N_max + te - 1) / te;
  return max((int64_t)1, min(ntiles, (512 + rows - 1) / rows));
}

hipError_t run_indexer(const IndexerLaunch& a, hipStream_t st) {
  const int64_t rows = a.B * a.Tq;
  if (rows == 0 || a.N_max == 0) return hipSuccess;
  if (a.q_dt == DT_BF16_MXFP4) {
    // the FP4 QK path (MXFP4 keys, 64 x 128): the row scan for any query count
    hipLaunchKernelGGL((idx_scan_reg_kernel<DT_MXFP4, true, 0>), dim3((unsigned)lp_per_row(a, rows), (unsigned)rows),
                       dim3(256), 0, st, reinterpret_cast<const uint16_t*>(a.q_idx), a.w,
                       reinterpret_cast<const uint8_t*>(a.k_idx), reinterpret_cast<const uint32_t*>(a.k_scale),
                       a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores, CompressArgs{}, (unsigned)rows, a.hint,
                       a.zero, a.zero_n);
    return hipGetLastError();
  }
  if (a.H_I == 64 && a.D_I == 128 && a.q_dt == DT_BF16 && a.Tq >= 8) {
    // many queries per sequence: key tiles shared by 8 queries per workgroup
    dim3 grid((unsigned)((a.Tq + 7) / 8), (unsigned)a.B);
    auto kern = a.k_dt == DT_FP8 ? idx_prefill_kernel<DT_FP8>
                : a.k_dt == DT_MXFP4 ? idx_prefill_kernel<DT_MXFP4> : idx_prefill_kernel<DT_BF16>;
    hipLaunchKernelGGL(kern, grid, dim3(512), 0, st, reinterpret_cast<const uint16_t*>(a.q_idx), a.w,
                       reinterpret_cast<const uint8_t*>(a.k_idx), reinterpret_cast<const uint32_t*>(a.k_scale),
                       a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores, a.hint, a.zero, a.zero_n);
    return hipGetLastError();
  }
  if (a.H_I == 64 && a.D_I == 128 && a.q_dt == DT_BF16) {
    if (a.N_max == 0) return hipSuccess;  // no entries: nothing to score (the kernels load entry 0 first)
    const int64_t te = a.k_dt == DT_FP8 ? 128 : a.k_dt == DT_MXFP4 ? 256 : IDX_BF16_TE;
    const int64_t ntiles = (a.N_max + te - 1) / te;
    // a few workgroups per CU in total, each walking a strided run of tiles
    // of its row
    int64_t per_row = (512 + rows - 1) / rows;
    per_row = max((int64_t)1, min(ntiles, per_row));
    dim3 grid((unsigned)per_row, (unsigned)rows);
    if (a.k_dt == DT_BF16 && a.Tq % 2 == 0) {
      // query rows of one sequence in pairs: each key tile loaded once for both
      const int64_t groups = rows / 2;
      const int64_t pg = max((int64_t)1, min(ntiles, (512 + groups - 1) / groups));
      hipLaunchKernelGGL((idx_scan_bf16_kernel<2, 0>), dim3((unsigned)pg, (unsigned)groups), dim3(256), 0, st,
                         reinterpret_cast<const uint16_t*>(a.q_idx), a.w, reinterpret_cast<const uint8_t*>(a.k_idx),
                         a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores, CompressArgs{}, (unsigned)groups, a.hint,
                         a.zero, a.zero_n);
      return hipGetLastError();
    }
    if (a.k_dt == DT_FP8 || a.k_dt == DT_MXFP4)
      hipLaunchKernelGGL((a.k_dt == DT_FP8 ? idx_scan_reg_kernel<DT_FP8, false, 0>
                                           : idx_scan_reg_kernel<DT_MXFP4, false, 0>), grid,
                         dim3(256), 0, st, reinterpret_cast<const uint16_t*>(a.q_idx), a.w,
                         reinterpret_cast<const uint8_t*>(a.k_idx), reinterpret_cast<const uint32_t*>(a.k_scale),
                         a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores, CompressArgs{}, (unsigned)rows, a.hint,
                         a.zero, a.zero_n);
    else
      hipLaunchKernelGGL((idx_scan_bf16_kernel<1, 0>), grid, dim3(256), 0, st,
                         reinterpret_cast<const uint16_t*>(a.q_idx), a.w, reinterpret_cast<const uint8_t*>(a.k_idx),
                         a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores, CompressArgs{}, (unsigned)rows, a.hint,
                         a.zero, a.zero_n);
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

// The compression rides in the bf16 scan's launch when the scan takes that
// path and the standalone compression would use the same kernel (any overlap
// compression, or m < 16: one thread per 8 channels), so the two give the
// same bits; otherwise the two run in turn.
hipError_t run_compress_indexer(const CompressLaunch& c, const IndexerLaunch& a, hipStream_t st) {
  const int64_t rows = a.B * a.Tq;
  const int64_t nblk = c.blk_end - c.blk_begin;
  const bool qf4 = a.q_dt == DT_BF16_MXFP4;
  const bool scan_dec = a.H_I == 64 && a.D_I == 128 && ((a.q_dt == DT_BF16 && a.Tq < 8) || qf4);
  const bool comp_ok = c.in_dt == DT_BF16 && (c.out_dt == DT_BF16 || c.out_dt == DT_KV_FP8) &&
                       (c.overlap || c.m < 16) && c.B > 0 && nblk > 0;
  // the compression's grid rows go after the scan's: keep the total within
  // the grid's y limit (at most ceil(threads / 256) rows, whatever the width)
  const bool fits = rows + (c.B * nblk * (c.d / 8) + 255) / 256 <= 65535;
  if (!(scan_dec && comp_ok && fits && rows > 0 && a.N_max > 0)) {
    hipError_t e = run_compress(c, st);
    if (e != hipSuccess) return e;
    return run_indexer(a, st);
  }
  const int64_t cthreads0 = c.B * nblk * (c.d / 8);
  const CompressArgs ca0 = compress_args(c);
  if (a.k_dt == DT_FP8 || a.k_dt == DT_MXFP4) {
    // the low-precision scan: one row per workgroup row, as run_indexer lays it out
    const int64_t te = a.k_dt == DT_FP8 ? 128 : 256;
    const int64_t nt = (a.N_max + te - 1) / te;
    const int64_t gx = max((int64_t)1, min(nt, (512 + rows - 1) / rows));
    const int64_t cy = (cthreads0 + gx * 256 - 1) / (gx * 256);
    const dim3 grid((unsigned)gx, (unsigned)(rows + cy));
    const auto* q = reinterpret_cast<const uint16_t*>(a.q_idx);
    const auto* k = reinterpret_cast<const uint8_t*>(a.k_idx);
    const auto* ks = reinterpret_cast<const uint32_t*>(a.k_scale);
    const bool f8 = a.k_dt == DT_FP8, o8 = c.out_dt == DT_KV_FP8;
    auto kern = f8 ? (o8 ? idx_scan_reg_kernel<DT_FP8, false, DT_KV_FP8> : idx_scan_reg_kernel<DT_FP8, false, DT_BF16>)
                   : qf4 ? (o8 ? idx_scan_reg_kernel<DT_MXFP4, true, DT_KV_FP8>
                               : idx_scan_reg_kernel<DT_MXFP4, true, DT_BF16>)
                         : (o8 ? idx_scan_reg_kernel<DT_MXFP4, false, DT_KV_FP8>
                               : idx_scan_reg_kernel<DT_MXFP4, false, DT_BF16>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q, a.w, k, ks, a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores,
                       ca0, (unsigned)rows, a.hint, a.zero, a.zero_n);
    return hipGetLastError();
  }
  if (a.k_dt != DT_BF16) {
    hipError_t e = run_compress(c, st);
    if (e != hipSuccess) return e;
    return run_indexer(a, st);
  }
  const int64_t ntiles = (a.N_max + IDX_BF16_TE - 1) / IDX_BF16_TE;
  const int nq = a.Tq % 2 == 0 ? 2 : 1;
  const int64_t sy = rows / nq;  // scan rows of the grid
  const int64_t gx = max((int64_t)1, min(ntiles, (512 + sy - 1) / sy));
  const int64_t cthreads = c.B * nblk * (c.d / 8);
  const int64_t cy = (cthreads + gx * 256 - 1) / (gx * 256);  // compression rows of the grid
  const CompressArgs ca = compress_args(c);
  const dim3 grid((unsigned)gx, (unsigned)(sy + cy));
  const auto* q = reinterpret_cast<const uint16_t*>(a.q_idx);
  const auto* k = reinterpret_cast<const uint8_t*>(a.k_idx);
  if (nq == 2) {
    if (c.out_dt == DT_KV_FP8)
      hipLaunchKernelGGL((idx_scan_bf16_kernel<2, DT_KV_FP8>), grid, dim3(256), 0, st, q, a.w, k, a.q_pos, a.n_comp,
                         a.Tq, a.N_max, a.m, a.scores, ca, (unsigned)sy, a.hint, a.zero, a.zero_n);
    else
      hipLaunchKernelGGL((idx_scan_bf16_kernel<2, DT_BF16>), grid, dim3(256), 0, st, q, a.w, k, a.q_pos, a.n_comp,
                         a.Tq, a.N_max, a.m, a.scores, ca, (unsigned)sy, a.hint, a.zero, a.zero_n);
  } else {
    if (c.out_dt == DT_KV_FP8)
      hipLaunchKernelGGL((idx_scan_bf16_kernel<1, DT_KV_FP8>), grid, dim3(256), 0, st, q, a.w, k, a.q_pos, a.n_comp,
                         a.Tq, a.N_max, a.m, a.scores, ca, (unsigned)sy, a.hint, a.zero, a.zero_n);
    else
      hipLaunchKernelGGL((idx_scan_bf16_kernel<1, DT_BF16>), grid, dim3(256), 0, st, q, a.w, k, a.q_pos, a.n_comp,
                         a.Tq, a.N_max, a.m, a.scores, ca, (unsigned)sy, a.hint, a.zero, a.zero_n);
  }
  return hipGetLastError();
}

}  // namespace csa
