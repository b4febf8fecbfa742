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
// v_mfma_f32_16x16x32_bf16 with heads as M (four 16-row tiles) and entries as
// N (16 per wave). The query operand stays in registers for the whole
// workgroup. Keys go HBM -> registers (coalesced) -> LDS (swizzled) -> MFMA
// operands; FP8 keys are decoded exactly to bf16 after the LDS read and their
// scale is applied after the head sum (it is positive). The epilogue never leaves registers: a lane
// holds 16 heads of one entry per tile, applies ReLU and w, sums, and two
// cross-lane shuffles complete the 64-head sum. K dims are visited in a
// permuted order (lane group G covers dims G*32..G*32+31), identical for q and
// k, which leaves the dot products unchanged.
#include <type_traits>

#include "common.h"
#include "compress_entry.h"
#include "kernels.h"

namespace csa {

#ifndef IDX_BF16_TE
#define IDX_BF16_TE 64
#endif

// XOR swizzle of the 16-byte chunk index of key row r in an LDS tile. The
// operand reads take one chunk of each of 16 consecutive rows; with 64 banks
// of 4 bytes those 16 chunks must fall in 16 different 16-byte bank groups.
// bf16 rows are 256 bytes (every row starts in group 0): chunk ^ (r & 15).
// fp8 rows are 128 bytes (odd rows start in group 8): chunk ^ ((r >> 1) & 7).
// MXFP4 rows are 64 bytes (four rows per 256 bytes): chunk ^ ((r >> 2) & 3).
template <int KDT>
__device__ __forceinline__ int kswz(int r) {
  return KDT == DT_FP8 ? ((r >> 1) & 7) : KDT == DT_MXFP4 ? ((r >> 2) & 3) : (r & 15);
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
                     float* __restrict__ scores, CompressArgs ca, unsigned scan_y) {
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
  if ((int64_t)blockIdx.x >= ntiles) return;
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
}

// fp8 (E4M3) keys with a per-entry fp32 scale, 64 heads x 128 dims. Grid:
// (workgroups per row, rows). A workgroup (4 waves) walks tiles of 128
// entries (16 KB) of one query row with a stride of gridDim.x tiles. Tiles
// move HBM -> LDS by DMA (global_load_lds, 1 KB per wave instruction) into a
// ring of four, so the bytes in flight cover the memory latency without
// costing registers; the scales travel with their tile (a 4-byte DMA per
// entry). The 16-byte chunk index is XOR-swizzled (kswz) on the way in, by
// permuting the lanes' source addresses, and read back in the operand layout
// of v_mfma_f32_16x16x32_bf16 with conflict-free ds_read_b128: wave w owns
// entries 32w .. 32w+31 of the tile as two 16-entry N tiles, heads are four
// 16-row M tiles. Codes become bf16 with v_cvt_scalef32_pk_bf16_fp8 (two per
// instruction, exact: every E4M3 value is a bf16 value); the scale multiplies
// the head-weighted sum. Scores collect in LDS and are written out every
// SC_TILES tiles: no store is in flight while DMA waits are counted.
// CO != 0: grid rows past scan_y are a decode step's compression, as in the
// bf16 scan.
template <int KDT, int CO>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
idx_scan_lp_kernel(const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                   const uint8_t* __restrict__ k_idx, const uint32_t* __restrict__ k_scale,
                   const int32_t* __restrict__ q_pos, const int32_t* __restrict__ n_comp, int64_t Tq,
                   int64_t N_max, int m, float* __restrict__ scores, CompressArgs ca, unsigned scan_y) {
  static_assert(KDT == DT_FP8 || KDT == DT_MXFP4, "low-precision keys");
  if constexpr (CO != 0) {
    if (blockIdx.y >= scan_y) {
      compress_entry<DT_BF16, CO>(ca, ((int64_t)(blockIdx.y - scan_y) * gridDim.x + blockIdx.x) * 256 + threadIdx.x);
      return;
    }
  }
  constexpr bool MX = KDT == DT_MXFP4;
  constexpr int H = 64, DI = 128, KS = 4;   // k-steps of 32
  constexpr int KROW = MX ? DI / 2 : DI;    // bytes per key row
  constexpr int TE = MX ? 256 : 128;        // entries per tile
  constexpr int NE = TE / 64;               // 16-entry N tiles per wave
  constexpr int TB = TE * KROW;             // 16 KB
  constexpr int NBUF = 4;                   // 64 KB ring
  constexpr int DPW = TB / 1024 / 4;        // 1 KB DMAs per wave per tile
  constexpr int PER_TILE = DPW + 1;         // + the scales (one dword per entry)
  constexpr int SC_TILES = 2048 / TE;       // score buffer (8 KB)
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k[NBUF][TB];
  __shared__ __attribute__((aligned(16))) uint32_t lds_s[NBUF][TE];  // fp32 scale bits, or four E8M0 bytes
  __shared__ __attribute__((aligned(16))) float lds_sc[SC_TILES][TE];
  __shared__ __attribute__((aligned(16))) float lds_w[H];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = l >> 4, l16 = l & 15;  // k-group (4 x 8 dims) and column of the MFMA operands
  const int64_t row = blockIdx.y;
  const int64_t b = row / Tq;
  int64_t V = min((int64_t)n_comp[b], ((int64_t)q_pos[row] + 1) / m);
  V = max((int64_t)0, min(V, N_max));
  const int64_t ntiles = (V + TE - 1) / TE;
  if ((int64_t)blockIdx.x >= ntiles) return;
  const int64_t nmine = (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;  // tiles of this workgroup

  // query operand A[m = head][k]: lane (head mt*16 + l16, group G) holds dims
  // G*32 + s*8 + 0..7 for k-step s (a fixed permutation of the 128 dims,
  // applied identically to the keys)
  bf16x8_t qa[4][KS];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* qp = q_idx + (row * H + mt * 16 + l16) * DI + G * 32;
#pragma unroll
    for (int s = 0; s < KS; ++s) qa[mt][s] = as_bf16x8(ld16(qp + s * 8));
  }
  if (tid < H) lds_w[tid] = w[row * H + tid];  // visible after the first barrier
  const uint8_t* kb = k_idx + b * N_max * KROW;
  float* srow = scores + row * N_max;

  // DMA j of wave wv fills tile bytes [(DPW wv + j) KB, +1 KB): lane l lands
  // at row r, chunk slot p, and so fetches chunk p ^ kswz(r) of row r
  int drow[DPW];
  uint32_t dcol[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int byte = (DPW * wv + j) * 1024 + 16 * l;
    drow[j] = byte / KROW;
    dcol[j] = (uint32_t)((((byte % KROW) / 16) ^ kswz<KDT>(drow[j])) * 16);
  }
  auto issue = [&](int64_t it) {
    const int64_t tile = blockIdx.x + it * gridDim.x;
    const int buf = (int)(it & (NBUF - 1));
    const int last = (int)min((int64_t)(TE - 1), N_max - 1 - tile * TE);  // rows past the cache repeat its end
    const uint8_t* tb = uniform_ptr(kb + tile * TB);
#pragma unroll
    for (int j = 0; j < DPW; ++j)
      dma_row(tb, (uint32_t)(min(drow[j], last) * KROW) + dcol[j], lds_addr(&lds_k[buf][(DPW * wv + j) * 1024]));
    if (l < TE / 4)  // wave wv moves the scales of entries TE/4 wv .. TE/4 wv + TE/4 - 1
      dma_dword(uniform_ptr(k_scale + b * N_max + tile * TE), (uint32_t)(min(TE / 4 * wv + l, last) * 4),
                lds_addr(&lds_s[buf][TE / 4 * wv]));
  };
  auto flush = [&](int64_t it_begin, int64_t it_end) {  // scores of tiles [it_begin, it_end)
    const int cnt = (int)(it_end - it_begin) * TE;
    for (int k = tid; k < cnt; k += 256) {
      const int64_t tile = blockIdx.x + (it_begin + k / TE) * gridDim.x;
      const int64_t e = tile * TE + (k % TE);
      if (e < V) srow[e] = lds_sc[k / TE][k % TE];
    }
    vm_wait_all();  // the stores retire before DMA counting resumes
  };

  // consume the query here: the compiler's wait for its loads lands before the
  // first DMA, never inside the loop
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qa[mt][s]));
  for (int64_t it = 0; it < nmine && it < NBUF - 1; ++it) issue(it);
  int64_t it_flushed = 0;
  for (int64_t it = 0; it < nmine; ++it) {
    const int ahead = (int)min((int64_t)(NBUF - 2), nmine - 1 - it);  // tiles issued after this one
    if (ahead >= 2)
      vm_barrier<2 * PER_TILE>();
    else if (ahead == 1)
      vm_barrier<PER_TILE>();
    else
      vm_barrier<0>();
    // every wave is done with tile it-1: its buffer takes tile it+NBUF-1
    if (it + NBUF - 1 < nmine) issue(it + NBUF - 1);
    const int buf = (int)(it & (NBUF - 1));
    float part[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      const int el = wv * (16 * NE) + n * 16 + l16;  // entry inside the tile
      const uint8_t* kr = &lds_k[buf][el * KROW];
      const int sw = kswz<KDT>(el);
      bf16x8_t kbv[KS];
      if constexpr (MX) {
        // dims G*32 + s*8 .. : block G, bytes G*16 + s*4 (one chunk), scaled
        // by the block's E8M0 byte G as the fp32 2^(E - 127)
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(kr + ((G ^ sw) * 16));
        const float sc = __uint_as_float(((lds_s[buf][el] >> (8 * G)) & 0xffu) << 23);
#pragma unroll
        for (int s = 0; s < KS; ++s) kbv[s] = fp4x8_to_bf16x8(v[s], sc);
      } else {
        // dims G*32 + s*8 .. : bytes G*32 + s*8, i.e. chunk G*2 + s/2, half s%2
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
      }
      part[n] = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma16(qa[mt][s], kbv[s], acc);
        // accumulator row r of this lane is head mt*16 + G*4 + r
        const f32x4_t wv4 = *reinterpret_cast<const f32x4_t*>(&lds_w[mt * 16 + G * 4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) part[n] += wv4[r] * relu_bits(acc[r]);
      }
    }
#pragma unroll
    for (int n = 0; n < NE; ++n) {
      part[n] = sum_rows16(part[n]);
    }
    if (G == 0) {
#pragma unroll
      for (int n = 0; n < NE; ++n) {
        const int el = wv * (16 * NE) + n * 16 + l16;
        // fp8: sigma_i scales the head-weighted sum (ReLU commutes with a
        // positive scale); MXFP4 scales are already inside the key values
        lds_sc[(it - it_flushed) % SC_TILES][el] = MX ? part[n] : part[n] * __uint_as_float(lds_s[buf][el]);
      }
    }
    if (it + 1 - it_flushed == SC_TILES && it + 1 < nmine) {
      __syncthreads();
      flush(it_flushed, it + 1);
      it_flushed = it + 1;
    }
  }
  __syncthreads();
  flush(it_flushed, nmine);
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
                   int64_t N_max, int m, float* __restrict__ scores) {
  constexpr int H = 64, DI = 128, KS = 4, QB = 8;
  constexpr bool MX = KDT == DT_MXFP4;
  constexpr int KROW = (KDT == DT_FP8) ? DI : MX ? DI / 2 : DI * 2;
  constexpr int TE = 64;
  constexpr int TB = TE * KROW;
  constexpr int NT = 64 * QB;
  constexpr int LPT = (TB + NT * 16 - 1) / (NT * 16);  // 16-byte loads per thread per tile
  static_assert(TB % (NT * 16) == 0 || TB < NT * 16, "tile load mapping");
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][TB];
  __shared__ __attribute__((aligned(16))) uint32_t lds_ks[2][MX ? TE : 1];  // MXFP4: four E8M0 bytes per entry
  __shared__ __attribute__((aligned(16))) float lds_w[QB][H];

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
  if (ntiles == 0) return;

  bf16x8_t qa[4][KS];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* qp = q_idx + (row * H + mt * 16 + l16) * DI + G * 32;
#pragma unroll
    for (int s = 0; s < KS; ++s) qa[mt][s] = as_bf16x8(qok ? ld16(qp + s * 8) : u32x4_t{0, 0, 0, 0});
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
  auto body = [&](int64_t tile, auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    stash(BUF);
    if (tile + 2 < ntiles) load(BUF, tile + 2);
    __syncthreads();
    if (qok && tile * TE < Vq) {
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
        part[nt] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) acc = mfma16(qa[mt][s], kbv[s], acc);
          const f32x4_t wv4 = *reinterpret_cast<const f32x4_t*>(&lds_w[wv][mt * 16 + G * 4]);
#pragma unroll
          for (int r = 0; r < 4; ++r) part[nt] += wv4[r] * relu_bits(acc[r]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float v = sum_rows16(part[nt]);
        const int64_t e = tile * TE + nt * 16 + l16;
        if (G == 0 && e < Vq) srow[e] = KDT == DT_FP8 ? v * __uint_as_float(k_scale[b * N_max + e]) : v;
      }
    }
  };
  load(I0{}, 0);
  if (ntiles > 1) load(I1{}, 1);
  for (int64_t it = 0; it < ntiles; it += 2) {
    body(it, I0{});
    if (it + 1 < ntiles) body(it + 1, I1{});
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

hipError_t run_indexer(const IndexerLaunch& a, hipStream_t st) {
  const int64_t rows = a.B * a.Tq;
  if (rows == 0 || a.N_max == 0) return hipSuccess;
  if (a.H_I == 64 && a.D_I == 128 && a.q_dt == DT_BF16 && a.Tq >= 8) {
    // many queries per sequence: key tiles shared by 8 queries per workgroup
    dim3 grid((unsigned)((a.Tq + 7) / 8), (unsigned)a.B);
    auto kern = a.k_dt == DT_FP8 ? idx_prefill_kernel<DT_FP8>
                : a.k_dt == DT_MXFP4 ? idx_prefill_kernel<DT_MXFP4> : idx_prefill_kernel<DT_BF16>;
    hipLaunchKernelGGL(kern, grid, dim3(512), 0, st, reinterpret_cast<const uint16_t*>(a.q_idx), a.w,
                       reinterpret_cast<const uint8_t*>(a.k_idx), reinterpret_cast<const uint32_t*>(a.k_scale),
                       a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores);
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
                         a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores, CompressArgs{}, (unsigned)groups);
      return hipGetLastError();
    }
    if (a.k_dt == DT_FP8 || a.k_dt == DT_MXFP4)
      hipLaunchKernelGGL((a.k_dt == DT_FP8 ? idx_scan_lp_kernel<DT_FP8, 0> : idx_scan_lp_kernel<DT_MXFP4, 0>), grid,
                         dim3(256), 0, st, reinterpret_cast<const uint16_t*>(a.q_idx), a.w,
                         reinterpret_cast<const uint8_t*>(a.k_idx), reinterpret_cast<const uint32_t*>(a.k_scale),
                         a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores, CompressArgs{}, (unsigned)rows);
    else
      hipLaunchKernelGGL((idx_scan_bf16_kernel<1, 0>), grid, dim3(256), 0, st,
                         reinterpret_cast<const uint16_t*>(a.q_idx), a.w, reinterpret_cast<const uint8_t*>(a.k_idx),
                         a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores, CompressArgs{}, (unsigned)rows);
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
  const bool scan_dec = a.H_I == 64 && a.D_I == 128 && a.q_dt == DT_BF16 && a.Tq < 8;
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
    auto kern = f8 ? (o8 ? idx_scan_lp_kernel<DT_FP8, DT_KV_FP8> : idx_scan_lp_kernel<DT_FP8, DT_BF16>)
                   : (o8 ? idx_scan_lp_kernel<DT_MXFP4, DT_KV_FP8> : idx_scan_lp_kernel<DT_MXFP4, DT_BF16>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q, a.w, k, ks, a.q_pos, a.n_comp, a.Tq, a.N_max, a.m, a.scores,
                       ca0, (unsigned)rows);
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
                         a.Tq, a.N_max, a.m, a.scores, ca, (unsigned)sy);
    else
      hipLaunchKernelGGL((idx_scan_bf16_kernel<2, DT_BF16>), grid, dim3(256), 0, st, q, a.w, k, a.q_pos, a.n_comp,
                         a.Tq, a.N_max, a.m, a.scores, ca, (unsigned)sy);
  } else {
    if (c.out_dt == DT_KV_FP8)
      hipLaunchKernelGGL((idx_scan_bf16_kernel<1, DT_KV_FP8>), grid, dim3(256), 0, st, q, a.w, k, a.q_pos, a.n_comp,
                         a.Tq, a.N_max, a.m, a.scores, ca, (unsigned)sy);
    else
      hipLaunchKernelGGL((idx_scan_bf16_kernel<1, DT_BF16>), grid, dim3(256), 0, st, q, a.w, k, a.q_pos, a.n_comp,
                         a.Tq, a.N_max, a.m, a.scores, ca, (unsigned)sy);
  }
  return hipGetLastError();
}

}  // namespace csa
