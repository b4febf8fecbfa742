// Shared-KV multi-query attention with a sliding window and a sink, for
// gfx950 (MI355X). One kernel template serves CSA sparse decode, CSA sparse
// prefill and HCA dense decode; they differ only in where the rows of the
// attended multiset come from.
//
// What is computed (DeepSeek V4 脱离 CUDA 全栈国产化, deepseek.csdn.net,
// section 二, CSA step 3 "共享 KV MQA" and the HCA paragraph; liduos.com
// deepseek-v4-engineering-tradeoffs, "1M Context 的结构与取舍", for the
// window and the sink): per query token and head h, a softmax over
// l_r = scale * <q_h, r> for every row r of the multiset plus a sink logit,
// then the weighted sum of the rows (each row is key and value at once).
//
// Design (MI355X-first):
//  * A workgroup owns one query token (all 64 heads) and a contiguous range of
//    row slots ("split"). Rows are processed in tiles of 32: the tile is
//    loaded with coalesced 16-byte loads into LDS, row-major with an XOR
//    chunk swizzle, and prefetched into registers one tile ahead.
//  * 8 waves = 4 dims-quarters x 2 head-halves. S^T = R Q^T runs on
//    v_mfma_f32_32x32x16_bf16 with M = rows, N = heads, each wave covering its
//    128 dims; partial logits meet in LDS. Every wave then runs the online
//    softmax for 8 heads (fp32, exp2 domain) and writes P (bf16) to LDS.
//  * O += P R runs on the same MFMA with M = heads, N = dims. Its B operand
//    (8 consecutive rows of one dim) comes from the row-major tile through
//    ds_read_b64_tr_b16, so the tile is stored once for both products.
//  * Splits write unnormalised (O, m, l) partials; a combine kernel merges
//    them in fixed split order and adds the sink. Split sizes depend only on
//    the per-query slot count, so results are batch invariant.
//  * The fp32 instantiation (tiny shapes) uses v_mfma_f32_32x32x2f32 with the
//    same structure; its tile has a padded pitch instead of the swizzle.
#include "common.h"
#include "kernels.h"

namespace csa {

enum { SRC_SPARSE_DEC = 0, SRC_HCA_DEC = 1, SRC_SPARSE_PRE = 2 };

template <typename T>
struct OpTraits;
template <>
struct OpTraits<uint16_t> {  // bf16 storage
  static constexpr int KSTEP = 16, VPL = 8;
  typedef bf16x8_t op_t;
};
template <>
struct OpTraits<float> {
  static constexpr int KSTEP = 2, VPL = 1;
  typedef float op_t;
};

// XOR swizzle of the 16-byte chunk index inside each 128-byte group of a
// tile row. Eight consecutive rows map a chunk to eight different bank
// groups (conflict-free b128 reads of one column by 32 rows), and the four
// rows of a transpose read cover all 32 banks.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

template <typename T, int HP, int D, int NWD, int NWH>
struct AttnCfg {
  static constexpr int NW = NWD * NWH;
  static constexpr int NT = 64 * NW;
  static constexpr int HPW = HP / NWH;  // heads per wave in QK / PV (32)
  static constexpr int DW = D / NWD;    // dims per wave
  static constexpr int ES = sizeof(T);
  static constexpr int KSTEP = OpTraits<T>::KSTEP;
  static constexpr int VPL = OpTraits<T>::VPL;
  static constexpr int KSQ = DW / KSTEP;  // QK k-steps per wave
  static constexpr int TR = 32;           // rows per tile
  static constexpr int CPR = D * ES / 16; // 16-byte chunks per row
  static constexpr int RPP = NT / CPR;    // rows per load pass
  static constexpr int PASSES = TR / RPP;
  static constexpr int HS = HP / NW;      // heads per wave in the softmax
  static constexpr int LPH = 64 / HS;     // lanes per head in the softmax
  static constexpr int RPL = TR / LPH;    // rows per lane in the softmax
  static constexpr int NTD = DW / 32;     // PV N-tiles per wave
  static constexpr int SP = TR + 4;       // Spart pitch (floats)
  static constexpr bool BF = (ES == 2);
  static constexpr int RPITCH = BF ? D * 2 : (D + 1) * 4;  // tile row pitch (bytes)
  static constexpr int PP = BF ? (TR + 8) : (TR + 1);      // P pitch (elements)
  static constexpr int LDS_R = TR * RPITCH;
  static constexpr int LDS_S = NWD * HP * SP * 4;
  static constexpr int LDS_P = HP * PP * ES;
  static_assert(HPW == 32, "one 32-head MFMA tile per wave");
  static_assert(DW % 32 == 0, "dims per wave must fill PV N-tiles");
  static_assert(NT % CPR == 0 && TR % RPP == 0, "tile load mapping");
  static_assert(RPL * LPH == TR && HS * NW == HP, "softmax mapping");
  static_assert(RPL % 4 == 0, "softmax reads in float4");
};

struct RowSrc {
  const uint8_t* kv_comp;
  const uint8_t* kv_win;  // window rows (decode) or raw tokens (prefill)
  const int32_t* idx;
  int64_t N_max;
  int64_t T_tok;
  int top_k;
  int W;
};

// The memory-resident part of a slot (its top-k index); loaded one tile ahead
// of the row itself so the index -> row dependency never stalls a tile.
template <int SRC>
__device__ __forceinline__ int slot_code(const RowSrc& s, int64_t qi, int j) {
  if ((SRC == SRC_SPARSE_DEC || SRC == SRC_SPARSE_PRE) && j < s.top_k) return s.idx[qi * s.top_k + j];
  return 0;
}

template <int SRC, int ROWB>
__device__ __forceinline__ const uint8_t* slot_row(const RowSrc& s, int64_t qi, int j, int code, int lim0,
                                                   int lim1) {
  // lim0: SPARSE: window length; HCA: visible entries V.  lim1: PRE: position p
  if (SRC == SRC_SPARSE_DEC || SRC == SRC_SPARSE_PRE) {
    if (j < s.top_k) {
      const int id = code;
      if (id < 0 || id >= s.N_max) return nullptr;
      int64_t row = (SRC == SRC_SPARSE_DEC) ? qi * s.N_max + id : (int64_t)id;
      return s.kv_comp + row * ROWB;
    }
    int w = j - s.top_k;
    if (SRC == SRC_SPARSE_DEC) {
      if (w >= lim0) return nullptr;
      return s.kv_win + (qi * s.W + w) * ROWB;
    }
    int64_t tok = (int64_t)lim1 - s.W + 1 + w;
    if (tok < 0 || tok >= s.T_tok) return nullptr;
    return s.kv_win + tok * ROWB;
  } else {
    if (j < s.N_max) {
      if (j >= lim0) return nullptr;
      return s.kv_comp + (qi * s.N_max + j) * ROWB;
    }
    int w = j - (int)s.N_max;
    if (w >= lim1) return nullptr;  // HCA: lim1 = window length
    return s.kv_win + (qi * s.W + w) * ROWB;
  }
}

template <typename T, int HP, int D, int NWD, int NWH, int SRC>
__global__ void __launch_bounds__(64 * NWD * NWH)
attn_kernel(const T* __restrict__ q, RowSrc src, const int32_t* __restrict__ win_len,
            const int32_t* __restrict__ n_comp, const int32_t* __restrict__ q_pos, int m_rate,
            const float* __restrict__ sink, float scale_log2, int H, int slots, int split_rows,
            float* __restrict__ part_o, float* __restrict__ part_ml, void* __restrict__ out,
            float* __restrict__ lse, int out_dt) {
  typedef AttnCfg<T, HP, D, NWD, NWH> C;
  typedef typename OpTraits<T>::op_t op_t;
  constexpr int ROWB = D * C::ES;

  __shared__ __attribute__((aligned(16))) uint8_t lds_r[C::LDS_R];
  __shared__ __attribute__((aligned(16))) float lds_s[C::LDS_S / 4];
  __shared__ __attribute__((aligned(16))) T lds_p[HP * C::PP];
  __shared__ __attribute__((aligned(16))) float lds_alpha[HP];
  __shared__ __attribute__((aligned(16))) float lds_ml[HP * 2];
  __shared__ int lds_valid[C::TR];
  __shared__ int lds_flag[C::NW];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int g = l >> 5;       // k-group of the MFMA operand
  const int l32 = l & 31;
  const int dq = wv % NWD;    // dims quarter
  const int hh = wv / NWD;    // head half
  const int64_t qi = blockIdx.x;  // query (decode: sequence)
  const int sp = blockIdx.y;       // split
  const int nsplit = gridDim.y;

  // per-query limits
  int lim0 = 0, lim1 = 0;
  if (SRC == SRC_SPARSE_DEC) {
    lim0 = win_len ? min(max(win_len[qi], 0), src.W) : 0;
  } else if (SRC == SRC_HCA_DEC) {
    if (n_comp) {
      int64_t v = min((int64_t)n_comp[qi], ((int64_t)q_pos[qi] + 1) / m_rate);
      lim0 = (int)max((int64_t)0, min(v, src.N_max));
    }
    lim1 = win_len ? min(max(win_len[qi], 0), src.W) : 0;
  } else {
    lim1 = q_pos[qi];
  }

  const int s_begin = sp * split_rows;
  const int s_end = min(slots, s_begin + split_rows);
  const int ntiles = (s_end > s_begin) ? (s_end - s_begin + C::TR - 1) / C::TR : 0;

  // ---- Q^T operands for this wave (heads hh*32 + l32, dims of quarter dq).
  op_t qb[C::KSQ];
  {
    const int head = hh * 32 + l32;
    const int dim0 = dq * C::DW + g * (C::DW / 2);
    if constexpr (C::BF) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(q) + (qi * H + head) * (int64_t)D + dim0;
#pragma unroll
      for (int s = 0; s < C::KSQ; ++s) {
        u32x4_t v = {0, 0, 0, 0};
        if (head < H) v = ld16(qp + s * 8);
        qb[s] = as_bf16x8(v);
      }
    } else {
      const float* qp = reinterpret_cast<const float*>(q) + (qi * H + head) * (int64_t)D + dim0;
#pragma unroll
      for (int s = 0; s < C::KSQ; ++s) qb[s] = (head < H) ? qp[s] : 0.0f;
    }
  }

  // ---- tile loader: thread handles chunk c of rows rsub + ps*RPP
  const int lc = tid % C::CPR;
  const int lrs = tid / C::CPR;
  u32x4_t pre[C::PASSES];
  int prev[C::PASSES];
  int pcode[C::PASSES];
  auto fetch_code = [&](int tile) {
    const int base = s_begin + tile * C::TR;
#pragma unroll
    for (int ps = 0; ps < C::PASSES; ++ps) {
      const int j = base + lrs + ps * C::RPP;
      pcode[ps] = (j < s_end) ? slot_code<SRC>(src, qi, j) : -1;
    }
  };
  auto fetch = [&](int tile) {
    const int base = s_begin + tile * C::TR;
#pragma unroll
    for (int ps = 0; ps < C::PASSES; ++ps) {
      const int r = lrs + ps * C::RPP;
      const int j = base + r;
      const uint8_t* rp = (j < s_end) ? slot_row<SRC, ROWB>(src, qi, j, pcode[ps], lim0, lim1) : nullptr;
      prev[ps] = rp != nullptr;
      u32x4_t v = {0, 0, 0, 0};
      if (rp) v = ld16(rp + lc * 16);
      pre[ps] = v;
    }
  };
  auto stash = [&]() -> int {
    int any = 0;
#pragma unroll
    for (int ps = 0; ps < C::PASSES; ++ps) {
      const int r = lrs + ps * C::RPP;
      if constexpr (C::BF) {
        const int phys = lc ^ swz(r);
        *reinterpret_cast<u32x4_t*>(lds_r + r * C::RPITCH + phys * 16) = pre[ps];
      } else {
        float* dst = reinterpret_cast<float*>(lds_r + r * C::RPITCH) + lc * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(pre[ps][e]);
      }
      if (lc == 0) lds_valid[r] = prev[ps];
      any |= prev[ps];
    }
    return any;
  };

  f32x16_t oacc[C::NTD];
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nt][r] = 0.0f;

  // softmax state of this lane's head (owned across tiles)
  const int sm_head = wv * C::HS + (l % C::HS);
  const int sm_rg = l / C::HS;
  float m_run = -INFINITY, l_run = 0.0f;

  if (ntiles > 0) {
    fetch_code(0);
    fetch(0);
    if (ntiles > 1) fetch_code(1);
  }
  for (int tile = 0; tile < ntiles; ++tile) {
    const int any = __syncthreads_or(stash());
    if (tile + 1 < ntiles) {
      fetch(tile + 1);  // uses the codes loaded one iteration ago
      if (tile + 2 < ntiles) fetch_code(tile + 2);
    }
    if (!any) continue;

    // ---- S^T partial = R(rows x DW) * Q^T(DW x 32 heads)
    f32x16_t sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
    {
      const int row = l32;
      if constexpr (C::BF) {
        const int c0 = (dq * C::DW + g * (C::DW / 2)) / 8;
        const uint8_t* rb = lds_r + row * C::RPITCH;
        const int sw = swz(row);
#pragma unroll
        for (int s = 0; s < C::KSQ; ++s) {
          u32x4_t a = *reinterpret_cast<const u32x4_t*>(rb + ((c0 + s) ^ sw) * 16);
          sacc = mfma32(as_bf16x8(a), qb[s], sacc);
        }
      } else {
        const float* rb = reinterpret_cast<const float*>(lds_r + row * C::RPITCH) + dq * C::DW + g * (C::DW / 2);
#pragma unroll
        for (int s = 0; s < C::KSQ; ++s) sacc = mfma32(rb[s], qb[s], sacc);
      }
    }
    {
      float* sp_base = lds_s + (dq * HP + hh * 32 + l32) * C::SP + g * 4;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4_t v = {sacc[r4 * 4 + 0], sacc[r4 * 4 + 1], sacc[r4 * 4 + 2], sacc[r4 * 4 + 3]};
        *reinterpret_cast<f32x4_t*>(sp_base + r4 * 8) = v;
      }
    }
    __syncthreads();

    // ---- online softmax for heads [wv*HS, (wv+1)*HS)
    {
      float sv[C::RPL];
#pragma unroll
      for (int i = 0; i < C::RPL; ++i) sv[i] = 0.0f;
#pragma unroll
      for (int d = 0; d < NWD; ++d) {
        const float* src_s = lds_s + (d * HP + sm_head) * C::SP + sm_rg * C::RPL;
#pragma unroll
        for (int i4 = 0; i4 < C::RPL / 4; ++i4) {
          f32x4_t v = *reinterpret_cast<const f32x4_t*>(src_s + i4 * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[i4 * 4 + e] += v[e];
        }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < C::RPL; ++i) {
        const bool ok = lds_valid[sm_rg * C::RPL + i] != 0;
        sv[i] = ok ? sv[i] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[i]);
      }
#pragma unroll
      for (int msk = C::HS; msk < 64; msk <<= 1) tmax = fmaxf(tmax, shfl_xor(tmax, msk));
      const float m_new = fmaxf(m_run, tmax);
      float alpha = 1.0f;
      float psum = 0.0f;
      float pv[C::RPL];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int i = 0; i < C::RPL; ++i) pv[i] = 0.0f;
      } else {
        alpha = exp2f(m_run - m_new);
#pragma unroll
        for (int i = 0; i < C::RPL; ++i) {
          const float p = exp2f(sv[i] - m_new);
          pv[i] = p;  // rounded to bf16 when stored for the PV product
          psum += p;
        }
      }
#pragma unroll
      for (int msk = C::HS; msk < 64; msk <<= 1) psum += shfl_xor(psum, msk);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if constexpr (C::BF) {
        uint32_t w0 = pack_bf16x2(pv[0], pv[1]), w1 = pack_bf16x2(pv[2], pv[3]);
        u32x2_t v = {w0, w1};
        *reinterpret_cast<u32x2_t*>(lds_p + sm_head * C::PP + sm_rg * C::RPL) = v;
      } else {
#pragma unroll
        for (int i = 0; i < C::RPL; ++i) lds_p[sm_head * C::PP + sm_rg * C::RPL + i] = pv[i];
      }
      if (sm_rg == 0) lds_alpha[sm_head] = alpha;
      const bool need = __any(alpha != 1.0f);
      if (l == 0) lds_flag[wv] = need;
    }
    __syncthreads();

    // ---- O = O*alpha + P R   (heads hh*32.., dims dq*DW..)
    {
      int need = 0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) need |= lds_flag[w];
      if (need) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4_t a = *reinterpret_cast<const f32x4_t*>(lds_alpha + hh * 32 + r4 * 8 + g * 4);
#pragma unroll
          for (int nt = 0; nt < C::NTD; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[nt][r4 * 4 + e] *= a[e];
        }
      }
      const int head = hh * 32 + l32;
#pragma unroll
      for (int s = 0; s < C::TR / C::KSTEP; ++s) {
        op_t a;
        if constexpr (C::BF) {
          a = as_bf16x8(*reinterpret_cast<const u32x4_t*>(lds_p + head * C::PP + s * 16 + g * 8));
        } else {
          a = lds_p[head * C::PP + s * 2 + g];
        }
#pragma unroll
        for (int nt = 0; nt < C::NTD; ++nt) {
          op_t b;
          if constexpr (C::BF) {
            const int g16 = l >> 4, j = l & 15;
            const int col = dq * C::DW + nt * 32 + (g16 & 1) * 16 + 4 * (j & 3);
            const int rowa = s * 16 + (g16 >> 1) * 8 + (j >> 2);
            const int rowb = rowa + 4;
            const int ch = col >> 3, cb = (col & 7) * 2;
            auto* pa = (s16x4_t __attribute__((address_space(3)))*)(lds_r + rowa * C::RPITCH + ((ch ^ swz(rowa)) * 16) + cb);
            auto* pb = (s16x4_t __attribute__((address_space(3)))*)(lds_r + rowb * C::RPITCH + ((ch ^ swz(rowb)) * 16) + cb);
            s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pa);
            s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pb);
            u32x4_t bv;
            bv[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
            bv[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
            bv[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
            bv[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
            b = as_bf16x8(bv);
          } else {
            const float* rb = reinterpret_cast<const float*>(lds_r + (s * 2 + g) * C::RPITCH);
            b = rb[dq * C::DW + nt * 32 + l32];
          }
          oacc[nt] = mfma32(a, b, oacc[nt]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue
  if (sm_rg == 0) {
    lds_ml[sm_head * 2 + 0] = m_run;
    lds_ml[sm_head * 2 + 1] = l_run;
  }
  __syncthreads();
  if (part_o != nullptr) {
    // split partials: unnormalised O (relative to m), m, l  (exp2 domain)
    const int64_t pbase = (qi * nsplit + sp) * (int64_t)H;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = hh * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
      if (head >= H) continue;
#pragma unroll
      for (int nt = 0; nt < C::NTD; ++nt)
        part_o[(pbase + head) * D + dq * C::DW + nt * 32 + l32] = oacc[nt][r];
    }
    if (sm_rg == 0 && sm_head < H) {
      part_ml[(pbase + sm_head) * 2 + 0] = m_run;
      part_ml[(pbase + sm_head) * 2 + 1] = l_run;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = hh * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
      if (head >= H) continue;
      const float mh = lds_ml[head * 2], lh = lds_ml[head * 2 + 1];
      const float s2 = sink ? sink[head] * LOG2E_F : -INFINITY;
      const float M = fmaxf(mh, s2);
      float fac = 0.0f;
      if (M != -INFINITY) {
        const float a = exp2f(mh - M);
        fac = a / (lh * a + exp2f(s2 - M));
      }
#pragma unroll
      for (int nt = 0; nt < C::NTD; ++nt) {
        const int64_t o = (qi * H + head) * (int64_t)D + dq * C::DW + nt * 32 + l32;
        const float v = oacc[nt][r] * fac;
        if (out_dt == DT_BF16)
          reinterpret_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16(v);
        else
          reinterpret_cast<float*>(out)[o] = v;
      }
    }
    if (lse && sm_rg == 0 && sm_head < H) {
      const float s2 = sink ? sink[sm_head] * LOG2E_F : -INFINITY;
      const float M = fmaxf(m_run, s2);
      float v = -INFINITY;
      if (M != -INFINITY) v = (M + log2f(l_run * exp2f(m_run - M) + exp2f(s2 - M))) * LN2_F;
      lse[qi * H + sm_head] = v;
    }
  }
}

// Merge split partials in fixed order s = 0..nsplit-1 and add the sink.
// One wave per (query, head); lanes cover the head's dims in float4 chunks.
__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                    const float* __restrict__ sink, int H, int D, int nsplit,
                    void* __restrict__ out, float* __restrict__ lse, int out_dt) {
  const int64_t qi = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (h >= H) return;
  const float s2 = sink ? sink[h] * LOG2E_F : -INFINITY;
  const int64_t row0 = qi * nsplit * (int64_t)H + h;  // partial (qi, s, h) at row0 + s*H
  float M = s2;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(row0 + (int64_t)s * H) * 2]);
  constexpr int MAXC = 2;  // float4 chunks per lane (D <= 512)
  f32x4_t acc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float Z = 0.0f;
  if (M != -INFINITY) {
    Z = exp2f(s2 - M);
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
      f32x4_t v[4][MAXC];
      float a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + u;
        a[u] = 0.0f;
        if (s < nsplit) {
          const int64_t pb = row0 + (int64_t)s * H;
          a[u] = exp2f(part_ml[pb * 2] - M);  // 0 for an empty split (m = -inf)
          Z += part_ml[pb * 2 + 1] * a[u];
#pragma unroll
          for (int c = 0; c < MAXC; ++c) {
            const int d = (c * 64 + l) * 4;
            v[u][c] = d < D ? *reinterpret_cast<const f32x4_t*>(part_o + pb * D + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < MAXC; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[c][e] += v[u][c][e] * a[u];
    }
  }
  const float inv = (M != -INFINITY) ? 1.0f / Z : 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int d = (c * 64 + l) * 4;
    if (d >= D) continue;
    const int64_t o = (qi * H + h) * (int64_t)D + d;
    if (out_dt == DT_BF16) {
      u32x2_t w = {pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv), pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv)};
      *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(out) + o) = w;
    } else {
      f32x4_t w = {acc[c][0] * inv, acc[c][1] * inv, acc[c][2] * inv, acc[c][3] * inv};
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + o) = w;
    }
  }
  if (lse && l == 0) lse[qi * H + h] = (M != -INFINITY) ? (M + log2f(Z)) * LN2_F : -INFINITY;
}

// ----------------------------------------------------------------------------
// host-side launchers
// ----------------------------------------------------------------------------

template <typename T, int HP, int D, int NWD, int NWH, int SRC>
static hipError_t launch_attn(const AttnLaunch& a, hipStream_t st) {
  RowSrc src;
  src.kv_comp = reinterpret_cast<const uint8_t*>(a.kv_comp);
  src.kv_win = reinterpret_cast<const uint8_t*>(a.kv_win);
  src.idx = a.idx;
  src.N_max = a.N_max;
  src.T_tok = a.T_tok;
  src.top_k = a.top_k;
  src.W = a.W;
  dim3 grid((unsigned)a.nq, a.nsplit);
  hipLaunchKernelGGL((attn_kernel<T, HP, D, NWD, NWH, SRC>), grid, dim3(64 * NWD * NWH), 0, st,
                     reinterpret_cast<const T*>(a.q), src, a.win_len, a.n_comp, a.q_pos, a.m_rate, a.sink,
                     a.scale * LOG2E_F, a.H, a.slots, a.split_rows, a.nsplit > 1 ? a.part_o : nullptr,
                     a.part_ml, a.out, a.lse, a.out_dt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)a.nq, (unsigned)((a.H + 3) / 4)), dim3(256), 0, st,
                     a.part_o, a.part_ml, a.sink, a.H, D, a.nsplit, a.out, a.lse, a.out_dt);
  return hipGetLastError();
}

template <int SRC>
static hipError_t dispatch_src(const AttnLaunch& a, hipStream_t st) {
  if (a.kv_dt == DT_BF16 && a.D == 512 && a.H <= 64 && a.H > 32)
    return launch_attn<uint16_t, 64, 512, 4, 2, SRC>(a, st);
  if (a.kv_dt == DT_F32 && a.D == 64 && a.H <= 32)
    return launch_attn<float, 32, 64, 2, 1, SRC>(a, st);
  return hipErrorInvalidValue;
}

hipError_t run_attn(const AttnLaunch& a, hipStream_t st) {
  if (a.nq == 0) return hipSuccess;
  switch (a.src) {
    case 0: return dispatch_src<SRC_SPARSE_DEC>(a, st);
    case 1: return dispatch_src<SRC_HCA_DEC>(a, st);
    default: return dispatch_src<SRC_SPARSE_PRE>(a, st);
  }
}

}  // namespace csa
