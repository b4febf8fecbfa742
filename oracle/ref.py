"""CPU oracle of the DeepSeek-V4 CSA/HCA attention hot path — TEST INFRASTRUCTURE.

This is the plain, slow, float64 NumPy statement of what the path computes.
It is only for checking: the tests, the smoke check and the CPU baseline leg of
the benchmark call it; the product (the HIP library and its Python binding)
never imports it. It shares no code with the GPU path.

Sources (web pages on DeepSeek-V4, cited by title and section):
  [CSDN]  "DeepSeek V4 脱离 CUDA 全栈国产化：1.6T MoE 逐层拆解 + 昇腾迁移数据"
          (deepseek.csdn.net), section 二 "CSA + HCA 混合注意力", sub-sections
          CSA (three steps, the CComp_i equation), HCA, 其他辅助设计.
  [LIDUOS] liduos.com "deepseek-v4-engineering-tradeoffs", section
          "1M Context 的结构与取舍" (HCA / CSA / SWA channels, attention sink).
  [LQNN]  "Deepseek-V4 技术报告里最值得复现的三个改动" (m.lqnn.cn), section 3
          (configuration block: m=4, 64 indexer heads x 128, top_k 512,
          m'=128, 64 query heads x 512, sliding window 128) and section 5
          (tokens beyond the last multiple of m are not compressed).
  [WIKI]  "DeepSeek V4 技术深度 …（DeepTech 深科技）", 5 大架构 item 1
          (CSA every 4 tokens, HCA every 128).
  [CSDN] section 八 "MegaMoE 超级内核与训练稳定性" carries the
          batch-invariance remark (a token's output does not depend on where
          it sits in a batch); every function here works on one row at a time.

Readings where the pages are silent or garbled (each also listed in the design
notes of the repository):
  R1  compression softmax runs over the m tokens of a block, separately for
      every channel; the bias B is indexed by position-in-block.
  R2  the overlapped "b" branch covers the previous block (i-1); block 0 has
      no b term.
  R3  the two branches have separate softmaxes, as the equation prints them;
      ``joint=True`` gives one softmax over both blocks' 2m logits.
  R4  a query at position p sees entries i < V(p) = min(N, floor((p+1)/m)).
  R5  indexer score s_i = sum_h w_h * ReLU(sigma_i * <q_h, k_i>), sigma_i the
      per-entry fp8 scale (1 for bf16/fp32 keys).
  R7  top-k keeps K' = min(k, V) entries, ties to the lower index, returned in
      ascending index order and padded with -1.
  R8  the window is the raw tokens max(0, p-W+1) .. p, current token included.
  R9  one softmax over selected entries, window rows and the sink; rows that
      appear in both sets are counted twice.
  R10 the sink is a per-head logit with a zero value vector.
  R11 queries are pre-scaled by the generator; the logit scale tau is a
      parameter (1.0 in all workloads).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# Storage decoding (the oracle's own, from the format definitions).
# ----------------------------------------------------------------------------

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 (FN variant) code -> value, from the bit definition:
    sign bit, 4-bit exponent with bias 7, 3-bit mantissa; exponent field 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(F64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0))
    v = s * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


def rms_norm(x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis ([CSDN] 其他辅助设计: QK normalisation
    before the core attention): x / sqrt(mean(x^2) + eps) * gamma."""
    x = np.asarray(x, F64)
    y = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return y if gamma is None else y * np.asarray(gamma, F64)


def rope_rotate(x, pos, rope_dims: int = 64, theta: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """Partial rotary position encoding ([CSDN] 其他辅助设计: only the last
    64 dims are rotated; [LIDUOS] 1M Context 的结构与取舍: the output side takes the inverse
    rotation). With R = rope_dims and s = D - R, the pair (x[s+2i], x[s+2i+1])
    is rotated by the angle p * theta^(-2i/R) (by minus that angle with
    inverse); the other dims pass through. x: [T, ..., D]; pos: [T]."""
    x = np.array(x, F64)
    D = x.shape[-1]
    s = D - rope_dims
    i = np.arange(rope_dims // 2, dtype=F64)
    inv_freq = np.power(F64(theta), -2.0 * i / rope_dims)
    ang = np.asarray(pos, F64).reshape((-1,) + (1,) * (x.ndim - 1)) * inv_freq  # [T, 1.., R/2]
    if inverse:
        ang = -ang
    c, sn = np.cos(ang), np.sin(ang)
    a, b = x[..., s::2].copy(), x[..., s + 1::2].copy()
    x[..., s::2] = a * c - b * sn
    x[..., s + 1::2] = a * sn + b * c
    return x


def kv_fp8_decode(rows: np.ndarray, D: int) -> np.ndarray:
    """Mixed-precision main-KV row -> values (the pages keep the RoPE dims in
    BF16 and the rest in FP8): bytes 0 .. D-65 are OCP E4M3 codes of dims
    0 .. D-65; the next 128 bytes are dims D-64 .. D-1 as bf16, little endian
    (value = the bf16 bits as the upper half of an IEEE binary32)."""
    r = np.asarray(rows, dtype=np.uint8)
    nope = D - 64
    assert r.shape[-1] == nope + 128
    lo = r[..., nope::2].astype(np.uint32)
    hi = r[..., nope + 1::2].astype(np.uint32)
    rope = ((hi << 24) | (lo << 16)).astype(np.uint32).view(np.float32).astype(F64)
    return np.concatenate([e4m3_decode(r[..., :nope]), rope], axis=-1)


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """OCP MXFP4 (Microscaling Formats v1.0) -> values, from the format
    definition. Element: FP4 E2M1, sign(1) exp(2, bias 1) mantissa(1), exponent
    field 0 subnormal (mantissa/2), so the magnitudes are 0, 0.5, 1, 1.5, 2, 3,
    4, 6. Two elements per byte, element 2j in the low nibble of byte j. One
    E8M0 scale byte E per block of 32 elements scales it by 2^(E - 127); the
    byte 255 is NaN. codes [..., D/2] uint8, scales [..., D/32] uint8 ->
    [..., D] float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    nib = np.stack([c & 0xF, c >> 4], axis=-1).reshape(c.shape[:-1] + (2 * c.shape[-1],))
    e = (nib >> 1) & 3
    mt = (nib & 1).astype(F64)
    mag = np.where(e == 0, 0.5 * mt, (1.0 + 0.5 * mt) * np.exp2(e.astype(F64) - 1.0))
    v = np.where(nib & 8, -mag, mag)
    E = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    sc = np.where(E == 255, np.nan, np.exp2(E.astype(F64) - 127.0))
    blk = v.reshape(v.shape[:-1] + (E.shape[-1], v.shape[-1] // E.shape[-1]))
    return (blk * sc[..., None]).reshape(v.shape)


def mxfp4_quantize(x) -> Tuple[np.ndarray, np.ndarray]:
    """Values -> OCP MXFP4 (Microscaling Formats v1.0, conversion of a block of
    32 wider values), along the last axis. The block's shared exponent is
    floor(log2 max|x|) minus 2, the largest exponent of an E2M1 element, kept
    as an E8M0 byte in 1..254 (127 for an all-zero block). Each value over
    the block scale is rounded to the nearest E2M1 value, ties to the even
    code: the grid spacing is 0.5 below 2, 1 from 2 to 4 and 2 above, so this
    is round-half-even of x / spacing; magnitudes beyond 6 saturate at 6, and
    a value that rounds to zero keeps no sign. Elements are packed two per
    byte, element 2j in the low nibble of byte j. Serves the query of the
    indexer's FP4 QK path ([CSDN] CSA step 2; reading R20).
    x [..., D] (D a multiple of 32) -> (codes uint8 [..., D/2], scales uint8
    [..., D/32])."""
    x = np.asarray(x, F64)
    D = x.shape[-1]
    assert D % 32 == 0
    xb = x.reshape(x.shape[:-1] + (D // 32, 32))
    amax = np.abs(xb).max(axis=-1)
    _, ex = np.frexp(amax)  # amax = f 2^ex with f in [0.5, 1): floor(log2 amax) = ex - 1
    E = np.where(amax > 0, np.clip(ex - 1 - 2 + 127, 1, 254), 127).astype(np.int64)
    y = xb * np.exp2(127.0 - E)[..., None]
    a = np.abs(y)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    mag = np.minimum(np.rint(a / step) * step, 6.0)
    code = np.where(mag < 2.0, 2.0 * mag, np.where(mag < 4.0, mag + 2.0, 0.5 * mag + 4.0)).astype(np.int64)
    code = code | (((y < 0) & (code > 0)).astype(np.int64) << 3)
    code = code.reshape(x.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, E.astype(np.uint8)


# ----------------------------------------------------------------------------
# A1: CSA / HCA KV compression  ([CSDN] CSA step 1, the CComp_i equation;
# [LQNN] section 5 for the dropped tail; [WIKI] item 1 for the rates).
# ----------------------------------------------------------------------------

def _softmax_axis0(z: np.ndarray) -> np.ndarray:
    zmax = z.max(axis=0, keepdims=True)
    e = np.exp(z - zmax)
    return e / e.sum(axis=0, keepdims=True)


def compress(Ca, Cb, Za, Zb, Ba, Bb, m: int, overlap: bool = True, joint: bool = False,
             blocks: Optional[range] = None) -> np.ndarray:
    """Compressed entries of one sequence.

    Ca, Cb, Za, Zb: [n, d] per-token candidate values and logits; Ba, Bb:
    [m, d] positional biases. Entry i (i < N = floor(n/m)) for channel c is
        sum_j softmax_j(Za[mi+j,c] + Ba[j,c]) * Ca[mi+j,c]
      + sum_j softmax_j(Zb[m(i-1)+j,c] + Bb[j,c]) * Cb[m(i-1)+j,c]   (i >= 1)
    Returns [len(blocks), d] float64 (all N blocks by default).
    """
    Ca, Cb, Za, Zb = (np.asarray(a, F64) if a is not None else None for a in (Ca, Cb, Za, Zb))
    Ba = np.asarray(Ba, F64)
    Bb = np.asarray(Bb, F64) if Bb is not None else None
    n, d = Ca.shape
    N = n // m  # tail tokens (n mod m) form no entry
    if blocks is None:
        blocks = range(N)
    out = np.zeros((len(blocks), d), F64)
    for r, i in enumerate(blocks):
        if not (0 <= i < N):
            raise ValueError("block out of range")
        a = slice(m * i, m * i + m)
        za = Za[a] + Ba
        has_b = overlap and i >= 1
        if has_b:
            b = slice(m * (i - 1), m * i)
            zb = Zb[b] + Bb
        if joint and has_b:
            wts = _softmax_axis0(np.concatenate([za, zb], axis=0))
            out[r] = (wts * np.concatenate([Ca[a], Cb[b]], axis=0)).sum(axis=0)
        else:
            out[r] = (_softmax_axis0(za) * Ca[a]).sum(axis=0)
            if has_b:
                out[r] += (_softmax_axis0(zb) * Cb[b]).sum(axis=0)
    return out


# ----------------------------------------------------------------------------
# A2: lightning indexer score ([CSDN] CSA step 2; [LQNN] section 3 for the
# 64 x 128 indexer; head weighting per reading R5).
# ----------------------------------------------------------------------------

def visible(p: int, n_comp: int, m: int) -> int:
    """V(p) = min(n_comp, floor((p+1)/m))  (reading R4)."""
    return max(0, min(int(n_comp), (int(p) + 1) // m))


def indexer_scores(q_idx, w, k_idx, V: int, k_scale=None, q_fp4: bool = False) -> np.ndarray:
    """s_i = sum_h w_h * max(0, sigma_i * <q_h, k_i>) for i < V.

    q_idx [H_I, D_I], w [H_I], k_idx [>=V, D_I] (values), k_scale [>=V] or None.
    q_fp4: the FP4 QK path with both operands in FP4 (reading R20): every head
    row of the query is first quantised to MXFP4 (mxfp4_quantize) and the
    product takes its decoded values.
    """
    q = np.asarray(q_idx, F64)
    if q_fp4:
        q = mxfp4_decode(*mxfp4_quantize(q))
    k = np.asarray(k_idx, F64)[:V]
    dots = k @ q.T  # [V, H_I]
    if k_scale is not None:
        dots = dots * np.asarray(k_scale, F64)[:V, None]
    return (np.maximum(dots, 0.0) * np.asarray(w, F64)[None, :]).sum(axis=1)


# ----------------------------------------------------------------------------
# A3: top-k selection ([CSDN] CSA step 2: keep the top-k compressed blocks;
# [LQNN] section 3 top_k 512; ties and order per reading R7).
# ----------------------------------------------------------------------------

def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the K' = min(k, V) largest scores (ties: lower index first),
    in ascending index order, padded with -1 to length k."""
    s = np.asarray(scores, F64)
    V = s.shape[0]
    kk = min(k, V)
    order = np.lexsort((np.arange(V), -s))  # primary: score desc, secondary: index asc
    sel = np.sort(order[:kk])
    out = np.full(k, -1, np.int64)
    out[:kk] = sel
    return out


# ----------------------------------------------------------------------------
# A4 / A5 / A6: shared-KV MQA with a sink ([CSDN] CSA step 3, HCA paragraph;
# [LIDUOS] the SWA channel and the attention sink).
# ----------------------------------------------------------------------------

def attend(q, rows, sink, tau: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One query token, all heads, over a row multiset (each row is both key
    and value) plus a per-head sink logit with a zero value.

    q [H, D], rows [R, D], sink [H] -> (o [H, D], lse [H]) with
      l_r = tau <q_h, r>,  M = max(sink_h, max_r l_r),
      Z = e^{sink_h - M} + sum_r e^{l_r - M},  o_h = sum_r e^{l_r - M} r / Z,
      lse_h = M + ln Z.
    """
    q = np.asarray(q, F64)
    R = np.asarray(rows, F64).reshape(-1, q.shape[1])
    sink = np.asarray(sink, F64)
    logits = tau * (q @ R.T)  # [H, R]
    if R.shape[0] > 0:
        M = np.maximum(sink, logits.max(axis=1))
    else:
        M = sink.copy()
    e = np.exp(logits - M[:, None])
    Z = np.exp(sink - M) + e.sum(axis=1)
    o = (e @ R) / Z[:, None]
    return o, M + np.log(Z)


def window_rows(kv_tok, p: int, W: int) -> np.ndarray:
    """Raw rows of tokens max(0, p-W+1) .. p (reading R8)."""
    return np.asarray(kv_tok[max(0, p - W + 1):p + 1], F64)


def sparse_rows(kv_comp, idx) -> np.ndarray:
    idx = np.asarray(idx)
    return np.asarray(np.asarray(kv_comp)[idx[idx >= 0]], F64)


# ----------------------------------------------------------------------------
# Whole-path drivers (per sequence / per query), in the pages' order:
# compress -> score -> select -> attend.
# ----------------------------------------------------------------------------

def csa_query(q, q_idx, w, kv_comp, k_idx, p: int, n_comp: int, m: int, top_k: int,
              win, sink, k_scale=None, tau: float = 1.0, q_fp4: bool = False):
    """One CSA query at position p: returns (idx, o, lse, scores)."""
    V = visible(p, n_comp, m)
    s = indexer_scores(q_idx, w, k_idx, V, k_scale, q_fp4=q_fp4)
    idx = topk_select(s, top_k)
    rows = np.concatenate([sparse_rows(kv_comp, idx), np.asarray(win, F64)], axis=0)
    o, lse = attend(q, rows, sink, tau)
    return idx, o, lse, s


def hca_query(q, kv_comp, p: int, n_comp: int, m: int, win, sink, tau: float = 1.0):
    """One HCA query: dense attention over all V(p) entries plus the window."""
    V = visible(p, n_comp, m)
    rows = np.concatenate([np.asarray(kv_comp, F64)[:V], np.asarray(win, F64)], axis=0)
    return attend(q, rows, sink, tau)
