"""Seeded synthetic inputs for the CSA/HCA attention path.

This module is shared by the CPU oracle, the GPU tests and the benchmark. It
draws random tensors and encodes them into the storage formats the path reads
(bf16, OCP FP8 E4M3 with a per-row fp32 scale). It contains none of the
method's arithmetic: no compression, no scoring, no selection, no attention.

Seeding: every tensor has a fixed id; its values come from
``PCG64(SeedSequence(entropy=config_seed, spawn_key=(tensor_id, part)))``,
where ``part`` is the sequence index (decode batches) or the 4096-query chunk
index (prefill queries). So any one sequence or chunk can be regenerated alone.

The workload shapes follow the settings the pages give for DeepSeek-V4:
compression rate m=4 (CSA) and m'=128 (HCA), 64 indexer heads of dim 128,
top-k 512 (Flash) / 1024 (Pro), 64 query heads of dim 512 with shared K=V,
a 128-token sliding window (page "Deepseek-V4 技术报告里最值得复现的三个改动",
section 3, configuration block), context lengths 128K and 1M tokens.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

# Fixed tensor ids (never reorder: they are part of every seed).
TID = {
    "Ca": 1, "Cb": 2, "Za": 3, "Zb": 4, "Ba": 5, "Bb": 6,
    "k_idx": 7, "q_idx": 8, "w": 9, "q": 10, "kv_comp": 11, "kv_win": 12,
    "kv_tok": 13, "sink": 14, "q_gamma": 15,
}

QCHUNK = 4096  # prefill query chunk (queries per chunk)


def rng(seed: int, name: str, part: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(TID[name], part))
    return np.random.Generator(np.random.PCG64(ss))


# ----------------------------------------------------------------------------
# Storage encodings (input preparation only).
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    bf16 is the upper 16 bits of an IEEE binary32; rounding adds 0x7FFF plus
    the kept LSB before truncation. Inputs here are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value (kept as float32)."""
    b = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


E4M3_MAX = 448.0


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 (the 'FN' variant: no inf, one NaN code per sign)
    codes as uint8, round to nearest even, saturating at +-448.

    Bit layout (OCP 8-bit floating point spec): sign(1) exp(4, bias 7)
    mantissa(3); exponent field 0 is subnormal with unit 2^-9; the code
    S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.minimum(np.abs(v), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal (and zero): integer multiples of 2^-9; rint is half-to-even
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)  # 8 -> min normal, code 0x08
    nrm = ~sub
    f, x = np.frexp(a[nrm])  # a = f * 2^x, f in [0.5, 1)
    e = x - 1
    q = np.rint(f * 16.0).astype(np.int64)  # in [8, 16]
    up = q == 16
    e = e + up
    q = np.where(up, 8, q)
    code[nrm] = ((e + 7) << 3) | (q - 8)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_quantize_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row (last axis) quantization: scale = amax/448 (1 if the row is all
    zero), codes = e4m3_encode(x / scale). Returns (codes uint8, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    codes = e4m3_encode(x / scale[..., None])
    return codes, scale


# Mixed-precision main KV rows: the RoPE dims (the last 64) stay bf16, the
# other D - 64 dims are E4M3 codes, with no scale.
KV_ROPE_DIMS = 64


def kv_fp8_rows(x: np.ndarray) -> np.ndarray:
    """float32 rows [..., D] -> mixed-precision rows uint8 [..., D - 64 + 128]:
    bytes 0 .. D-65 are the E4M3 codes of dims 0 .. D-65 (e4m3_encode: round to
    nearest even, saturating at +-448), then the 64 RoPE dims as bf16 (round
    to nearest even), two bytes each, little endian."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    nope = D - KV_ROPE_DIMS
    codes = e4m3_encode(x[..., :nope])
    rope = np.ascontiguousarray(bf16_bits(x[..., nope:])).view(np.uint8)
    return np.ascontiguousarray(np.concatenate([codes, rope], axis=-1))


MXFP4_BLOCK = 32


def mxfp4_encode_elems(v: np.ndarray) -> np.ndarray:
    """float -> OCP FP4 E2M1 codes (uint8, low 4 bits), round to nearest even,
    saturating at +-6.

    Bit layout (OCP Microscaling Formats v1.0, FP4 E2M1): sign(1) exp(2, bias 1)
    mantissa(1); exponent field 0 is subnormal (0 or 0.5); no inf or NaN. The
    eight magnitudes in code order are 0, 0.5, 1, 1.5, 2, 3, 4, 6, so the even
    codes are the ones with mantissa bit 0."""
    v = np.asarray(v, dtype=np.float64)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[..., None] - grid)                       # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)          # nearest codes (two on a tie)
    even = np.where((cand % 2 == 0) & (cand < 99), cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1))   # a tie goes to the even code
    sign = (np.signbit(v) & (code > 0)).astype(np.int64)  # -0 encodes as +0
    return (code | (sign << 3)).astype(np.uint8)


def mxfp4_quantize_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """OCP MXFP4 quantization of the last axis in blocks of 32: per block the
    shared E8M0 exponent is floor(log2(amax)) - 2 (2 = emax of E2M1), kept in
    1..254 (scale byte 127 for an all-zero block); elements are E2M1 codes of
    x / 2^(E - 127). Two codes per byte, element 2j in the low nibble of byte j.
    Returns (codes uint8 [..., D/2], scales uint8 [..., D/32])."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % MXFP4_BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (D // MXFP4_BLOCK, MXFP4_BLOCK))
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0, 0.0)
    E = np.clip(ex + 127.0, 1.0, 254.0).astype(np.int64)
    codes = mxfp4_encode_elems(xb / np.exp2(E - 127.0)[..., None]).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, E.astype(np.uint8)


# ----------------------------------------------------------------------------
# Workload configurations.
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Cfg:
    name: str
    seed: int
    kind: str            # "tiny" | "csa_decode" | "csa_prefill" | "hca_decode" | "hca_prefill"
    B: int               # sequences (decode) / 1 (prefill)
    n: int               # context length in tokens
    m: int               # compression rate
    H: int               # query heads of the shared-KV MQA
    D: int               # head dim (shared K=V)
    H_I: int = 0         # indexer heads
    D_I: int = 0         # indexer head dim
    top_k: int = 0
    W: int = 128         # sliding window
    dtype: str = "bf16"  # storage dtype of activations / caches
    k_dtype: str = "bf16"  # indexer key storage
    kv_dtype: str = "bf16"  # main KV rows: "bf16", or "fp8" (E4M3 + bf16 RoPE dims)
    qk_rope: bool = False   # decode step with the query prologue (RMSNorm, RoPE) and output inverse RoPE
    Tq: int = 1          # queries per sequence (decode: the last Tq tokens, e.g. 2 with a drafted token)
    q_fp4: bool = False  # indexer query quantised to MXFP4 by the call (FP4 x FP4 QK; MXFP4 keys)

    @property
    def N(self) -> int:  # compressed entries; tail tokens (n mod m) are dropped
        return self.n // self.m


# The five workloads (tiny parity case, Flash decode 128K, prefill 64K,
# HCA decode 1M, Pro decode 1M).
C1 = Cfg("c1_tiny_fp32", 1, "tiny", B=1, n=1024, m=4, H=4, D=64, H_I=4, D_I=32,
         top_k=16, W=16, dtype="f32", k_dtype="f32", Tq=64)
C2 = Cfg("c2_csa_decode_flash_128k", 2, "csa_decode", B=32, n=131072, m=4, H=64, D=512,
         H_I=64, D_I=128, top_k=512, W=128)
C3 = Cfg("c3_csa_prefill_64k", 3, "csa_prefill", B=1, n=65536, m=4, H=64, D=512,
         H_I=64, D_I=128, top_k=512, W=128, Tq=65536)
C4 = Cfg("c4_hca_decode_1m", 4, "hca_decode", B=16, n=1 << 20, m=128, H=64, D=512, W=128)
C5 = Cfg("c5_csa_decode_pro_1m_fp8", 5, "csa_decode", B=4, n=1 << 20, m=4, H=64, D=512,
         H_I=64, D_I=128, top_k=1024, W=128, k_dtype="fp8")
# C2 with the indexer keys stored as the pages keep them (FP4; OCP MXFP4 here),
# same seed and shapes: a measurement of the next step, not one of the five
C2X = dataclasses.replace(C2, name="c2x_csa_decode_flash_128k_mxfp4", k_dtype="mxfp4")
# HCA prefill of one 64K sequence: single-branch compression at m' = 128
# (512 entries), then every query over all entries it can see plus its window
C6 = Cfg("c6_hca_prefill_64k", 6, "hca_prefill", B=1, n=65536, m=128, H=64, D=512, W=128, Tq=65536)
# C4 and C2 with the main KV cache as the pages store it (RoPE dims bf16, the
# rest FP8), same seeds and shapes
C4F = dataclasses.replace(C4, name="c4f_hca_decode_1m_kv_fp8", kv_dtype="fp8")
C2F = dataclasses.replace(C2, name="c2f_csa_decode_flash_128k_kv_fp8", kv_dtype="fp8")
C3F = dataclasses.replace(C3, name="c3f_csa_prefill_64k_kv_fp8", kv_dtype="fp8")
# C2 with the attention's prologue and epilogue: raw queries are RMS-normalised
# (gamma ~ U(0.5, 1.5)) and rotated at their position, the output is rotated
# back; the logit scale is then 1/sqrt(D)
C2R = dataclasses.replace(C2, name="c2r_csa_decode_flash_128k_qk_rope", qk_rope=True)
# C2 with two query tokens per sequence and step (the current token and a
# drafted one, as a depth-1 multi-token predictor verifies them)
C2M = dataclasses.replace(C2, name="c2m_csa_decode_flash_128k_2tok", Tq=2)
# C2X with both operands of the indexer's QK product in FP4: the bf16 indexer
# query is quantised to MXFP4 inside the call
C2Q = dataclasses.replace(C2X, name="c2q_csa_decode_flash_128k_fp4_qk", q_fp4=True)
CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5, C2X, C6, C4F, C2F, C3F, C2R, C2M, C2Q)}


def scaled(cfg: Cfg, **kw) -> Cfg:
    """Same distributions, smaller (or other) sizes; used by the tests."""
    return dataclasses.replace(cfg, **kw)


def _normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else x.astype(np.float32)


# ---------------------------- decode workloads ------------------------------

def gen_decode_seq(cfg: Cfg, b: int, with_compress: bool = True) -> Dict[str, np.ndarray]:
    """Inputs of one sequence b of a decode workload (CSA or HCA).

    The query is the last token, position p = n-1. kv_comp holds N entries.
    With ``with_compress`` the raw inputs that produce entry N-1 are also
    drawn, so that the step can make that entry itself (it completes at this
    token when m divides n): for CSA the last two blocks (2m tokens, rows for
    tokens n-2m .. n-1, both branches), for HCA the last block (m tokens,
    one branch).
    """
    s, D = cfg.seed, cfg.D
    out: Dict[str, np.ndarray] = {}
    tq = (cfg.Tq,) if cfg.Tq > 1 else ()  # several query tokens: a leading query axis
    out["q"] = _store(_normal(rng(s, "q", b), tq + (cfg.H, D), 1.0 / math.sqrt(D)), cfg.dtype)
    kv = _normal(rng(s, "kv_comp", b), (cfg.N, D))
    # the window buffer holds the latest W + Tq - 1 tokens
    win = _normal(rng(s, "kv_win", b), (min(cfg.W + cfg.Tq - 1, cfg.n), D))
    if cfg.kv_dtype == "fp8":  # uint8 rows [.., D + 64]
        out["kv_comp"], out["kv_win"] = kv_fp8_rows(kv), kv_fp8_rows(win)
    else:
        out["kv_comp"], out["kv_win"] = _store(kv, cfg.dtype), _store(win, cfg.dtype)
    if cfg.kind == "csa_decode":
        HI, DI = cfg.H_I, cfg.D_I
        out["q_idx"] = _store(_normal(rng(s, "q_idx", b), tq + (HI, DI), 1.0 / math.sqrt(DI)), cfg.dtype)
        out["w"] = _normal(rng(s, "w", b), tq + (HI,))
        k = _normal(rng(s, "k_idx", b), (cfg.N, DI))
        if cfg.k_dtype == "fp8":
            codes, scale = e4m3_quantize_rows(k)
            out["k_idx_codes"] = codes
            out["k_scale"] = scale
        elif cfg.k_dtype == "mxfp4":
            codes, scale = mxfp4_quantize_rows(k)
            out["k_idx_codes"] = codes  # [N, D_I/2] two codes per byte
            out["k_scale"] = scale      # [N, D_I/32] E8M0 bytes
        else:
            out["k_idx"] = _store(k, cfg.dtype)
        if with_compress:
            rows = 2 * cfg.m
            for nm in ("Ca", "Cb", "Za", "Zb"):
                out[nm] = _store(_normal(rng(s, nm, b), (rows, D)), cfg.dtype)
    elif cfg.kind == "hca_decode" and with_compress:
        for nm in ("Ca", "Za"):
            out[nm] = _store(_normal(rng(s, nm, b), (cfg.m, D)), cfg.dtype)
    return out


def gen_shared(cfg: Cfg) -> Dict[str, np.ndarray]:
    """Tensors shared by all sequences: the sink logits and compression biases."""
    s = cfg.seed
    out = {}
    if cfg.kind == "tiny":
        out["sink"] = np.zeros((cfg.H,), np.float32)  # sink logit 0
        out["Ba"] = _normal(rng(s, "Ba"), (cfg.m, cfg.D), 0.1)
        out["Bb"] = _normal(rng(s, "Bb"), (cfg.m, cfg.D), 0.1)
    else:
        out["sink"] = _normal(rng(s, "sink"), (cfg.H,))
        out["Ba"] = _normal(rng(s, "Ba"), (cfg.m, cfg.D))
        out["Bb"] = _normal(rng(s, "Bb"), (cfg.m, cfg.D))
    if cfg.qk_rope:
        out["q_gamma"] = rng(s, "q_gamma").uniform(0.5, 1.5, size=cfg.D).astype(np.float32)
    return out


def gen_decode(cfg: Cfg, with_compress: bool = True) -> Dict[str, np.ndarray]:
    """Whole decode batch, stacked along a leading B axis."""
    seqs = [gen_decode_seq(cfg, b, with_compress) for b in range(cfg.B)]
    out = {k: np.stack([sq[k] for sq in seqs]) for k in seqs[0]}
    out.update(gen_shared(cfg))
    return out


# ------------------------- prefill / tiny workloads -------------------------

def gen_prefill_tokens(cfg: Cfg) -> Dict[str, np.ndarray]:
    """Per-token tensors of the single prefill sequence (or the tiny case):
    compression inputs [n, D], raw KV [n, D] for the window, indexer keys
    [N, D_I] (one per compressed entry)."""
    s, n, D = cfg.seed, cfg.n, cfg.D
    hca = cfg.kind == "hca_prefill"  # one branch, no indexer
    out = {}
    for nm in (("Ca", "Za") if hca else ("Ca", "Cb", "Za", "Zb")):
        out[nm] = _store(_normal(rng(s, nm), (n, D)), cfg.dtype)
    kv_tok = _normal(rng(s, "kv_tok"), (n, D))
    out["kv_tok"] = kv_fp8_rows(kv_tok) if cfg.kv_dtype == "fp8" else _store(kv_tok, cfg.dtype)
    if not hca:
        out["k_idx"] = _store(_normal(rng(s, "k_idx"), (cfg.N, cfg.D_I)), cfg.dtype)
    out.update(gen_shared(cfg))
    if hca:
        del out["Bb"]
    return out


def query_positions(cfg: Cfg) -> np.ndarray:
    """Absolute positions of all queries: the last Tq tokens of the sequence."""
    return np.arange(cfg.n - cfg.Tq, cfg.n, dtype=np.int32)


def gen_prefill_queries(cfg: Cfg, chunk: int) -> Dict[str, np.ndarray]:
    """Queries of one chunk of up to QCHUNK consecutive query positions.

    Chunk c covers query slots [c*QCHUNK, min((c+1)*QCHUNK, Tq)); their
    positions are query_positions(cfg)[slots]."""
    s = cfg.seed
    lo = chunk * QCHUNK
    hi = min(lo + QCHUNK, cfg.Tq)
    T = hi - lo
    qscale = 1.0 / math.sqrt(cfg.D) if cfg.kind != "tiny" else 1.0 / 8.0
    out = {
        "q": _store(_normal(rng(s, "q", chunk), (T, cfg.H, cfg.D), qscale), cfg.dtype),
        "q_pos": query_positions(cfg)[lo:hi].copy(),
    }
    if cfg.kind == "hca_prefill":  # no indexer
        return out
    qi_scale = 1.0 / math.sqrt(cfg.D_I) if cfg.kind != "tiny" else 1.0
    out["q_idx"] = _store(_normal(rng(s, "q_idx", chunk), (T, cfg.H_I, cfg.D_I), qi_scale), cfg.dtype)
    g = rng(s, "w", chunk)
    if cfg.kind == "tiny":
        out["w"] = g.uniform(0.0, 1.0, size=(T, cfg.H_I)).astype(np.float32)
    else:
        out["w"] = _normal(g, (T, cfg.H_I))
    return out


def num_chunks(cfg: Cfg) -> int:
    return (cfg.Tq + QCHUNK - 1) // QCHUNK
