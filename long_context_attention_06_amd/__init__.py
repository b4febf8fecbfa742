"""Python binding of libcsa_hca.so: DeepSeek-V4 CSA/HCA hybrid attention on
MI355X (gfx950).

Each function has the name of the C entry point it calls (include/csa_hca.h)
and only marshals arguments: shapes are read from the tensors, pointers and
the current HIP stream are passed through, and a non-zero status becomes a
CsaError. All computation happens in the library's kernels. Importing this
package fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa_hca.so")

F32, BF16, FP8_E4M3, MXFP4, KV_FP8, BF16_MXFP4 = 0, 1, 2, 3, 4, 5
OK, INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP_ERROR = 0, -1, -2, -3, -4
OVERLAP, JOINT_SOFTMAX = 1, 2
RMSNORM, ROPE, ROPE_INVERSE = 1, 2, 4


class CsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m long_context_attention_06_amd.build`")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "csa_hca_version": ([], _i32),
    "csa_last_error": ([], ctypes.c_char_p),
    "csa_compress": ([_vp] * 7 + [_i64, _i64, _i64, _i32, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _vp], _i32),
    "indexer_score": ([_vp] * 6 + [_i64, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp], _i32),
    "indexer_topk": ([_vp] * 3 + [_i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "csa_compress_indexer_score": ([_vp] * 7 + [_i64, _i64, _i64, _i32, _i32, _i64, _i64, _i64, _i32, _i32, _i32]
                                   + [_vp] * 6 + [_i64, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp], _i32),
    "csa_compress_indexer_score_topk": ([_vp] * 7 + [_i64, _i64, _i64, _i32, _i32, _i64, _i64, _i64, _i32, _i32,
                                                      _i32] + [_vp] * 6 + [_i64, _i64, _i32, _i32, _i64, _i32, _i32,
                                                                           _i32, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "csa_decode_step": ([_vp] * 6 + [_i64, _i64, _i32, _i32, _i64, _i64, _i32, _i32] + [_vp] * 6
                        + [_i64, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _i32] + [_vp] * 5
                        + [_f32, _i32, _i32, _i32, _i32, _i32] + [_vp] * 5 + [_sz, _vp], _i32),
    "csa_decode_step_workspace_bytes": ([_i64, _i64, _i64, _i32, _i32, _i32, _i32], _sz),
    "csa_trace_phases": ([ctypes.POINTER(ctypes.c_void_p), _i32], _i32),
    "csa_decode_step_qk": ([_vp] * 6 + [_i64, _i64, _i32, _i32, _i64, _i64, _i32, _i32] + [_vp] * 6
                           + [_i64, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _i32] + [_vp] * 5
                           + [_f32, _i32, _i32, _i32, _i32, _i32] + [_vp] * 5 + [_f32, _i32, _f32, _i32]
                           + [_vp, _sz, _vp], _i32),
    "csa_decode_step_qk_workspace_bytes": ([_i64, _i64, _i64, _i32, _i32, _i32, _i32], _sz),
    "csa_decode_step_noalloc": ([_vp] * 6 + [_i64, _i64, _i32, _i32, _i64, _i64, _i32, _i32] + [_vp] * 6
                                + [_i64, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _i32] + [_vp] * 5
                                + [_f32, _i32, _i32, _i32, _i32, _i32] + [_vp] * 5, _i32),
    "indexer_topk_workspace_bytes": ([_i64, _i64, _i64, _i32], _sz),
    "indexer_score_topk": ([_vp] * 6 + [_i64, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                        _vp], _i32),
    "indexer_score_topk_workspace_bytes": ([_i64, _i64, _i64, _i32], _sz),
    "sparse_mqa_decode": ([_vp] * 6 + [_f32, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                       _vp], _i32),
    "sparse_mqa_decode_workspace_bytes": ([_i64, _i32, _i32, _i32, _i32], _sz),
    "sparse_mqa_decode_multi": ([_vp] * 6 + [_f32, _i64, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                                             _vp, _sz, _vp], _i32),
    "sparse_mqa_decode_multi_workspace_bytes": ([_i64, _i64, _i32, _i32, _i32, _i32], _sz),
    "sparse_mqa_prefill": ([_vp] * 6 + [_f32, _i64, _i32, _i32, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                        _sz, _vp], _i32),
    "sparse_mqa_prefill_workspace_bytes": ([_i64, _i32, _i32, _i32, _i32], _sz),
    "hca_dense_mqa": ([_vp] * 4 + [_i32, _vp, _vp, _vp, _f32, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp,
                                   _vp, _sz, _vp], _i32),
    "hca_dense_mqa_workspace_bytes": ([_i64, _i32, _i32, _i64, _i32], _sz),
    "hca_decode_step": ([_vp] * 3 + [_i64, _i64, _i32, _i32, _i64, _i64, _i32] + [_vp] * 4 + [_i32] + [_vp] * 3
                        + [_f32, _i64, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "hca_decode_step_workspace_bytes": ([_i64, _i32, _i32, _i64, _i32], _sz),
    "hca_prefill": ([_vp] * 5 + [_f32, _i64, _i32, _i32, _i64, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                 _vp], _i32),
    "hca_prefill_workspace_bytes": ([_i64, _i32, _i32, _i64, _i32], _sz),
    "qk_norm_rope": ([_vp] * 4 + [_i64, _i32, _i32, _i32, _f32, _f32, _i32, _i32, _vp], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTS = tuple(_SIGS)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _dt(t) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    if t.dtype == torch.float4_e2m1fn_x2:  # MXFP4 codes, two per byte (indexer keys)
        return MXFP4
    raise ValueError(f"unsupported dtype {t.dtype}")


def _qdt(q_idx, q_fp4: bool) -> int:
    """Indexer query dtype: with q_fp4 a bf16 query that the call quantises
    to MXFP4 for the FP4 x FP4 QK product (MXFP4 keys only)."""
    if q_fp4:
        if q_idx.dtype != torch.bfloat16:
            raise ValueError("q_fp4 takes a bf16 query")
        return BF16_MXFP4
    return _dt(q_idx)


def _kv_dt(q, kv) -> int:
    """Row dtype of a KV cache: uint8 rows D + 64 bytes wide are the
    mixed-precision layout (D - 64 E4M3 bytes, then 64 bf16 RoPE dims) read
    with bf16 queries; otherwise the rows have the query's dtype."""
    if kv is not None and kv.dtype == torch.uint8 and kv.shape[-1] == q.shape[-1] + 64:
        return KV_FP8
    return _dt(q)


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(rc: int) -> None:
    if rc != OK:
        raise CsaError(rc, lib.csa_last_error().decode())


def _ws(nbytes: int, ws, device) -> tuple:
    if nbytes == 0:
        return None, 0
    if ws is None:
        # zero-filled: a top-k workspace whose digit histogram starts at zero
        # takes the fast path from the first call (results never depend on it)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        return ws, ws.numel() * ws.element_size()
    return ws, ws.numel() * ws.element_size()


def version() -> int:
    return lib.csa_hca_version()


# ---------------------------------------------------------------- compression

def csa_compress(Ca, Cb, Za, Zb, Ba, Bb, out, *, m: int, tok_begin: int = 0, blk_begin: int = 0,
                 blk_end: Optional[int] = None, overlap: bool = True, joint: bool = False,
                 stream=None) -> None:
    """Ca, Cb, Za, Zb: [B, n_rows, d]; Ba, Bb: [m, d] fp32; out: [B, out_cap, d]."""
    B, n_rows, d = Ca.shape
    out_cap = out.shape[1]
    if blk_end is None:
        blk_end = (tok_begin + n_rows) // m
    flags = (OVERLAP if overlap else 0) | (JOINT_SOFTMAX if joint else 0)
    out_dt = KV_FP8 if out.dtype == torch.uint8 and out.shape[-1] == d + 64 else _dt(out)
    _check(lib.csa_compress(_ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb), _ptr(out), B, n_rows,
                            tok_begin, d, m, blk_begin, blk_end, out_cap, flags, _dt(Ca), out_dt,
                            _stream(stream)))


# -------------------------------------------------------------------- indexer

def indexer_score(q_idx, w, k_idx, k_scale, q_pos, n_comp, scores, *, m: int, q_fp4: bool = False,
                  stream=None) -> None:
    """q_idx [B, Tq, H_I, D_I]; w [B, Tq, H_I]; k_idx [B, N_max, D_I] (MXFP4: [B, N_max, D_I/2] of
    float4_e2m1fn_x2); k_scale: fp8 keys [B, N_max] fp32, MXFP4 keys [B, N_max, D_I/32] E8M0 bytes,
    else None; q_pos [B, Tq] int32; n_comp [B] int32; scores [B, Tq, N_max] fp32."""
    B, Tq, H_I, D_I = q_idx.shape
    N_max = k_idx.shape[1]
    _check(lib.indexer_score(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(q_pos), _ptr(n_comp), B, Tq,
                             H_I, D_I, N_max, m, _qdt(q_idx, q_fp4), _dt(k_idx), _ptr(scores), _stream(stream)))


def csa_compress_indexer_score(Ca, Cb, Za, Zb, Ba, Bb, kv_out, q_idx, w, k_idx, k_scale, q_pos, n_comp, scores, *,
                               m_c: int, m: int, tok_begin: int = 0, blk_begin: int = 0, blk_end: Optional[int] = None,
                               overlap: bool = True, joint: bool = False, q_fp4: bool = False, stream=None) -> None:
    """csa_compress(Ca .. Bb -> kv_out) and indexer_score(q_idx .. -> scores) in one call."""
    Bc, n_rows, d = Ca.shape
    out_cap = kv_out.shape[1]
    if blk_end is None:
        blk_end = (tok_begin + n_rows) // m_c
    flags = (OVERLAP if overlap else 0) | (JOINT_SOFTMAX if joint else 0)
    out_dt = KV_FP8 if kv_out.dtype == torch.uint8 and kv_out.shape[-1] == d + 64 else _dt(kv_out)
    B, Tq, H_I, D_I = q_idx.shape
    N_max = k_idx.shape[1]
    _check(lib.csa_compress_indexer_score(
        _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb), _ptr(kv_out), Bc, n_rows, tok_begin, d, m_c,
        blk_begin, blk_end, out_cap, flags, _dt(Ca), out_dt, _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale),
        _ptr(q_pos), _ptr(n_comp), B, Tq, H_I, D_I, N_max, m, _qdt(q_idx, q_fp4), _dt(k_idx), _ptr(scores),
        _stream(stream)))


def csa_compress_indexer_score_topk(Ca, Cb, Za, Zb, Ba, Bb, kv_out, q_idx, w, k_idx, k_scale, q_pos, n_comp,
                                    topk_idx, topk_score=None, *, m_c: int, m: int, tok_begin: int = 0,
                                    blk_begin: int = 0, blk_end: Optional[int] = None, overlap: bool = True,
                                    joint: bool = False, ws=None, q_fp4: bool = False, stream=None) -> None:
    """csa_compress(Ca .. Bb -> kv_out) and indexer_score_topk(q_idx .. -> topk_idx) in one call, the
    scores living in the workspace (indexer_score_topk_workspace_bytes)."""
    Bc, n_rows, d = Ca.shape
    out_cap = kv_out.shape[1]
    if blk_end is None:
        blk_end = (tok_begin + n_rows) // m_c
    flags = (OVERLAP if overlap else 0) | (JOINT_SOFTMAX if joint else 0)
    out_dt = KV_FP8 if kv_out.dtype == torch.uint8 and kv_out.shape[-1] == d + 64 else _dt(kv_out)
    B, Tq, H_I, D_I = q_idx.shape
    N_max = k_idx.shape[1]
    top_k = topk_idx.shape[-1]
    ws, nb = _ws(indexer_score_topk_workspace_bytes(B, Tq, N_max, top_k), ws, q_idx.device)
    _check(lib.csa_compress_indexer_score_topk(
        _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb), _ptr(kv_out), Bc, n_rows, tok_begin, d, m_c,
        blk_begin, blk_end, out_cap, flags, _dt(Ca), out_dt, _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale),
        _ptr(q_pos), _ptr(n_comp), B, Tq, H_I, D_I, N_max, m, top_k, _qdt(q_idx, q_fp4), _dt(k_idx), _ptr(topk_idx),
        _ptr(topk_score), _ptr(ws), nb, _stream(stream)))


def csa_decode_step_workspace_bytes(B: int, Tq: int, N_max: int, top_k: int, H: int, D: int, W: int) -> int:
    return lib.csa_decode_step_workspace_bytes(B, Tq, N_max, top_k, H, D, W)


def csa_decode_step(Ca, Cb, Za, Zb, Ba, Bb, q_idx, w, k_idx, k_scale, q_pos, n_comp, q, kv_comp, kv_win, win_len,
                    sink, topk_idx, out, lse=None, topk_score=None, *, m_c: int, m: int, tok_begin: int = 0,
                    blk_begin: int = 0, blk_end: Optional[int] = None, overlap: bool = True, joint: bool = False,
                    scale: float = 1.0, ws=None, q_fp4: bool = False, stream=None) -> None:
    """One CSA decode step: compression of blocks [blk_begin, blk_end) into kv_comp, indexer scores,
    top-k (-> topk_idx [B, Tq, top_k]) and sparse MQA (q [B, Tq, H, D] or [B, H, D] -> out)."""
    _, n_rows, d = Ca.shape
    if blk_end is None:
        blk_end = (tok_begin + n_rows) // m_c
    flags = (OVERLAP if overlap else 0) | (JOINT_SOFTMAX if joint else 0)
    B, Tq, H_I, D_I = q_idx.shape
    N_max = k_idx.shape[1]
    top_k = topk_idx.shape[-1]
    H, D = q.shape[-2], q.shape[-1]
    W = kv_win.shape[1] - Tq + 1
    ws, nb = _ws(csa_decode_step_workspace_bytes(B, Tq, N_max, top_k, H, D, W), ws, q.device)
    _check(lib.csa_decode_step(
        _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb), n_rows, tok_begin, d, m_c, blk_begin, blk_end,
        flags, _dt(Ca), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(q_pos), _ptr(n_comp), B, Tq, H_I, D_I,
        N_max, m, top_k, _qdt(q_idx, q_fp4), _dt(k_idx), _ptr(q), _ptr(kv_comp), _ptr(kv_win), _ptr(win_len),
        _ptr(sink),
        scale, H, D, W, _kv_dt(q, kv_comp), _dt(out), _ptr(topk_idx), _ptr(topk_score), _ptr(out), _ptr(lse),
        _ptr(ws), nb, _stream(stream)))


def csa_decode_step_qk_workspace_bytes(B: int, Tq: int, N_max: int, top_k: int, H: int, D: int, W: int) -> int:
    return lib.csa_decode_step_qk_workspace_bytes(B, Tq, N_max, top_k, H, D, W)


def csa_decode_step_qk(Ca, Cb, Za, Zb, Ba, Bb, q_idx, w, k_idx, k_scale, q_pos, n_comp, q, kv_comp, kv_win, win_len,
                       sink, topk_idx, out, lse=None, topk_score=None, *, m_c: int, m: int, q_gamma=None,
                       eps: float = 1e-6, rope_dims: int = 64, rope_theta: float = 10000.0, norm: bool = True,
                       rope: bool = True, tok_begin: int = 0, blk_begin: int = 0, blk_end: Optional[int] = None,
                       overlap: bool = True, joint: bool = False, scale: float = 1.0, ws=None, q_fp4: bool = False,
                       stream=None) -> None:
    """csa_decode_step on raw queries: RMSNorm (q_gamma) + RoPE of the last rope_dims dims at q_pos
    before the attention, the inverse rotation of the output after it."""
    _, n_rows, d = Ca.shape
    if blk_end is None:
        blk_end = (tok_begin + n_rows) // m_c
    flags = (OVERLAP if overlap else 0) | (JOINT_SOFTMAX if joint else 0)
    qk_flags = (RMSNORM if norm else 0) | (ROPE if rope else 0)
    B, Tq, H_I, D_I = q_idx.shape
    N_max = k_idx.shape[1]
    top_k = topk_idx.shape[-1]
    H, D = q.shape[-2], q.shape[-1]
    W = kv_win.shape[1] - Tq + 1
    ws, nb = _ws(csa_decode_step_qk_workspace_bytes(B, Tq, N_max, top_k, H, D, W), ws, q.device)
    _check(lib.csa_decode_step_qk(
        _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb), n_rows, tok_begin, d, m_c, blk_begin, blk_end,
        flags, _dt(Ca), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(q_pos), _ptr(n_comp), B, Tq, H_I, D_I,
        N_max, m, top_k, _qdt(q_idx, q_fp4), _dt(k_idx), _ptr(q), _ptr(kv_comp), _ptr(kv_win), _ptr(win_len),
        _ptr(sink),
        scale, H, D, W, _kv_dt(q, kv_comp), _dt(out), _ptr(topk_idx), _ptr(topk_score), _ptr(out), _ptr(lse),
        _ptr(q_gamma), eps, rope_dims, rope_theta, qk_flags, _ptr(ws), nb, _stream(stream)))


def trace_phases(events) -> None:
    """Record these torch.cuda.Event objects (up to 5, each recorded once
    before, so that it exists) at the phase boundaries of the decode calls on
    this thread; None or [] turns it off. Instrumentation only."""
    if not events:
        _check(lib.csa_trace_phases(None, 0))
        return
    hs = [e.cuda_event for e in events]
    if any(h == 0 for h in hs):
        raise ValueError("record every event once before tracing with it")
    arr = (ctypes.c_void_p * len(hs))(*hs)
    _check(lib.csa_trace_phases(arr, len(hs)))


STEP_SCRATCH_BYTES = 64 << 20  # CSA_STEP_SCRATCH_BYTES: the scratch csa_decode_step_noalloc holds per device


def csa_decode_step_noalloc(Ca, Cb, Za, Zb, Ba, Bb, q_idx, w, k_idx, k_scale, q_pos, n_comp, q, kv_comp, kv_win,
                            win_len, sink, topk_idx, out, lse=None, topk_score=None, *, m_c: int, m: int,
                            tok_begin: int = 0, blk_begin: int = 0, blk_end: Optional[int] = None,
                            overlap: bool = True, joint: bool = False, scale: float = 1.0, q_fp4: bool = False,
                            stream=None) -> None:
    """csa_decode_step with the library's own per-device scratch: allocates nothing."""
    _, n_rows, d = Ca.shape
    if blk_end is None:
        blk_end = (tok_begin + n_rows) // m_c
    flags = (OVERLAP if overlap else 0) | (JOINT_SOFTMAX if joint else 0)
    B, Tq, H_I, D_I = q_idx.shape
    N_max = k_idx.shape[1]
    top_k = topk_idx.shape[-1]
    H, D = q.shape[-2], q.shape[-1]
    W = kv_win.shape[1] - Tq + 1
    _check(lib.csa_decode_step_noalloc(
        _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb), n_rows, tok_begin, d, m_c, blk_begin, blk_end,
        flags, _dt(Ca), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(q_pos), _ptr(n_comp), B, Tq, H_I, D_I,
        N_max, m, top_k, _qdt(q_idx, q_fp4), _dt(k_idx), _ptr(q), _ptr(kv_comp), _ptr(kv_win), _ptr(win_len),
        _ptr(sink),
        scale, H, D, W, _kv_dt(q, kv_comp), _dt(out), _ptr(topk_idx), _ptr(topk_score), _ptr(out), _ptr(lse),
        _stream(stream)))


def indexer_topk_workspace_bytes(B: int, Tq: int, N_max: int, top_k: int) -> int:
    return lib.indexer_topk_workspace_bytes(B, Tq, N_max, top_k)


def indexer_topk(scores, q_pos, n_comp, topk_idx, topk_score=None, *, m: int, ws=None, stream=None) -> None:
    """scores [B, Tq, N_max] fp32 -> topk_idx [B, Tq, top_k] int32 (+ topk_score)."""
    B, Tq, N_max = scores.shape
    top_k = topk_idx.shape[-1]
    ws, nb = _ws(indexer_topk_workspace_bytes(B, Tq, N_max, top_k), ws, scores.device)
    _check(lib.indexer_topk(_ptr(scores), _ptr(q_pos), _ptr(n_comp), B, Tq, N_max, m, top_k, _ptr(topk_idx),
                            _ptr(topk_score), _ptr(ws), nb, _stream(stream)))


def indexer_score_topk_workspace_bytes(B: int, Tq: int, N_max: int, top_k: int) -> int:
    return lib.indexer_score_topk_workspace_bytes(B, Tq, N_max, top_k)


def indexer_score_topk(q_idx, w, k_idx, k_scale, q_pos, n_comp, topk_idx, topk_score=None, *, m: int, ws=None,
                       q_fp4: bool = False, stream=None) -> None:
    B, Tq, H_I, D_I = q_idx.shape
    N_max = k_idx.shape[1]
    top_k = topk_idx.shape[-1]
    ws, nb = _ws(indexer_score_topk_workspace_bytes(B, Tq, N_max, top_k), ws, q_idx.device)
    _check(lib.indexer_score_topk(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(q_pos), _ptr(n_comp), B,
                                  Tq, H_I, D_I, N_max, m, top_k, _qdt(q_idx, q_fp4), _dt(k_idx), _ptr(topk_idx),
                                  _ptr(topk_score), _ptr(ws), nb, _stream(stream)))


# ------------------------------------------------------------------ attention

def sparse_mqa_decode_workspace_bytes(B: int, H: int, D: int, top_k: int, W: int) -> int:
    return lib.sparse_mqa_decode_workspace_bytes(B, H, D, top_k, W)


def sparse_mqa_decode(q, kv_comp, topk_idx, kv_win, win_len, sink, out, lse=None, *, scale: float = 1.0, ws=None,
                      stream=None) -> None:
    """q [B, H, D]; kv_comp [B, N_max, D]; topk_idx [B, top_k]; kv_win [B, W, D]; win_len [B];
    sink [H] fp32 or None; out [B, H, D]; lse [B, H] or None. kv_comp and kv_win
    may be mixed-precision uint8 rows [.., D + 64] (KV_FP8) with bf16 q."""
    B, H, D = q.shape
    N_max = kv_comp.shape[1]
    top_k = topk_idx.shape[-1]
    W = kv_win.shape[1] if kv_win is not None else 0
    ws, nb = _ws(sparse_mqa_decode_workspace_bytes(B, H, D, top_k, W), ws, q.device)
    _check(lib.sparse_mqa_decode(_ptr(q), _ptr(kv_comp), _ptr(topk_idx), _ptr(kv_win), _ptr(win_len), _ptr(sink),
                                 scale, B, H, D, N_max, top_k, W, _kv_dt(q, kv_comp), _dt(out), _ptr(out), _ptr(lse),
                                 _ptr(ws), nb, _stream(stream)))


def sparse_mqa_decode_multi_workspace_bytes(B: int, Tq: int, H: int, D: int, top_k: int, W: int) -> int:
    return lib.sparse_mqa_decode_multi_workspace_bytes(B, Tq, H, D, top_k, W)


def sparse_mqa_decode_multi(q, kv_comp, topk_idx, kv_win, win_len, sink, out, lse=None, *, scale: float = 1.0,
                            ws=None, stream=None) -> None:
    """q [B, Tq, H, D]; kv_comp [B, N_max, D]; topk_idx [B, Tq, top_k]; kv_win [B, W + Tq - 1, D];
    win_len [B]; out [B, Tq, H, D]; lse [B, Tq, H] or None."""
    B, Tq, H, D = q.shape
    N_max = kv_comp.shape[1]
    top_k = topk_idx.shape[-1]
    W = kv_win.shape[1] - (Tq - 1) if kv_win is not None else 0
    ws, nb = _ws(sparse_mqa_decode_multi_workspace_bytes(B, Tq, H, D, top_k, W), ws, q.device)
    _check(lib.sparse_mqa_decode_multi(_ptr(q), _ptr(kv_comp), _ptr(topk_idx), _ptr(kv_win), _ptr(win_len),
                                       _ptr(sink), scale, B, Tq, H, D, N_max, top_k, W, _kv_dt(q, kv_comp), _dt(out),
                                       _ptr(out), _ptr(lse), _ptr(ws), nb, _stream(stream)))


def sparse_mqa_prefill_workspace_bytes(Tq: int, H: int, D: int, top_k: int, W: int) -> int:
    return lib.sparse_mqa_prefill_workspace_bytes(Tq, H, D, top_k, W)


def sparse_mqa_prefill(q, kv_comp, topk_idx, kv_tok, q_pos, sink, out, lse=None, *, W: int, scale: float = 1.0,
                       ws=None, stream=None) -> None:
    """q [Tq, H, D]; kv_comp [N, D]; topk_idx [Tq, top_k]; kv_tok [T_tok, D]; q_pos [Tq]."""
    Tq, H, D = q.shape
    N = kv_comp.shape[0]
    top_k = topk_idx.shape[-1]
    T_tok = kv_tok.shape[0]
    ws, nb = _ws(sparse_mqa_prefill_workspace_bytes(Tq, H, D, top_k, W), ws, q.device)
    _check(lib.sparse_mqa_prefill(_ptr(q), _ptr(kv_comp), _ptr(topk_idx), _ptr(kv_tok), _ptr(q_pos), _ptr(sink),
                                  scale, Tq, H, D, N, T_tok, top_k, W, _kv_dt(q, kv_comp), _dt(out), _ptr(out), _ptr(lse),
                                  _ptr(ws), nb, _stream(stream)))


def hca_decode_step_workspace_bytes(B: int, H: int, D: int, N_max: int, W: int) -> int:
    return lib.hca_decode_step_workspace_bytes(B, H, D, N_max, W)


def hca_decode_step(Ca, Za, Ba, q, kv_comp, n_comp, q_pos, kv_win, win_len, sink, out, lse=None, *, m_c: int,
                    m: int, tok_begin: int = 0, blk_begin: int = 0, blk_end: Optional[int] = None, scale: float = 1.0,
                    ws=None, stream=None) -> None:
    """One HCA decode step: single-branch compression of blocks [blk_begin, blk_end) of Ca/Za
    [B, n_rows, D] into kv_comp, then dense MQA of q [B, H, D] over every visible entry,
    the window and the sink (-> out [B, H, D])."""
    B, n_rows, d = Ca.shape
    if blk_end is None:
        blk_end = (tok_begin + n_rows) // m_c
    H, D = q.shape[-2], q.shape[-1]
    N_max = kv_comp.shape[1]
    W = kv_win.shape[1]
    ws, nb = _ws(hca_decode_step_workspace_bytes(B, H, D, N_max, W), ws, q.device)
    _check(lib.hca_decode_step(_ptr(Ca), _ptr(Za), _ptr(Ba), n_rows, tok_begin, d, m_c, blk_begin, blk_end, _dt(Ca),
                               _ptr(q), _ptr(kv_comp), _ptr(n_comp), _ptr(q_pos), m, _ptr(kv_win), _ptr(win_len),
                               _ptr(sink), scale, B, H, D, N_max, W, _kv_dt(q, kv_comp), _dt(out), _ptr(out),
                               _ptr(lse), _ptr(ws), nb, _stream(stream)))


def hca_prefill_workspace_bytes(Tq: int, H: int, D: int, N: int, W: int) -> int:
    return lib.hca_prefill_workspace_bytes(Tq, H, D, N, W)


def hca_prefill(q, kv_comp, kv_tok, q_pos, sink, out, lse=None, *, m: int, W: int, scale: float = 1.0,
                ws=None, stream=None) -> None:
    """q [Tq, H, D]; kv_comp [N, D] (HCA entries); kv_tok [T_tok, D]; q_pos [Tq]."""
    Tq, H, D = q.shape
    N = kv_comp.shape[0] if kv_comp is not None else 0
    T_tok = kv_tok.shape[0] if kv_tok is not None else 0
    ws, nb = _ws(hca_prefill_workspace_bytes(Tq, H, D, N, W), ws, q.device)
    _check(lib.hca_prefill(_ptr(q), _ptr(kv_comp), _ptr(kv_tok), _ptr(q_pos), _ptr(sink), scale, Tq, H, D, N, m,
                           T_tok, W, _kv_dt(q, kv_comp), _dt(out), _ptr(out), _ptr(lse), _ptr(ws), nb,
                           _stream(stream)))


def qk_norm_rope(x, out, pos=None, gamma=None, *, norm: bool = False, rope: bool = False, inverse: bool = False,
                 rope_dims: int = 64, eps: float = 1e-6, theta: float = 10000.0, stream=None) -> None:
    """x, out [T, H, D] (out may be x); pos [T] int32; gamma [D] fp32 or None."""
    T, H, D = x.shape
    flags = (RMSNORM if norm else 0) | (ROPE if rope else 0) | (ROPE_INVERSE if inverse else 0)
    _check(lib.qk_norm_rope(_ptr(x), _ptr(out), _ptr(gamma), _ptr(pos), T, H, D, rope_dims, eps, theta, flags,
                            _dt(x), _stream(stream)))


def hca_dense_mqa_workspace_bytes(B: int, H: int, D: int, N_max: int, W: int) -> int:
    return lib.hca_dense_mqa_workspace_bytes(B, H, D, N_max, W)


def hca_dense_mqa(q, kv_comp, n_comp, q_pos, kv_win, win_len, sink, out, lse=None, *, m: int, scale: float = 1.0,
                  ws=None, stream=None) -> None:
    """q [B, H, D]; kv_comp [B, N_max, D]; n_comp, q_pos [B]; kv_win [B, W, D]; win_len [B]."""
    B, H, D = q.shape
    N_max = kv_comp.shape[1]
    W = kv_win.shape[1] if kv_win is not None else 0
    ws, nb = _ws(hca_dense_mqa_workspace_bytes(B, H, D, N_max, W), ws, q.device)
    _check(lib.hca_dense_mqa(_ptr(q), _ptr(kv_comp), _ptr(n_comp), _ptr(q_pos), m, _ptr(kv_win), _ptr(win_len),
                             _ptr(sink), scale, B, H, D, N_max, W, _kv_dt(q, kv_comp), _dt(out), _ptr(out),
                             _ptr(lse), _ptr(ws), nb, _stream(stream)))
