"""Planted mistakes in copies of the oracle (on the CPU) must each fail at
least one pin: evidence that the pins can see a dropped term, a wrong sign,
index or axis."""
import types

import numpy as np
import pytest

import oracle
from oracle import ref
from tests import oracle_pins


def _ns(**over):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in oracle.__dict__ if not k.startswith("_")})
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _compress_variant(kind):
    def f(Ca, Cb, Za, Zb, Ba, Bb, m, overlap=True, joint=False, blocks=None):
        Ca = np.asarray(Ca, float); Za = np.asarray(Za, float); Ba = np.asarray(Ba, float)
        n, d = Ca.shape
        N = n // m
        out = np.zeros((N, d))
        for i in range(N):
            a = slice(m * i, m * i + m)
            za = Za[a] + (Ba[[i % m] * m] if kind == "bias_by_block" else Ba)
            ax = 1 if kind == "softmax_over_channels" else 0
            wa = np.exp(za - za.max(axis=ax, keepdims=True)); wa /= wa.sum(axis=ax, keepdims=True)
            out[i] = (wa * Ca[a]).sum(axis=0)
            if overlap and kind != "no_b_branch":
                j = i + 1 if kind == "b_reads_next_block" else i - 1
                if 0 <= j < N and (i >= 1 or kind == "b_reads_next_block"):
                    b = slice(m * j, m * j + m)
                    zb = np.asarray(Zb, float)[b] + np.asarray(Bb, float)
                    wb = np.exp(zb - zb.max(axis=0)); wb /= wb.sum(axis=0)
                    out[i] += (wb * np.asarray(Cb, float)[b]).sum(axis=0)
        return out
    return f


def _scores_relu_after_weight(q_idx, w, k_idx, V, k_scale=None):
    dots = np.asarray(k_idx, float)[:V] @ np.asarray(q_idx, float).T
    if k_scale is not None:
        dots = dots * np.asarray(k_scale, float)[:V, None]
    return np.maximum(dots * np.asarray(w, float)[None, :], 0).sum(axis=1)


def _scores_scale_ignored(q_idx, w, k_idx, V, k_scale=None):
    return ref.indexer_scores(q_idx, w, k_idx, V, None)


def _topk_ties_high(scores, k):
    s = np.asarray(scores, float)
    V = len(s)
    order = np.lexsort((-np.arange(V), -s))
    out = np.full(k, -1)
    out[:min(k, V)] = np.sort(order[:min(k, V)])
    return out


def _attend_no_sink(q, rows, sink, tau=1.0):
    return ref.attend(q, rows, np.full(np.shape(sink), -np.inf), tau)


def _attend_sink_sign(q, rows, sink, tau=1.0):
    return ref.attend(q, rows, -np.asarray(sink, float), tau)


def _attend_tau_squared(q, rows, sink, tau=1.0):
    return ref.attend(q, rows, sink, tau * tau)


def _window_excl_current(kv_tok, p, W):
    return np.asarray(kv_tok, float)[max(0, p - W):p]


def _visible_floor_p(p, n_comp, m):
    return max(0, min(int(n_comp), int(p) // m))


def _quantize_variant(kind):
    def f(x):
        x = np.asarray(x, float)
        D = x.shape[-1]
        xb = x.reshape(x.shape[:-1] + (D // 32, 32))
        amax = np.abs(xb).max(axis=-1)
        _, ex = np.frexp(amax)
        off = 1 if kind == "emax_1" else 2
        E = np.where(amax > 0, np.clip(ex - 1 - off + 127, 1, 254), 127).astype(np.int64)
        y = xb * np.exp2(127.0 - E)[..., None]
        a = np.abs(y)
        step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
        r = np.floor(a / step + 0.5) if kind == "ties_away" else np.rint(a / step)
        mag = np.minimum(r * step, 6.0)
        code = np.where(mag < 2.0, 2.0 * mag, np.where(mag < 4.0, mag + 2.0, 0.5 * mag + 4.0)).astype(np.int64)
        code = code | (((y < 0) & (code > 0)).astype(np.int64) << 3)
        code = code.reshape(x.shape)
        lo, hi = (code[..., 1::2], code[..., 0::2]) if kind == "nibbles_swapped" else (code[..., 0::2], code[..., 1::2])
        return (lo | (hi << 4)).astype(np.uint8), E.astype(np.uint8)
    return f


def _scores_fp4_query_ignored(q_idx, w, k_idx, V, k_scale=None, q_fp4=False):
    return ref.indexer_scores(q_idx, w, k_idx, V, k_scale)


MUTANTS = {
    "compress_b_reads_next_block": dict(compress=_compress_variant("b_reads_next_block")),
    "compress_softmax_over_channels": dict(compress=_compress_variant("softmax_over_channels")),
    "compress_bias_indexed_by_block": dict(compress=_compress_variant("bias_by_block")),
    "compress_drops_b_branch": dict(compress=_compress_variant("no_b_branch")),
    "indexer_relu_after_weight": dict(indexer_scores=_scores_relu_after_weight),
    "indexer_ignores_fp8_scale": dict(indexer_scores=_scores_scale_ignored),
    "topk_ties_to_higher_index": dict(topk_select=_topk_ties_high),
    "attend_drops_sink": dict(attend=_attend_no_sink),
    "attend_sink_sign_flipped": dict(attend=_attend_sink_sign),
    "attend_wrong_logit_scale": dict(attend=_attend_tau_squared),
    "window_excludes_current_token": dict(window_rows=_window_excl_current),
    "visibility_off_by_one": dict(visible=_visible_floor_p),
    "mxfp4_quantize_ties_away": dict(mxfp4_quantize=_quantize_variant("ties_away")),
    "mxfp4_quantize_emax_1": dict(mxfp4_quantize=_quantize_variant("emax_1")),
    "mxfp4_quantize_nibbles_swapped": dict(mxfp4_quantize=_quantize_variant("nibbles_swapped")),
    "indexer_ignores_fp4_query": dict(indexer_scores=_scores_fp4_query_ignored),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    ns = _ns(**MUTANTS[name])
    failed = []
    for chk in oracle_pins.ALL_CHECKS:
        try:
            chk(ns)
        except Exception:
            failed.append(chk.__name__)
    assert failed, f"no pin catches mutant {name}"
