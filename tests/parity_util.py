"""Helpers of the GPU parity tests: device upload of generator output and the
comparison rules.

Comparison contract:
  * top-k index sets: exact, except for entries whose oracle score lies in
    the tie band of the K-th score s_K:  |s_i - s_K| <= max(1e-3 |s_K|,
    1e-6 max|s|). Outside the band the GPU and oracle sets must be equal, and
    both must hold K' = min(k, V) entries, in ascending order, -1 padded.
  * attention outputs: max-abs <= 2e-2 against the float64 oracle, plus a
    tighter bound derived from the arithmetic, scaled with the output
    (out_bound), both asserted. Every check is recorded with its max-abs and
    the oracle's RMS and largest magnitude; the session prints the worst
    ratios at its end (tests/conftest.py).
"""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"
OUT_TOL = 2e-2
# (what, max-abs error, rms of the oracle output, max |oracle output|) of every output check
REPORT = []


def out_bound(ref, exact: bool = False) -> float:
    """The bound the arithmetic allows, proportional to the output's size.

    bf16 paths round each softmax weight P to bf16 for the PV product and the
    output to bf16 once more: each rounding errs by at most 2^-9 relative, and
    the P roundings enter as a weighted sum of independent errors, so the
    error stays a small multiple of 2^-9 max|o|; 2^-7 max|o| leaves a factor 4.
    fp32 rows and outputs (exact=True) keep every value in fp32: 1e-5 max|o|.
    There is no absolute floor: an all-zero output must come out exactly zero.
    """
    mx = float(np.abs(np.asarray(ref, np.float64)).max(initial=0.0))
    return (1e-5 if exact else 2.0 ** -7) * mx


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def bf(x: np.ndarray) -> torch.Tensor:
    """float32 values that are bf16-representable -> bf16 device tensor (exact)."""
    return dev(np.asarray(x, np.float32), torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy() if t.is_floating_point() else t.cpu().numpy()


def tie_band(scores: np.ndarray, k: int):
    """Oracle K-th score and the band of indices tied with it."""
    s = np.asarray(scores, np.float64)
    V = s.shape[0]
    K = min(k, V)
    if K == 0 or K == V:
        return None, np.zeros(V, bool)
    sk = np.sort(s)[::-1][K - 1]
    tol = max(1e-3 * abs(sk), 1e-6 * np.abs(s).max())
    return sk, np.abs(s - sk) <= tol


def check_topk_row(gpu_idx: np.ndarray, oracle_idx: np.ndarray, oracle_scores: np.ndarray, k: int, what=""):
    g = np.asarray(gpu_idx)
    o = np.asarray(oracle_idx)
    V = oracle_scores.shape[0]
    K = min(k, V)
    assert g.shape == (k,)
    assert np.all(g[K:] == -1), f"{what}: padding"
    gk = g[:K]
    assert np.all(gk >= 0) and np.all(gk < V), f"{what}: out-of-range index"
    assert np.all(np.diff(gk) > 0), f"{what}: not ascending / duplicate"
    _, band = tie_band(oracle_scores, k)
    gs, os_ = set(gk.tolist()), set(o[:K].tolist())
    bset = set(np.nonzero(band)[0].tolist())
    assert gs - bset == os_ - bset, f"{what}: sets differ outside the tie band " \
        f"(gpu-only {sorted((gs - os_) - bset)[:8]}, oracle-only {sorted((os_ - gs) - bset)[:8]})"


def check_out(gpu: np.ndarray, ref: np.ndarray, tight: float, what=""):
    ref = np.asarray(ref, np.float64)
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    mx = float(err.max()) if err.size else 0.0
    rms = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    big = float(np.abs(ref).max(initial=0.0))
    REPORT.append((what, mx, rms, big))
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert mx <= OUT_TOL, f"{what}: max-abs {mx:.3e} > {OUT_TOL}"
    assert mx <= tight, (f"{what}: max-abs {mx:.3e} > derived bound {tight:.2e} "
                         f"(max-abs/rms {mx / rms if rms else 0:.3e}, max|ref| {big:.3e})")
    return mx, rms
