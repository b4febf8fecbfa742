"""csa_decode_step_noalloc, the decode step that allocates nothing (its
scratch is the library's own per-device array), against csa_decode_step with
a caller workspace: the same bits on two calls in a row, the second with a
smaller input, and the size limit refused before any GPU work."""
import numpy as np
import pytest
import torch

from synth import gen
from tests.parity_util import DEV, host


def _L():
    import long_context_attention_06_amd as L
    return L


def _bf(v):
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(DEV)


def _t(v):
    return torch.from_numpy(np.ascontiguousarray(v)).to(DEV)


def _run(cfg, x, noalloc: bool):
    L = _L()
    B, N, m, k, W, Tq = cfg.B, cfg.N, cfg.m, cfg.top_k, cfg.W, cfg.Tq
    pos = _t(np.tile(np.arange(cfg.n - Tq, cfg.n, dtype=np.int32), (B, 1)))
    nc = _t(np.full((B,), N, np.int32))
    if cfg.k_dtype == "fp8":
        k_t, sc = _t(x["k_idx_codes"]), _t(x["k_scale"])
    else:
        k_t, sc = _bf(x["k_idx"]), None
    qi = _bf(x["q_idx"] if Tq > 1 else x["q_idx"][:, None])
    wt = _t(x["w"] if Tq > 1 else x["w"][:, None])
    q = _bf(x["q"] if Tq > 1 else x["q"][:, None])
    win, wl = _bf(x["kv_win"]), _t(np.full((B,), W + Tq - 1, np.int32))
    comp = [_bf(x[nm]) for nm in ("Ca", "Cb", "Za", "Zb")]
    kv = _bf(x["kv_comp"])
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=DEV)
    tsc = torch.full((B, Tq, k), 7.0, device=DEV)
    out = torch.empty((B, Tq, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Tq, cfg.H), device=DEV)
    args = (*comp, _t(x["Ba"]), _t(x["Bb"]), qi, wt, k_t, sc, pos, nc, q, kv, win, wl, _t(x["sink"]), idx, out, lse,
            tsc)
    kw = dict(m_c=m, m=m, tok_begin=cfg.n - 2 * m, blk_begin=N - 1, blk_end=N)
    if noalloc:
        L.csa_decode_step_noalloc(*args, **kw)
    else:
        L.csa_decode_step(*args, **kw)
    torch.cuda.synchronize()
    return host(kv[:, N - 1]), host(idx), host(tsc), host(out), host(lse)


@pytest.mark.gpu
def test_decode_step_noalloc_matches_workspace_form():
    # two calls in a row on one device, the second smaller (fewer sequences,
    # shorter contexts); then the first shape again, after the smaller one
    cases = [("C2 B=8 32K", gen.scaled(gen.C2, B=8, n=32768)),
             ("C2 B=3 16K", gen.scaled(gen.C2, B=3, n=16384)),
             ("C5 B=2 160K fp8 keys", gen.scaled(gen.C5, B=2, n=4 * 40000)),
             ("C2 B=8 32K again", gen.scaled(gen.C2, B=8, n=32768))]
    for name, cfg in cases:
        print(f"[case] no-alloc step {name}", flush=True)
        x = gen.gen_decode(cfg)
        a = _run(cfg, x, noalloc=True)
        b = _run(cfg, x, noalloc=False)
        for i, nm in enumerate(("kv row N-1", "idx", "topk scores", "out", "lse")):
            assert np.array_equal(a[i], b[i], equal_nan=True), f"{name}: {nm} differs from csa_decode_step"
        assert np.all(np.isfinite(a[3])), name


def test_decode_step_noalloc_size_limit():
    """A shape whose scratch exceeds the array is refused on the host, before
    any HIP call (so this runs without a GPU)."""
    L = _L()
    B, Tq, N, k, H, D, W = 64, 2, 65536, 1024, 64, 512, 128
    need = L.csa_decode_step_workspace_bytes(B, Tq, N, k, H, D, W)
    assert need > L.STEP_SCRATCH_BYTES
    rc = L.lib.csa_decode_step_noalloc(*([None] * 6), 8, 0, D, 4, N - 1, N, 1, L.BF16, *([None] * 6), B, Tq, 64,
                                       128, N, 4, k, L.BF16, L.BF16, *([None] * 5), 1.0, H, D, W, L.BF16, L.BF16,
                                       *([None] * 5))
    assert rc == L.WORKSPACE_TOO_SMALL
    assert b"above" in L.lib.csa_last_error()
