"""A CSA decode step captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must give the eager result bit for bit, with eager
work of another shape and synchronisations between the replays, and the
outputs overwritten before each replay so a stale result cannot pass."""
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


class _Step:
    """Device tensors of one decode step and a call that runs it."""

    def __init__(self, cfg, form):
        L = _L()
        self.cfg, self.form = cfg, form
        x = gen.gen_decode(cfg)
        B, N, m, k, W = cfg.B, cfg.N, cfg.m, cfg.top_k, cfg.W
        self.pos = _t(np.full((B, 1), cfg.n - 1, np.int32))
        self.nc = _t(np.full((B,), N, np.int32))
        self.k_t = _bf(x["k_idx"])
        self.qi, self.wt, self.q = _bf(x["q_idx"][:, None]), _t(x["w"][:, None]), _bf(x["q"][:, None])
        self.win, self.wl = _bf(x["kv_win"]), _t(np.full((B,), W, np.int32))
        self.comp = [_bf(x[nm]) for nm in ("Ca", "Cb", "Za", "Zb")]
        self.Ba, self.Bb, self.sink = _t(x["Ba"]), _t(x["Bb"]), _t(x["sink"])
        self.kv = _bf(x["kv_comp"])
        self.idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
        self.tsc = torch.empty((B, 1, k), device=DEV)
        self.out = torch.empty((B, 1, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
        self.lse = torch.empty((B, 1, cfg.H), device=DEV)
        nb = L.csa_decode_step_workspace_bytes(B, 1, N, k, cfg.H, cfg.D, W)
        self.ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
        self.kw = dict(m_c=m, m=m, tok_begin=cfg.n - 2 * m, blk_begin=N - 1, blk_end=N)

    def __call__(self):
        L = _L()
        args = (*self.comp, self.Ba, self.Bb, self.qi, self.wt, self.k_t, None, self.pos, self.nc, self.q, self.kv,
                self.win, self.wl, self.sink, self.idx, self.out, self.lse, self.tsc)
        if self.form == "noalloc":
            L.csa_decode_step_noalloc(*args, **self.kw)
        else:
            L.csa_decode_step(*args, **self.kw, ws=self.ws)

    def spoil(self):
        self.idx.fill_(-7)
        self.tsc.fill_(7.0)
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))

    def result(self):
        N = self.cfg.N
        return host(self.kv[:, N - 1]), host(self.idx), host(self.tsc), host(self.out), host(self.lse)


@pytest.mark.gpu
@pytest.mark.parametrize("form", ["workspace", "noalloc"])
def test_decode_step_graph_replays(form):
    print(f"[case] graph capture of a decode step, {form}", flush=True)
    step = _Step(gen.scaled(gen.C2, B=6, n=32768), form)
    other = _Step(gen.scaled(gen.C2, B=3, n=16384), form)  # eager work of another shape between replays
    step()
    torch.cuda.synchronize()
    ref = step.result()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        step.spoil()
        if rep % 2:
            other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = step.result()
        for i, nm in enumerate(("kv row N-1", "idx", "topk scores", "out", "lse")):
            assert np.array_equal(got[i], ref[i], equal_nan=True), f"replay {rep}: {nm} differs from the eager call"


class _HcaStep:
    """Device tensors of one HCA decode step (append + dense MQA, one call)."""

    def __init__(self, cfg):
        L = _L()
        self.cfg = cfg
        x = gen.gen_decode(cfg, with_compress=True)
        B, N, m, W = cfg.B, cfg.N, cfg.m, cfg.W
        self.args = (_bf(x["Ca"]), _bf(x["Za"]), _t(x["Ba"]), _bf(x["q"]))
        self.kv = _bf(x["kv_comp"])
        self.rest = (_t(np.full((B,), N, np.int32)), _t(np.full((B,), cfg.n - 1, np.int32)), _bf(x["kv_win"]),
                     _t(np.full((B,), W, np.int32)), _t(x["sink"]))
        self.out = torch.empty((B, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
        self.lse = torch.empty((B, cfg.H), device=DEV)
        self.ws = torch.zeros(L.hca_decode_step_workspace_bytes(B, cfg.H, cfg.D, N, W), dtype=torch.uint8,
                              device=DEV)
        self.kw = dict(m_c=m, m=m, tok_begin=cfg.n - m, blk_begin=N - 1, blk_end=N)

    def __call__(self):
        _L().hca_decode_step(*self.args, self.kv, *self.rest, self.out, self.lse, **self.kw, ws=self.ws)

    def spoil(self):
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))
        self.kv[:, self.cfg.N - 1].fill_(7.0)

    def result(self):
        return host(self.kv[:, self.cfg.N - 1]), host(self.out), host(self.lse)


@pytest.mark.gpu
def test_hca_decode_step_graph_replays():
    """Replays reuse one launch, so its merge counter must come back to zero
    after every call; the appended entry is recomputed by each replay."""
    print("[case] graph capture of an HCA decode step", flush=True)
    step = _HcaStep(gen.scaled(gen.C4, B=4, n=1 << 17))
    other = _HcaStep(gen.scaled(gen.C4, B=2, n=1 << 16))
    step()
    torch.cuda.synchronize()
    ref = step.result()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        step.spoil()
        if rep % 2:
            other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = step.result()
        for i, nm in enumerate(("entry N-1", "out", "lse")):
            assert np.array_equal(got[i], ref[i], equal_nan=True), f"replay {rep}: {nm} differs from the eager call"
