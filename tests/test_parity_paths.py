"""GPU parity of whole paths, in the launch configuration bench.py times:
CSA decode step (compress the completed block, score, select, attend) with
bf16, E4M3 or MXFP4 indexer keys, HCA decode step (append the completed
entry, attend), CSA prefill and HCA prefill by 4096-query chunks. Reduced sizes check every
query; the full workload sizes check sampled sequences / queries against the
oracle computed one by one."""
import numpy as np
import pytest
import torch

import oracle
from synth import gen
from tests.parity_util import DEV, check_out, check_topk_row, host, out_bound

pytestmark = pytest.mark.gpu


def _L():
    import long_context_attention_06_amd as L
    return L


def _bf(v):
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(DEV)


def _t(v):
    return torch.from_numpy(np.ascontiguousarray(v)).to(DEV)


def _tight(ref):
    return out_bound(ref)


def _kv(cfg, rows):
    """A main-KV tensor to the device: bf16 values, or mixed-precision bytes."""
    return _t(rows) if cfg.kv_dtype == "fp8" else _bf(rows)


def _kv_values(cfg, rows):
    return oracle.kv_fp8_decode(rows, cfg.D) if cfg.kv_dtype == "fp8" else np.asarray(rows, np.float64)


def _check_entry(cfg, got_row, ent, what):
    """The appended entry: bf16 within its rounding; mixed-precision rows
    within half an E4M3 step (bf16 for the RoPE dims)."""
    if cfg.kv_dtype == "fp8":
        v = oracle.kv_fp8_decode(got_row, cfg.D)
        step = np.where(np.arange(cfg.D) < cfg.D - 64, 2.0 ** -4, 2.0 ** -8)
        assert np.all(np.abs(v - ent) <= np.maximum(np.abs(ent) * step, 2.0 ** -10) + 1e-5), what
    else:
        check_out(got_row, ent, 2.0 ** -8 * max(1.0, np.abs(ent).max()), what)


def run_csa_decode(cfg, x):
    """One decode token per sequence, as bench.py runs it."""
    L = _L()
    B, N, m, k, W = cfg.B, cfg.N, cfg.m, cfg.top_k, cfg.W
    kv = _kv(cfg, x["kv_comp"])
    q_pos = _t(np.full((B, 1), cfg.n - 1, np.int32))
    n_comp = _t(np.full((B,), N, np.int32))
    if cfg.k_dtype == "fp8":
        k_t, sc = _t(x["k_idx_codes"]), _t(x["k_scale"])
    elif cfg.k_dtype == "mxfp4":
        k_t, sc = _t(x["k_idx_codes"]).view(torch.float4_e2m1fn_x2), _t(x["k_scale"])
    else:
        k_t, sc = _bf(x["k_idx"]), None
    # the completed block's entry, the scan and the top-k in one call, as
    # bench.py runs them; twice on one workspace (the second call reads the
    # digit histogram the first one left cleared), the scores in its first bytes
    ws = torch.zeros(L.indexer_score_topk_workspace_bytes(B, 1, N, k), dtype=torch.uint8, device=DEV)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    idx1 = torch.empty_like(idx)
    for dst in (idx1, idx):
        L.csa_compress_indexer_score_topk(_bf(x["Ca"]), _bf(x["Cb"]), _bf(x["Za"]), _bf(x["Zb"]), _t(x["Ba"]),
                                          _t(x["Bb"]), kv, _bf(x["q_idx"][:, None]), _t(x["w"][:, None]), k_t, sc,
                                          q_pos, n_comp, dst, m_c=m, m=m, tok_begin=cfg.n - 2 * m, blk_begin=N - 1,
                                          blk_end=N, ws=ws, q_fp4=cfg.q_fp4)
    scores = ws[:B * N * 4].view(torch.float32).view(B, 1, N)
    out = torch.empty((B, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, cfg.H), device=DEV)
    q, scale = _bf(x["q"]), 1.0
    if cfg.qk_rope:  # prologue on the raw queries, at position n-1
        pos = _t(np.full((B,), cfg.n - 1, np.int32))
        qn = torch.empty_like(q)
        L.qk_norm_rope(q, qn, pos, _t(x["q_gamma"]), norm=True, rope=True)
        q, scale = qn, 1.0 / np.sqrt(cfg.D)
    L.sparse_mqa_decode(q, kv, idx.view(B, k), _kv(cfg, x["kv_win"]), _t(np.full((B,), W, np.int32)),
                        _t(x["sink"]), out, lse, scale=scale)
    if cfg.qk_rope:  # epilogue: the output rotated back
        L.qk_norm_rope(out, out, pos, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx1), "the step's selection differs between two calls on one workspace"
    # the cache stays on the device (GBs at full size); only its last two rows come back
    return host(kv[:, N - 2:]), host(scores)[:, 0], host(idx)[:, 0], host(out), host(lse)


def check_csa_decode(cfg, x, seqs):
    kv2, S, I, O, LSE = run_csa_decode(cfg, x)
    m, N = cfg.m, cfg.N
    for b in seqs:
        print(f"[case] {cfg.name} b={b}", flush=True)
        # the 2m raw rows are tokens n-2m .. n-1, i.e. blocks N-2 and N-1: entry N-1 is
        # their second block, with the first as its overlapping predecessor
        ent = oracle.compress(x["Ca"][b], x["Cb"][b], x["Za"][b], x["Zb"][b], x["Ba"], x["Bb"], m,
                              blocks=range(1, 2))[0]
        _check_entry(cfg, kv2[b, 1], ent, "compressed entry N-1")
        assert np.array_equal(kv2[b, 0], x["kv_comp"][b, N - 2]), "compress wrote outside its block"
        comp = _kv_values(cfg, x["kv_comp"][b])
        comp[N - 1] = _kv_values(cfg, kv2[b, 1])  # the stored entry is what the step attends
        if cfg.k_dtype == "fp8":
            keys, sc = oracle.e4m3_decode(x["k_idx_codes"][b]), x["k_scale"][b]
        elif cfg.k_dtype == "mxfp4":
            keys, sc = oracle.mxfp4_decode(x["k_idx_codes"][b], x["k_scale"][b]), None
        else:
            keys, sc = x["k_idx"][b], None
        q, tau = x["q"][b], 1.0
        if cfg.qk_rope:
            # the prologue's result, stored in bf16 as the attention reads it
            q = gen.bf16_round(oracle.rope_rotate(oracle.rms_norm(q[None], x["q_gamma"], 1e-6), [cfg.n - 1])[0]
                               .astype(np.float32)).astype(np.float64)
            tau = 1.0 / np.sqrt(cfg.D)
        oidx, o_ref, lse_ref, s = oracle.csa_query(q, x["q_idx"][b], x["w"][b], comp, keys, cfg.n - 1, N,
                                                   m, cfg.top_k, _kv_values(cfg, x["kv_win"][b]), x["sink"],
                                                   k_scale=sc, tau=tau, q_fp4=cfg.q_fp4)
        if cfg.qk_rope:
            o_ref = oracle.rope_rotate(o_ref[None], [cfg.n - 1], inverse=True)[0]
        assert np.abs(S[b] - s).max() <= 2e-5 * 8 * (1 + np.abs(s).max())
        check_topk_row(I[b], oidx, s, cfg.top_k, f"b={b}")
        rows = np.concatenate([comp[I[b][I[b] >= 0]], _kv_values(cfg, x["kv_win"][b])])
        o_own, lse_own = oracle.attend(q, rows, x["sink"], tau)
        if cfg.qk_rope:
            o_own = oracle.rope_rotate(o_own[None], [cfg.n - 1], inverse=True)[0]
        check_out(O[b], o_own, _tight(o_own), f"out on gpu idx b={b}")
        assert np.abs(LSE[b] - lse_own).max() < 1e-3
        if np.array_equal(I[b], oidx):
            check_out(O[b], o_ref, _tight(o_ref), f"out end to end b={b}")


def test_csa_decode_flash_reduced():
    cfg = gen.scaled(gen.C2, B=4, n=16384)
    check_csa_decode(cfg, gen.gen_decode(cfg), range(cfg.B))


def test_csa_decode_pro_fp8_reduced():
    cfg = gen.scaled(gen.C5, B=2, n=65536 * 4)
    check_csa_decode(cfg, gen.gen_decode(cfg), range(cfg.B))


def test_csa_decode_flash_full_size_sampled():
    cfg = gen.C2  # 32 sequences x 128K tokens, as bench.py
    check_csa_decode(cfg, gen.gen_decode(cfg), [0, 1, 7, 8, 13, 20, 30, 31])


def test_csa_decode_pro_1m_fp8_full_size_sampled():
    cfg = gen.C5  # 4 sequences x 1M tokens, fp8 indexer keys
    check_csa_decode(cfg, gen.gen_decode(cfg), range(cfg.B))


def run_hca_decode(cfg, x, step=False, ws=None, nc=None):
    """One HCA decode token per sequence, as bench.py runs it: the token
    completes block N-1 (m' divides n), whose entry is appended by
    single-branch compression, then dense MQA over all entries + window.
    step=True runs both through hca_decode_step (one launch)."""
    L = _L()
    B, N, m, W = cfg.B, cfg.N, cfg.m, cfg.W
    kv = _kv(cfg, x["kv_comp"])
    out = torch.empty((B, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, cfg.H), device=DEV)
    n_comp = _t(np.full((B,), N, np.int32) if nc is None else np.asarray(nc, np.int32))
    q_pos = _t(np.full((B,), cfg.n - 1, np.int32))
    if step:
        L.hca_decode_step(_bf(x["Ca"]), _bf(x["Za"]), _t(x["Ba"]), _bf(x["q"]), kv, n_comp, q_pos,
                          _kv(cfg, x["kv_win"]), _t(np.full((B,), W, np.int32)), _t(x["sink"]), out, lse, m_c=m, m=m,
                          tok_begin=cfg.n - m, blk_begin=N - 1, blk_end=N, ws=ws)
    else:
        L.csa_compress(_bf(x["Ca"]), None, _bf(x["Za"]), None, _t(x["Ba"]), None, kv, m=m, tok_begin=cfg.n - m,
                       blk_begin=N - 1, blk_end=N, overlap=False)
        L.hca_dense_mqa(_bf(x["q"]), kv, n_comp, q_pos, _kv(cfg, x["kv_win"]), _t(np.full((B,), W, np.int32)),
                        _t(x["sink"]), out, lse, m=m)
    torch.cuda.synchronize()
    return host(kv[:, N - 2:]), host(out), host(lse)


def check_hca_decode(cfg, seqs, step=False):
    x = gen.gen_decode(cfg, with_compress=True)
    kv2, O, LS = run_hca_decode(cfg, x, step=step)
    N, m = cfg.N, cfg.m
    for b in seqs:
        print(f"[case] {cfg.name} b={b} step={step}", flush=True)
        ent = oracle.compress(x["Ca"][b], None, x["Za"][b], None, x["Ba"], None, m, overlap=False)[0]
        _check_entry(cfg, kv2[b, 1], ent, "hca entry N-1")
        assert np.array_equal(kv2[b, 0], x["kv_comp"][b, N - 2]), "compress wrote outside its block"
        comp = _kv_values(cfg, x["kv_comp"][b])
        comp[N - 1] = _kv_values(cfg, kv2[b, 1])  # the stored entry is what the step attends
        ref, rlse = oracle.hca_query(x["q"][b], comp, cfg.n - 1, N, m, _kv_values(cfg, x["kv_win"][b]), x["sink"])
        check_out(O[b], ref, _tight(ref), f"hca b={b}")
        assert np.abs(LS[b] - rlse).max() < 1e-3


def test_hca_decode_reduced():
    check_hca_decode(gen.scaled(gen.C4, B=3, n=1 << 16), range(3))


def test_hca_decode_1m_full_size():
    cfg = gen.C4  # 16 sequences x 8192 entries, every sequence checked
    check_hca_decode(cfg, range(cfg.B))


def test_hca_decode_1m_kv_fp8_full_size():
    cfg = gen.C4F  # mixed-precision main KV, as bench.py runs it
    check_hca_decode(cfg, range(cfg.B))


def test_hca_decode_step_reduced():
    check_hca_decode(gen.scaled(gen.C4, B=3, n=1 << 16), range(3), step=True)


def test_hca_decode_step_1m_full_size():
    cfg = gen.C4  # one launch: append, split attention and merge; every sequence checked
    check_hca_decode(cfg, range(cfg.B), step=True)


def test_hca_decode_step_1m_kv_fp8_full_size():
    cfg = gen.C4F
    check_hca_decode(cfg, range(cfg.B), step=True)


def test_hca_decode_step_matches_separate_calls():
    """The one-launch step against csa_compress + hca_dense_mqa: the appended
    entry differs at most by the rounding of its fp32 sum (one step of the
    stored format), and so the outputs by far less than the derived bound;
    sequences see all, some or none of the appended block; a garbage
    workspace and its reuse give the same bits as a zeroed one."""
    cfg = gen.scaled(gen.C4, B=6, n=1 << 17)
    x = gen.gen_decode(cfg, with_compress=True)
    N = cfg.N
    nc = [N, N - 1, N, 3, 0, N // 2]
    kv_s, O_s, L_s = run_hca_decode(cfg, x, step=False, nc=nc)
    nb = _L().hca_decode_step_workspace_bytes(cfg.B, cfg.H, cfg.D, N, cfg.W)
    ref = None
    for what, ws in (("zeroed", torch.zeros(nb, dtype=torch.uint8, device=DEV)),
                     ("garbage", torch.randint(0, 256, (nb,), dtype=torch.uint8, device=DEV))):
        for rep in range(2):
            print(f"[case] hca step vs separate, {what} workspace, call {rep}", flush=True)
            kv_f, O_f, L_f = run_hca_decode(cfg, x, step=True, ws=ws, nc=nc)
            if ref is None:
                ref = (kv_f, O_f, L_f)
            for a_, b_, nm in zip((kv_f, O_f, L_f), ref, ("entry", "out", "lse")):
                assert np.array_equal(a_, b_, equal_nan=True), f"{what} call {rep}: {nm} differs"
    assert np.array_equal(kv_f[:, 0], kv_s[:, 0]), "entry N-2 changed"
    ent_f, ent_s = kv_f[:, 1].astype(np.float64), kv_s[:, 1].astype(np.float64)
    # one bf16 step at most: 2^-7 of the value
    assert np.all(np.abs(ent_f - ent_s) <= 2.0 ** -7 * np.abs(ent_s)), "entry N-1"
    for b in range(cfg.B):
        check_out(O_f[b], O_s[b], out_bound(O_s[b]) / 4, f"hca step vs separate b={b}")
        assert np.abs(L_f[b] - L_s[b]).max() < 1e-4


def test_csa_decode_flash_kv_fp8_full_size_sampled():
    cfg = gen.C2F  # mixed-precision main KV, as bench.py runs it
    check_csa_decode(cfg, gen.gen_decode(cfg), [0, 13, 31])


def run_prefill_chunk(cfg, tok, comp_t, chunk):
    L = _L()
    qs = gen.gen_prefill_queries(cfg, chunk)
    T = len(qs["q_pos"])
    N, m, k = cfg.N, cfg.m, cfg.top_k
    q_pos = _t(qs["q_pos"][None])
    n_comp = _t(np.array([N], np.int32))
    # scores and top-k in one call, as bench.py runs them (scores in the workspace's first bytes)
    ws = torch.empty(L.indexer_score_topk_workspace_bytes(1, T, N, k), dtype=torch.uint8, device=DEV)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    L.indexer_score_topk(_bf(qs["q_idx"][None]), _t(qs["w"][None]), _bf(tok["k_idx"][None]), None, q_pos, n_comp,
                         idx, m=m, ws=ws)
    scores = ws[:T * N * 4].view(torch.float32).view(1, T, N)
    out = torch.empty((T, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, cfg.H), device=DEV)
    L.sparse_mqa_prefill(_bf(qs["q"]), comp_t[0], idx[0], _kv(cfg, tok["kv_tok"]), q_pos[0], _t(tok["sink"]), out,
                         lse, W=cfg.W)
    torch.cuda.synchronize()
    return qs, host(scores)[0], host(idx)[0], host(out), host(lse)


def check_prefill(cfg, chunks, picks):
    L = _L()
    tok = gen.gen_prefill_tokens(cfg)
    fp8 = cfg.kv_dtype == "fp8"
    comp_t = (torch.empty((1, cfg.N, cfg.D + 64), dtype=torch.uint8, device=DEV) if fp8
              else torch.empty((1, cfg.N, cfg.D), dtype=torch.bfloat16, device=DEV))
    L.csa_compress(*(_bf(tok[nm][None]) for nm in ("Ca", "Cb", "Za", "Zb")), _t(tok["Ba"]), _t(tok["Bb"]), comp_t,
                   m=cfg.m)
    torch.cuda.synchronize()
    comp_rows = host(comp_t)[0]
    comp = _kv_values(cfg, comp_rows)  # the stored entries' values
    kv_tok = _kv_values(cfg, tok["kv_tok"])
    ref_comp_rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(cfg.N // 2 - 32, cfg.N // 2 + 32),
                                              np.arange(cfg.N - 64, cfg.N)]))
    ref_comp = oracle.compress(tok["Ca"], tok["Cb"], tok["Za"], tok["Zb"], tok["Ba"], tok["Bb"], cfg.m,
                               blocks=[int(r) for r in ref_comp_rows])
    for r, ent in zip(ref_comp_rows, ref_comp):
        _check_entry(cfg, comp_rows[r], ent, f"prefill compress row {r}")
    for c in chunks:
        qs, S, I, O, LSE = run_prefill_chunk(cfg, tok, comp_t, c)
        T = len(qs["q_pos"])
        pk = picks(c) if getattr(picks, "per_chunk", False) else picks
        for t in pk(T):
            p = int(qs["q_pos"][t])
            print(f"[case] {cfg.name} chunk {c} query {t} pos {p}", flush=True)
            win = oracle.window_rows(kv_tok, p, cfg.W)
            V = oracle.visible(p, cfg.N, cfg.m)
            s = oracle.indexer_scores(qs["q_idx"][t], qs["w"][t], tok["k_idx"], V)
            assert np.abs(S[t, :V] - s).max(initial=0.0) <= 2e-5 * 8 * (1 + np.abs(s).max(initial=0.0))
            oidx = oracle.topk_select(s, cfg.top_k)
            check_topk_row(I[t], oidx, s, cfg.top_k, f"prefill t={t}")
            rows = np.concatenate([comp[I[t][I[t] >= 0]].astype(np.float64), win])
            o_own, lse_own = oracle.attend(qs["q"][t], rows, tok["sink"])
            check_out(O[t], o_own, _tight(o_own), f"prefill out t={t}")
            assert np.abs(LSE[t] - lse_own).max() < 1e-3


def test_csa_prefill_reduced_two_chunks():
    cfg = gen.scaled(gen.C3, n=8192, Tq=8192)
    rng = np.random.default_rng(7)
    check_prefill(cfg, [0, 1], lambda T: sorted(set([0, 1, 2, 3, 4, 63, 64, 2047, T - 2, T - 1]
                                                     + list(rng.integers(0, T, 20)))))


def test_csa_prefill_kv_fp8_reduced_two_chunks():
    cfg = gen.scaled(gen.C3F, n=8192, Tq=8192)
    rng = np.random.default_rng(11)
    check_prefill(cfg, [0, 1], lambda T: sorted(set([0, 1, 2, 3, 4, 2047, T - 1] + list(rng.integers(0, T, 16)))))


def test_csa_prefill_64k_kv_fp8_last_chunk_sampled():
    cfg = gen.C3F  # mixed-precision main KV, as bench.py runs it
    rng = np.random.default_rng(12)
    check_prefill(cfg, [gen.num_chunks(cfg) - 1], lambda T: sorted(set([0, T - 1] + list(rng.integers(0, T, 6)))))


def test_csa_prefill_64k_last_chunk_sampled():
    cfg = gen.C3  # 65536 tokens; the last (largest) 4096-query chunk, as bench.py runs it
    rng = np.random.default_rng(8)
    check_prefill(cfg, [gen.num_chunks(cfg) - 1], lambda T: sorted(set([0, 1, T - 1] + list(rng.integers(0, T, 8)))))


def test_csa_prefill_64k_all_chunks_sampled():
    """Every 4096-query chunk of the 64K prefill through the GPU path, sampled:
    the first and last 64 queries of the sequence, the 8 queries on each side
    of every chunk boundary, and a few random queries per chunk."""
    cfg = gen.C3
    nch = gen.num_chunks(cfg)
    rng = np.random.default_rng(13)

    def picks(c):
        def f(T):
            p = set(range(8)) | set(range(T - 8, T)) | set(rng.integers(0, T, 4).tolist())
            if c == 0:
                p |= set(range(64))
            if c == nch - 1:
                p |= set(range(T - 64, T))
            return sorted(p)
        return f

    picks.per_chunk = True
    check_prefill(cfg, list(range(nch)), picks)


def check_csa_decode_multi(cfg, seqs):
    """Tq query tokens per sequence in one step (positions n-Tq .. n-1): the
    completed entry is appended, each token is scored and selected at its own
    position, and attends its own rows and its window (the W buffer rows
    ending at its token), as bench.py runs it."""
    L = _L()
    x = gen.gen_decode(cfg)
    B, N, m, k, W, Tq = cfg.B, cfg.N, cfg.m, cfg.top_k, cfg.W, cfg.Tq
    kv = _kv(cfg, x["kv_comp"])
    pos = np.tile(np.arange(cfg.n - Tq, cfg.n, dtype=np.int32), (B, 1))
    q_pos, n_comp = _t(pos), _t(np.full((B,), N, np.int32))
    ws = torch.zeros(L.indexer_score_topk_workspace_bytes(B, Tq, N, k), dtype=torch.uint8, device=DEV)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    L.csa_compress_indexer_score_topk(_bf(x["Ca"]), _bf(x["Cb"]), _bf(x["Za"]), _bf(x["Zb"]), _t(x["Ba"]),
                                      _t(x["Bb"]), kv, _bf(x["q_idx"]), _t(x["w"]), _bf(x["k_idx"]), None, q_pos,
                                      n_comp, idx, m_c=m, m=m, tok_begin=cfg.n - 2 * m, blk_begin=N - 1, blk_end=N,
                                      ws=ws)
    scores = ws[:B * Tq * N * 4].view(torch.float32).view(B, Tq, N)
    out = torch.empty((B, Tq, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Tq, cfg.H), device=DEV)
    L.sparse_mqa_decode_multi(_bf(x["q"]), kv, idx, _kv(cfg, x["kv_win"]), _t(np.full((B,), W + Tq - 1, np.int32)),
                              _t(x["sink"]), out, lse)
    torch.cuda.synchronize()
    kv2, S, I, O, LSE = host(kv[:, N - 2:]), host(scores), host(idx), host(out), host(lse)
    for b in seqs:
        ent = oracle.compress(x["Ca"][b], x["Cb"][b], x["Za"][b], x["Zb"][b], x["Ba"], x["Bb"], m,
                              blocks=range(1, 2))[0]
        _check_entry(cfg, kv2[b, 1], ent, "compressed entry N-1")
        comp = _kv_values(cfg, x["kv_comp"][b])
        comp[N - 1] = _kv_values(cfg, kv2[b, 1])
        win = _kv_values(cfg, x["kv_win"][b])
        for t in range(Tq):
            p = cfg.n - Tq + t
            print(f"[case] {cfg.name} b={b} t={t} pos {p}", flush=True)
            wrows = win[t:t + W]  # full buffer: token t's window is rows t .. t+W-1
            oidx, o_ref, lse_ref, sc = oracle.csa_query(x["q"][b][t], x["q_idx"][b][t], x["w"][b][t], comp,
                                                        x["k_idx"][b], p, N, m, k, wrows, x["sink"])
            V = oracle.visible(p, N, m)
            assert np.abs(S[b, t, :V] - sc).max() <= 2e-5 * 8 * (1 + np.abs(sc).max())
            check_topk_row(I[b, t], oidx, sc, k, f"b={b} t={t}")
            rows = np.concatenate([comp[I[b, t][I[b, t] >= 0]], wrows])
            o_own, lse_own = oracle.attend(x["q"][b][t], rows, x["sink"])
            check_out(O[b, t], o_own, _tight(o_own), f"multi out b={b} t={t}")
            assert np.abs(LSE[b, t] - lse_own).max() < 1e-3
            if np.array_equal(I[b, t], oidx):
                check_out(O[b, t], o_ref, _tight(o_ref), f"multi end to end b={b} t={t}")


def test_csa_decode_flash_2tok_reduced():
    check_csa_decode_multi(gen.scaled(gen.C2M, B=4, n=16384), range(4))


def test_csa_decode_flash_2tok_full_size_sampled():
    check_csa_decode_multi(gen.C2M, [0, 19, 31])


def test_csa_decode_flash_qk_rope_reduced():
    cfg = gen.scaled(gen.C2R, B=4, n=16384)  # query RMSNorm + RoPE prologue, output inverse RoPE
    check_csa_decode(cfg, gen.gen_decode(cfg), range(cfg.B))


def test_csa_decode_flash_qk_rope_full_size_sampled():
    cfg = gen.C2R
    check_csa_decode(cfg, gen.gen_decode(cfg), [0, 21, 31])


def test_csa_decode_flash_mxfp4_reduced():
    cfg = gen.scaled(gen.C2X, B=4, n=16384)
    check_csa_decode(cfg, gen.gen_decode(cfg), range(cfg.B))


def test_csa_decode_flash_mxfp4_full_size_sampled():
    cfg = gen.C2X  # 32 sequences x 32768 entries, MXFP4 indexer keys, as bench.py runs it
    check_csa_decode(cfg, gen.gen_decode(cfg), [0, 17, 31])


def test_csa_decode_flash_fp4_qk_reduced():
    cfg = gen.scaled(gen.C2Q, B=4, n=16384)
    check_csa_decode(cfg, gen.gen_decode(cfg), range(cfg.B))


def test_csa_decode_flash_fp4_qk_full_size_sampled():
    cfg = gen.C2Q  # C2X with the indexer query quantised to MXFP4 in the call, as bench.py runs it
    check_csa_decode(cfg, gen.gen_decode(cfg), [0, 13, 31])


def check_hca_prefill(cfg, chunks, picks):
    """Single-branch compression of the whole sequence at m' (HCA), then
    hca_prefill by 4096-query chunks, as bench.py runs it."""
    L = _L()
    tok = gen.gen_prefill_tokens(cfg)
    comp_t = torch.empty((1, cfg.N, cfg.D), dtype=torch.bfloat16, device=DEV)
    L.csa_compress(_bf(tok["Ca"][None]), None, _bf(tok["Za"][None]), None, _t(tok["Ba"]), None, comp_t, m=cfg.m,
                   overlap=False)
    torch.cuda.synchronize()
    comp = host(comp_t)[0]
    rows = sorted(set([0, 1, cfg.N // 2, cfg.N - 2, cfg.N - 1]))
    ref_comp = oracle.compress(tok["Ca"], None, tok["Za"], None, tok["Ba"], None, cfg.m, overlap=False, blocks=rows)
    check_out(comp[rows], ref_comp, 2.0 ** -8 * max(1.0, np.abs(ref_comp).max()), "hca prefill compress")
    kv_tok = _bf(tok["kv_tok"])
    for c in chunks:
        qs = gen.gen_prefill_queries(cfg, c)
        T = len(qs["q_pos"])
        out = torch.empty((T, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((T, cfg.H), device=DEV)
        L.hca_prefill(_bf(qs["q"]), comp_t[0], kv_tok, _t(qs["q_pos"]), _t(tok["sink"]), out, lse, m=cfg.m, W=cfg.W)
        torch.cuda.synchronize()
        O, LSE = host(out), host(lse)
        for t in picks(T):
            p = int(qs["q_pos"][t])
            print(f"[case] {cfg.name} chunk {c} query {t} pos {p}", flush=True)
            # the stored (bf16) entries are what the queries attend
            ref, rlse = oracle.hca_query(qs["q"][t], comp.astype(np.float64), p, cfg.N, cfg.m,
                                         oracle.window_rows(tok["kv_tok"], p, cfg.W), tok["sink"])
            check_out(O[t], ref, _tight(ref), f"hca prefill out t={t}")
            assert np.abs(LSE[t] - rlse).max() < 1e-3


def test_hca_prefill_reduced_two_chunks():
    cfg = gen.scaled(gen.C6, n=8192, Tq=8192)
    rng = np.random.default_rng(9)
    check_hca_prefill(cfg, [0, 1], lambda T: sorted(set([0, 1, 126, 127, 128, 255, 2047, T - 2, T - 1]
                                                         + list(rng.integers(0, T, 20)))))


def test_hca_prefill_64k_last_chunk_sampled():
    cfg = gen.C6  # 65536 tokens; the last 4096-query chunk (512 entries visible), as bench.py runs it
    rng = np.random.default_rng(10)
    check_hca_prefill(cfg, [gen.num_chunks(cfg) - 1], lambda T: sorted(set([0, 1, T - 1] + list(rng.integers(0, T, 8)))))


def test_determinism_and_batch_invariance():
    """Two runs are bitwise equal, and a sequence's output does not depend on
    the batch it is in."""
    cfg = gen.scaled(gen.C2, B=4, n=8192)
    x = gen.gen_decode(cfg)
    a = run_csa_decode(cfg, x)
    b = run_csa_decode(cfg, x)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    x1 = {k: v[None] for k, v in gen.gen_decode_seq(cfg, 2).items()}
    x1.update(gen.gen_shared(cfg))
    one = run_csa_decode(gen.scaled(cfg, B=1), x1)
    for u, v in zip(one, a):
        assert np.array_equal(u[0], v[2])


def run_decode_step(cfg, x, ws=None, seqs_nc=None):
    """The whole step through csa_decode_step, and the same step through the
    separate calls; returns both results (kv row N-1, idx, out, lse)."""
    L = _L()
    B, N, m, k, W, Tq = cfg.B, cfg.N, cfg.m, cfg.top_k, cfg.W, cfg.Tq
    pos = np.tile(np.arange(cfg.n - Tq, cfg.n, dtype=np.int32), (B, 1))
    nc = np.full((B,), N, np.int32) if seqs_nc is None else np.asarray(seqs_nc, np.int32)
    q_pos, n_comp = _t(pos), _t(nc)
    if cfg.k_dtype == "fp8":
        k_t, sc = _t(x["k_idx_codes"]), _t(x["k_scale"])
    elif cfg.k_dtype == "mxfp4":
        k_t, sc = _t(x["k_idx_codes"]).view(torch.float4_e2m1fn_x2), _t(x["k_scale"])
    else:
        k_t, sc = _bf(x["k_idx"]), None
    qi = _bf(x["q_idx"] if Tq > 1 else x["q_idx"][:, None])
    wt = _t(x["w"] if Tq > 1 else x["w"][:, None])
    q = _bf(x["q"] if Tq > 1 else x["q"][:, None])
    win, wl = _kv(cfg, x["kv_win"]), _t(np.full((B,), W + Tq - 1, np.int32))
    comp = [_bf(x[nm]) for nm in ("Ca", "Cb", "Za", "Zb")]
    res = []
    for fused in (True, False):
        kv = _kv(cfg, x["kv_comp"])
        idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=DEV)
        tsc = torch.full((B, Tq, k), 7.0, device=DEV)
        out = torch.empty((B, Tq, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, Tq, cfg.H), device=DEV)
        if fused:
            L.csa_decode_step(*comp, _t(x["Ba"]), _t(x["Bb"]), qi, wt, k_t, sc, q_pos, n_comp, q, kv, win, wl,
                              _t(x["sink"]), idx, out, lse, tsc, m_c=m, m=m, tok_begin=cfg.n - 2 * m, blk_begin=N - 1,
                              blk_end=N, ws=ws, q_fp4=cfg.q_fp4)
        else:
            L.csa_compress_indexer_score_topk(*comp, _t(x["Ba"]), _t(x["Bb"]), kv, qi, wt, k_t, sc, q_pos, n_comp,
                                              idx, tsc, m_c=m, m=m, tok_begin=cfg.n - 2 * m, blk_begin=N - 1,
                                              blk_end=N, q_fp4=cfg.q_fp4)
            L.sparse_mqa_decode_multi(q, kv, idx, win, wl, _t(x["sink"]), out, lse)
        torch.cuda.synchronize()
        res.append((host(kv[:, N - 1]), host(idx), host(tsc), host(out), host(lse)))
    return res


def _same(a, b, what):
    for i, nm in enumerate(("kv row N-1", "idx", "topk scores", "out", "lse")):
        assert np.array_equal(a[i], b[i], equal_nan=True), f"{what}: {nm} differs between the fused and separate paths"


@pytest.mark.parametrize("name", ["c2_reduced", "c2m_reduced", "c2f_reduced", "c2x_reduced", "c2q_reduced",
                                  "c5_reduced"])
def test_decode_step_equals_separate_reduced(name):
    base = {"c2_reduced": gen.C2, "c2m_reduced": gen.C2M, "c2f_reduced": gen.C2F, "c2x_reduced": gen.C2X,
            "c2q_reduced": gen.C2Q, "c5_reduced": gen.C5}[name]
    cfg = gen.scaled(base, B=6, n=4 * 40000 if base is gen.C5 else 16384)
    x = gen.gen_decode(cfg)
    print(f"[case] decode step {name}", flush=True)
    fz, sp = run_decode_step(cfg, x)
    _same(fz, sp, name)
    # short rows: sequences that see fewer entries than top_k or just over it
    nc = [cfg.N, 3, cfg.top_k, cfg.top_k + 1, cfg.N // 2 + 1, 1]
    fz, sp = run_decode_step(cfg, x, seqs_nc=nc)
    _same(fz, sp, name + " short rows")
    K = np.minimum(cfg.top_k, np.asarray(nc))
    for b in range(cfg.B):
        for t in range(cfg.Tq):
            assert np.all(fz[1][b, t, K[b]:] == -1) and np.all(np.isneginf(fz[2][b, t, K[b]:]))


def test_decode_step_workspace_garbage_and_reuse():
    cfg = gen.scaled(gen.C2, B=5, n=65536)
    x = gen.gen_decode(cfg)
    L = _L()
    nb = L.csa_decode_step_workspace_bytes(cfg.B, 1, cfg.N, cfg.top_k, cfg.H, cfg.D, cfg.W)
    for what, ws in (("garbage", torch.randint(0, 256, (nb,), dtype=torch.uint8, device=DEV)),
                     ("zeroed", torch.zeros(nb, dtype=torch.uint8, device=DEV))):
        for rep in range(2):  # the second call reads what the first left
            print(f"[case] decode step workspace {what} call {rep}", flush=True)
            fz, sp = run_decode_step(cfg, x, ws=ws)
            _same(fz, sp, f"{what} workspace, call {rep}")


@pytest.mark.parametrize("name", ["c2", "c5", "c2m"])
def test_decode_step_full_size_sampled(name):
    """The step as bench.py runs it, at full size: the same bits as the
    separate calls, and sampled sequences against the oracle."""
    cfg = {"c2": gen.C2, "c5": gen.C5, "c2m": gen.C2M}[name]
    x = gen.gen_decode(cfg)
    print(f"[case] decode step {cfg.name}", flush=True)
    fz, sp = run_decode_step(cfg, x)
    _same(fz, sp, cfg.name)
    kvN1, I, TS, O, LSE = fz
    m, N = cfg.m, cfg.N
    for b in ([0, cfg.B - 1] if cfg.B > 2 else [0]):
        ent = oracle.compress(x["Ca"][b], x["Cb"][b], x["Za"][b], x["Zb"][b], x["Ba"], x["Bb"], m,
                              blocks=range(1, 2))[0]
        _check_entry(cfg, kvN1[b], ent, "compressed entry N-1")
        comp = _kv_values(cfg, x["kv_comp"][b])
        comp[N - 1] = _kv_values(cfg, kvN1[b])
        if cfg.k_dtype == "fp8":
            keys, ksc = oracle.e4m3_decode(x["k_idx_codes"][b]), x["k_scale"][b]
        else:
            keys, ksc = x["k_idx"][b], None
        win = _kv_values(cfg, x["kv_win"][b])
        for t in range(cfg.Tq):
            p = cfg.n - cfg.Tq + t
            print(f"[case] {cfg.name} b={b} t={t}", flush=True)
            q = x["q"][b][t] if cfg.Tq > 1 else x["q"][b]
            qi = x["q_idx"][b][t] if cfg.Tq > 1 else x["q_idx"][b]
            wv = x["w"][b][t] if cfg.Tq > 1 else x["w"][b]
            wrows = win[t:t + cfg.W]
            oidx, o_ref, lse_ref, s = oracle.csa_query(q, qi, wv, comp, keys, p, N, m, cfg.top_k, wrows, x["sink"],
                                                       k_scale=ksc)
            check_topk_row(I[b, t], oidx, s, cfg.top_k, f"b={b} t={t}")
            rows = np.concatenate([comp[I[b, t][I[b, t] >= 0]], wrows])
            o_own, lse_own = oracle.attend(q, rows, x["sink"])
            check_out(O[b, t], o_own, _tight(o_own), f"out on gpu idx b={b} t={t}")
            assert np.abs(LSE[b, t] - lse_own).max() < 1e-3


def run_decode_step_qk(cfg, x):
    """csa_decode_step_qk on the raw queries, and the same through
    qk_norm_rope + csa_decode_step + the inverse rotation."""
    L = _L()
    B, N, m, k, W = cfg.B, cfg.N, cfg.m, cfg.top_k, cfg.W
    pos = np.full((B, 1), cfg.n - 1, np.int32)
    q_pos, n_comp = _t(pos), _t(np.full((B,), N, np.int32))
    k_t = _bf(x["k_idx"])
    qi, wt, q = _bf(x["q_idx"][:, None]), _t(x["w"][:, None]), _bf(x["q"][:, None])
    win, wl = _kv(cfg, x["kv_win"]), _t(np.full((B,), W, np.int32))
    comp = [_bf(x[nm]) for nm in ("Ca", "Cb", "Za", "Zb")]
    gamma, scale = _t(x["q_gamma"]), 1.0 / np.sqrt(cfg.D)
    res = []
    for fused in (True, False):
        kv = _kv(cfg, x["kv_comp"])
        idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
        out = torch.empty((B, 1, cfg.H, cfg.D), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, 1, cfg.H), device=DEV)
        args = (*comp, _t(x["Ba"]), _t(x["Bb"]), qi, wt, k_t, None, q_pos, n_comp)
        kw = dict(m_c=m, m=m, tok_begin=cfg.n - 2 * m, blk_begin=N - 1, blk_end=N, scale=scale)
        if fused:
            L.csa_decode_step_qk(*args, q, kv, win, wl, _t(x["sink"]), idx, out, lse, q_gamma=gamma, **kw)
        else:
            qn = torch.empty_like(q)
            L.qk_norm_rope(q.view(B, cfg.H, cfg.D), qn.view(B, cfg.H, cfg.D), q_pos.view(B), gamma, norm=True,
                           rope=True)
            L.csa_decode_step(*args, qn, kv, win, wl, _t(x["sink"]), idx, out, lse, **kw)
            L.qk_norm_rope(out.view(B, cfg.H, cfg.D), out.view(B, cfg.H, cfg.D), q_pos.view(B), inverse=True)
        torch.cuda.synchronize()
        res.append((host(kv[:, N - 1]), host(idx)[:, 0], host(out)[:, 0], host(lse)[:, 0]))
    return res


def _check_step_qk(cfg, seqs):
    x = gen.gen_decode(cfg, with_compress=True)
    (kvf, If, Of, Lf), (kvs, Is, Os, Ls) = run_decode_step_qk(cfg, x)
    assert np.array_equal(kvf, kvs) and np.array_equal(If, Is), "entry / selection differ from the separate calls"
    N, m = cfg.N, cfg.m
    for b in range(cfg.B):
        # the fused prologue sums its squares in another order, and the
        # fused epilogue rotates before the one rounding of the output
        check_out(Of[b], Os[b], out_bound(Os[b]), f"step_qk vs separate b={b}")
        assert np.abs(Lf[b] - Ls[b]).max() < 1e-3
    for b in seqs:
        print(f"[case] {cfg.name} step_qk b={b}", flush=True)
        comp = _kv_values(cfg, x["kv_comp"][b])
        comp[N - 1] = _kv_values(cfg, kvf[b])
        p = cfg.n - 1
        q = gen.bf16_round(oracle.rope_rotate(oracle.rms_norm(x["q"][b][None], x["q_gamma"], 1e-6), [p])[0]
                           .astype(np.float32)).astype(np.float64)
        tau = 1.0 / np.sqrt(cfg.D)
        oidx, o_ref, lse_ref, s = oracle.csa_query(q, x["q_idx"][b], x["w"][b], comp, x["k_idx"][b], p, N, m,
                                                   cfg.top_k, _kv_values(cfg, x["kv_win"][b]), x["sink"], tau=tau)
        check_topk_row(If[b], oidx, s, cfg.top_k, f"b={b}")
        rows = np.concatenate([comp[If[b][If[b] >= 0]], _kv_values(cfg, x["kv_win"][b])])
        o_own, lse_own = oracle.attend(q, rows, x["sink"], tau)
        o_own = oracle.rope_rotate(o_own[None], [p], inverse=True)[0]
        check_out(Of[b], o_own, _tight(o_own), f"step_qk out on gpu idx b={b}")
        assert np.abs(Lf[b] - lse_own).max() < 1e-3


def test_decode_step_qk_reduced():
    _check_step_qk(gen.scaled(gen.C2R, B=5, n=16384), range(5))


def test_decode_step_qk_full_size_sampled():
    _check_step_qk(gen.C2R, [0, 17, 31])
