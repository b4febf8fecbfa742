"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, invariants, limits, library routines (torch SDPA, numpy sort,
torch's float8 decoding), brute force on tiny inputs and the figures the pages
state (tests/golden/page_constants.json).

Every check takes the oracle as an argument (``o``), so the mutation tests can
run the same checks against deliberately broken copies of it and show that a
plausible mistake fails at least one check.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- compression

def check_compress_constant_values(o):
    """C_a and C_b constant per channel => every entry is c_a (+ c_b for i>=1),
    whatever the logits and biases: the softmax weights sum to one."""
    g = _rng(1)
    n, d, m = 37, 5, 4
    ca, cb = g.normal(size=d), g.normal(size=d)
    Ca, Cb = np.tile(ca, (n, 1)), np.tile(cb, (n, 1))
    Za, Zb = g.normal(size=(n, d)) * 3, g.normal(size=(n, d)) * 3
    Ba, Bb = g.normal(size=(m, d)), g.normal(size=(m, d))
    out = o.compress(Ca, Cb, Za, Zb, Ba, Bb, m)
    assert out.shape == (n // m, d)
    assert np.allclose(out[0], ca, atol=1e-12)
    assert np.allclose(out[1:], ca + cb, atol=1e-12)


def check_compress_uniform_logits_block_means(o):
    """Equal logits and zero bias => entry i = mean of C_a over block i plus
    mean of C_b over block i-1 (numpy mean, not the oracle's softmax)."""
    g = _rng(2)
    n, d, m = 40, 6, 4
    Ca, Cb = g.normal(size=(n, d)), g.normal(size=(n, d))
    Z = np.full((n, d), 0.7)
    B0 = np.zeros((m, d))
    out = o.compress(Ca, Cb, Z, Z, B0, B0, m)
    for i in range(n // m):
        want = Ca[m * i:m * i + m].mean(axis=0)
        if i >= 1:
            want = want + Cb[m * (i - 1):m * i].mean(axis=0)
        assert np.allclose(out[i], want, atol=1e-12)


def check_compress_dominant_token(o):
    """A logit far above the others selects that one token of the block:
    entry i = C_a[m*i + j*] + C_b[m*(i-1) + j2] (exact up to e^-1000)."""
    g = _rng(3)
    n, d, m = 32, 3, 4
    Ca, Cb = g.normal(size=(n, d)), g.normal(size=(n, d))
    Za, Zb = g.normal(size=(n, d)), g.normal(size=(n, d))
    ja = g.integers(0, m, size=(n // m, d))
    jb = g.integers(0, m, size=(n // m, d))
    for i in range(n // m):
        for c in range(d):
            Za[m * i + ja[i, c], c] += 1000.0
            Zb[m * i + jb[i, c], c] += 1000.0
    z = np.zeros((m, d))
    out = o.compress(Ca, Cb, Za, Zb, z, z, m)
    for i in range(n // m):
        for c in range(d):
            want = Ca[m * i + ja[i, c], c]
            if i >= 1:
                want += Cb[m * (i - 1) + jb[i - 1, c], c]
            assert abs(out[i, c] - want) < 1e-12


def check_compress_bias_is_positional(o):
    """A large bias at position j* of the block selects token j* of every
    block (the bias is indexed by position-in-block, per channel)."""
    g = _rng(4)
    n, d, m = 24, 2, 4
    Ca, Cb = g.normal(size=(n, d)), g.normal(size=(n, d))
    Z = g.normal(size=(n, d))
    Ba = np.zeros((m, d)); Ba[1, 0] = 1000.0; Ba[3, 1] = 1000.0
    Bb = np.zeros((m, d)); Bb[2, 0] = 1000.0; Bb[0, 1] = 1000.0
    out = o.compress(Ca, Cb, Z, Z, Ba, Bb, m)
    for i in range(n // m):
        want0 = Ca[m * i + 1, 0] + (Cb[m * (i - 1) + 2, 0] if i else 0.0)
        want1 = Ca[m * i + 3, 1] + (Cb[m * (i - 1) + 0, 1] if i else 0.0)
        assert abs(out[i, 0] - want0) < 1e-12 and abs(out[i, 1] - want1) < 1e-12


def check_compress_m1_identity(o):
    """m = 1 without the overlap branch is the identity."""
    g = _rng(5)
    n, d = 9, 4
    Ca = g.normal(size=(n, d))
    out = o.compress(Ca, None, g.normal(size=(n, d)), None, g.normal(size=(1, d)), None, 1,
                     overlap=False)
    assert np.allclose(out, Ca, atol=1e-15)


def check_compress_causal_support_and_tail(o):
    """Entry i reads exactly tokens [m(i-1), m(i+1)); tail tokens form no entry."""
    g = _rng(6)
    n, d, m = 27, 3, 4  # 3 tail tokens
    arrs = [g.normal(size=(n, d)) for _ in range(4)]
    Ba, Bb = g.normal(size=(m, d)), g.normal(size=(m, d))
    base = o.compress(*arrs, Ba, Bb, m)
    assert base.shape[0] == n // m
    for t in range(n):
        pert = [a.copy() for a in arrs]
        for a in pert:
            a[t] += 1.5
        out = o.compress(*pert, Ba, Bb, m)
        changed = np.abs(out - base).max(axis=1) > 0
        expect = np.array([(m * (i - 1) <= t < m * (i + 1)) if i >= 1 else (t < m)
                           for i in range(n // m)])
        assert np.array_equal(changed, expect), (t, changed, expect)


def check_compress_joint_closed_form(o):
    """Joint reading: one softmax over both blocks' 2m logits. With equal
    logits and constant values it averages: (c_a + c_b)/2 for i >= 1."""
    n, d, m = 16, 2, 4
    ca, cb = np.array([1.0, -2.0]), np.array([3.0, 5.0])
    Ca, Cb = np.tile(ca, (n, 1)), np.tile(cb, (n, 1))
    Z = np.zeros((n, d)); B0 = np.zeros((m, d))
    out = o.compress(Ca, Cb, Z, Z, B0, B0, m, joint=True)
    assert np.allclose(out[0], ca) and np.allclose(out[1:], (ca + cb) / 2)


def check_compress_hca_sizes(o):
    """Page figure: one million tokens at m' = 128 give 7812 entries."""
    fx = json.load(open(os.path.join(GOLDEN, "page_constants.json")))["hca_entries_at_1m_tokens"]
    n, m = fx["n_tokens"], fx["m_prime"]
    x = np.zeros((n, 1))
    out = o.compress(x, None, x, None, np.zeros((m, 1)), None, m, overlap=False)
    assert out.shape[0] == fx["entries"]


# --------------------------------------------------------------------- indexer

def check_indexer_single_head_argsort(o):
    """One head, weight 1: the selection is numpy's stable argsort of
    -ReLU(k @ q), first K, ascending."""
    g = _rng(7)
    V, D, k = 50, 8, 7
    q, K = g.normal(size=(1, D)), g.normal(size=(V, D))
    s = o.indexer_scores(q, np.ones(1), K, V)
    ref = np.maximum(K @ q[0], 0.0)
    assert np.allclose(s, ref, atol=1e-12)
    want = np.sort(np.argsort(-ref, kind="stable")[:k])
    assert np.array_equal(o.topk_select(s, k)[:k], want)


def check_indexer_unit_query(o):
    """q = unit vector e_c => <q, k_i> is k_i[c]; s_i = sum_h w_h max(0, k_i[c_h])."""
    g = _rng(8)
    V, D, H = 20, 6, 3
    K = g.normal(size=(V, D))
    cs = [0, 4, 2]
    q = np.zeros((H, D))
    for h, c in enumerate(cs):
        q[h, c] = 1.0
    w = np.array([0.5, -1.25, 2.0])
    s = o.indexer_scores(q, w, K, V)
    for i in range(V):
        want = sum(w[h] * max(0.0, K[i, cs[h]]) for h in range(H))
        assert abs(s[i] - want) < 1e-12


def check_indexer_relu_before_weight(o):
    """Negative weights act after the ReLU: an entry whose dots are all
    negative scores exactly 0, never a positive value."""
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    K = np.array([[-1.0, -2.0], [1.0, 1.0]])
    s = o.indexer_scores(q, np.array([-1.0, -1.0]), K, 2)
    assert s[0] == 0.0 and abs(s[1] + 2.0) < 1e-15


def check_indexer_fp8_scale(o):
    """The per-entry scale multiplies the dot product: scoring codes with
    scale sigma equals scoring the dequantized keys without a scale."""
    g = _rng(9)
    V, D, H = 30, 16, 4
    codes = g.integers(0, 256, size=(V, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10  # no NaN codes
    vals = o.e4m3_decode(codes)
    sc = g.uniform(0.01, 2.0, size=V)
    q, w = g.normal(size=(H, D)), g.normal(size=H)
    a = o.indexer_scores(q, w, vals, V, sc)
    b = o.indexer_scores(q, w, vals * sc[:, None], V)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def check_indexer_visibility(o):
    """Only entries i < V(p) = min(N, floor((p+1)/m)) are scored."""
    assert o.visible(0, 100, 4) == 0 and o.visible(3, 100, 4) == 1
    assert o.visible(6, 100, 4) == 1 and o.visible(7, 100, 4) == 2
    assert o.visible(10 ** 6, 5, 4) == 5
    g = _rng(10)
    K = g.normal(size=(10, 4))
    s = o.indexer_scores(g.normal(size=(2, 4)), np.ones(2), K, 6)
    assert s.shape == (6,)


def check_indexer_invariances_and_needle(o):
    """Positive rescaling of q and w and a permutation of heads leave the
    selection unchanged; a planted needle entry is always selected."""
    g = _rng(11)
    V, D, H, k = 300, 16, 8, 12
    q, w, K = g.normal(size=(H, D)) / 4, g.uniform(0.1, 1, size=H), g.normal(size=(V, D))
    base = o.topk_select(o.indexer_scores(q, w, K, V), k)
    perm = g.permutation(H)
    assert np.array_equal(o.topk_select(o.indexer_scores(q[perm] * 3.0, w[perm] * 0.25, K, V), k), base)
    K2 = K.copy()
    K2[137] = 10.0 * q.mean(axis=0) * D
    assert 137 in o.topk_select(o.indexer_scores(q, w, K2, V), k)


def check_topk_ties_short_rows_padding(o):
    """All-equal scores: the k lowest indices win; V < k keeps all V and pads
    with -1; the output is ascending."""
    assert list(o.topk_select(np.zeros(10), 4)) == [0, 1, 2, 3]
    assert list(o.topk_select(np.array([3.0, 1.0, 2.0]), 5)) == [0, 1, 2, -1, -1]
    s = np.array([5.0, 9.0, 5.0, 1.0, 9.0, 5.0])
    assert list(o.topk_select(s, 3)) == [0, 1, 4]
    assert list(o.topk_select(np.zeros(0), 2)) == [-1, -1]


def check_e4m3_decode_vs_torch(o):
    """All 256 E4M3 codes decode to torch.float8_e4m3fn's values (library),
    NaN codes to NaN."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    mine = o.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])


# ------------------------------------------------------------------- attention

def _sdpa_with_sink(q, rows, sink, tau):
    """torch scaled_dot_product_attention (float64, CPU); the sink is an extra
    zero key/value column whose logit is set by the additive mask."""
    import torch
    H, D = q.shape
    R = rows.shape[0]
    qt = torch.tensor(q, dtype=torch.float64).reshape(1, H, 1, D)
    kv = np.concatenate([rows, np.zeros((1, D))], axis=0)
    kt = torch.tensor(kv, dtype=torch.float64).reshape(1, 1, R + 1, D).expand(1, H, R + 1, D).contiguous()
    mask = torch.zeros(1, H, 1, R + 1, dtype=torch.float64)
    mask[0, :, 0, R] = torch.tensor(sink, dtype=torch.float64)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=mask, scale=tau)
    logits = torch.cat([(qt[0, :, 0] @ kt[0, 0, :R].T) * tau, torch.tensor(sink, dtype=torch.float64)[:, None]], 1)
    return out.reshape(H, D).numpy(), torch.logsumexp(logits, dim=1).numpy()


def check_attend_vs_sdpa(o):
    g = _rng(12)
    H, D, R = 4, 16, 23
    q, rows, sink = g.normal(size=(H, D)) / 4, g.normal(size=(R, D)), g.normal(size=H)
    for tau in (1.0, 0.37):
        out, lse = o.attend(q, rows, sink, tau)
        ref, rlse = _sdpa_with_sink(q, rows, sink, tau)
        assert np.allclose(out, ref, atol=1e-12) and np.allclose(lse, rlse, atol=1e-12)


def check_attend_sink_limits(o):
    g = _rng(13)
    H, D, R = 3, 8, 10
    q, rows = g.normal(size=(H, D)), g.normal(size=(R, D))
    out, _ = o.attend(q, rows, np.full(H, -1e30))
    ref, _ = _sdpa_with_sink(q, rows, np.full(H, -1e30), 1.0)
    assert np.allclose(out, ref, atol=1e-12)
    out, lse = o.attend(q, rows, np.full(H, 1e30))
    assert np.abs(out).max() == 0.0 and np.allclose(lse, 1e30)


def check_attend_closed_forms(o):
    g = _rng(14)
    H, D = 2, 5
    q = g.normal(size=(H, D))
    r = g.normal(size=D)
    out, lse = o.attend(q, r[None, :], np.full(H, -np.inf))
    assert np.allclose(out, np.tile(r, (H, 1)), atol=1e-15)
    sink = np.array([0.3, -1.2])
    cnt = 7
    out, lse = o.attend(q, np.tile(r, (cnt, 1)), sink)
    l = q @ r
    frac = 1.0 - np.exp(sink) / (np.exp(sink) + cnt * np.exp(l))
    assert np.allclose(out, frac[:, None] * r[None, :], atol=1e-13)
    assert np.allclose(lse, np.log(np.exp(sink) + cnt * np.exp(l)), atol=1e-13)
    # no rows at all: output 0, lse = sink
    out, lse = o.attend(q, np.zeros((0, D)), sink)
    assert np.abs(out).max() == 0.0 and np.allclose(lse, sink)


def check_attend_weights_sum_to_one(o):
    """Rows = identity rows: o_h holds the attention weights themselves; they
    plus the sink weight e^{sink - lse} sum to 1."""
    g = _rng(15)
    H, D = 3, 9
    q = g.normal(size=(H, D)) * 2
    sink = g.normal(size=H)
    out, lse = o.attend(q, np.eye(D), sink)
    assert np.allclose(out.sum(axis=1) + np.exp(sink - lse), 1.0, atol=1e-13)


def check_topk_all_equals_dense(o):
    """top-k >= V: the sparse CSA query equals dense attention over all
    visible entries plus the window (HCA-style with m=4), and SDPA."""
    g = _rng(16)
    n, d, m, H, HI, DI, W = 64, 8, 4, 2, 2, 4, 5
    kv_comp = g.normal(size=(n // m, d))
    kv_tok = g.normal(size=(n, d))
    K = g.normal(size=(n // m, DI))
    for p in (0, 3, 17, 63):
        q = g.normal(size=(H, d)) / 3
        win = o.window_rows(kv_tok, p, W)
        idx, out, lse, _ = o.csa_query(q, g.normal(size=(HI, DI)), g.uniform(size=HI), kv_comp, K,
                                       p, n // m, m, 10 ** 3, win, np.array([0.2, -0.4]))
        dense, dlse = o.hca_query(q, kv_comp, p, n // m, m, win, np.array([0.2, -0.4]))
        V = (p + 1) // m
        rows = np.concatenate([kv_comp[:V], kv_tok[max(0, p - W + 1):p + 1]])
        ref, rlse = _sdpa_with_sink(q, rows, np.array([0.2, -0.4]), 1.0)
        assert np.array_equal(idx[:V], np.arange(V)) and np.all(idx[V:] == -1)
        assert np.allclose(out, dense, atol=1e-12) and np.allclose(out, ref, atol=1e-12)
        assert np.allclose(lse, rlse, atol=1e-12)


def check_window_rows(o):
    kv = np.arange(20.0)[:, None]
    assert o.window_rows(kv, 10, 4)[:, 0].tolist() == [7.0, 8.0, 9.0, 10.0]
    assert o.window_rows(kv, 1, 4)[:, 0].tolist() == [0.0, 1.0]


def check_pipeline_causal(o):
    """The whole chain (compress -> score -> select -> attend) for a query at
    p is unchanged, bit for bit, when any token after p changes."""
    g = _rng(17)
    n, d, m, H, HI, DI, W, k = 48, 6, 4, 2, 3, 4, 6, 3
    T = {nm: g.normal(size=(n, d)) for nm in ("Ca", "Cb", "Za", "Zb", "kv")}
    Ba, Bb = g.normal(size=(m, d)), g.normal(size=(m, d))
    Kt = g.normal(size=(n // m, DI))  # indexer key of entry i is made from block i
    q, qi, w, sink = g.normal(size=(H, d)), g.normal(size=(HI, DI)), g.uniform(size=HI), g.normal(size=H)

    def run(T, Kt, p):
        comp = o.compress(T["Ca"][:p + 1], T["Cb"][:p + 1], T["Za"][:p + 1], T["Zb"][:p + 1], Ba, Bb, m)
        return o.csa_query(q, qi, w, comp, Kt, p, comp.shape[0], m, k, o.window_rows(T["kv"], p, W), sink)

    for p in (5, 22, 47):
        a = run(T, Kt, p)
        T2 = {kk: v.copy() for kk, v in T.items()}
        for v in T2.values():
            v[p + 1:] += 3.0
        K2 = Kt.copy()
        K2[(p + 1) // m:] += 3.0
        b = run(T2, K2, p)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def check_brute_force_tiny(o):
    """Pure-Python loops over a tiny case, written from the definitions
    without numpy linear algebra, against the oracle."""
    g = _rng(18)
    n, d, m, H, HI, DI, W, k = 20, 3, 4, 2, 2, 3, 3, 2
    Ca, Cb, Za, Zb = (g.normal(size=(n, d)) for _ in range(4))
    Ba, Bb = g.normal(size=(m, d)), g.normal(size=(m, d))
    N = n // m
    bf = [[0.0] * d for _ in range(N)]
    for i in range(N):
        for c in range(d):
            za = [Za[m * i + j][c] + Ba[j][c] for j in range(m)]
            mx = max(za); ea = [math.exp(z - mx) for z in za]
            bf[i][c] = sum(ea[j] * Ca[m * i + j][c] for j in range(m)) / sum(ea)
            if i >= 1:
                zb = [Zb[m * (i - 1) + j][c] + Bb[j][c] for j in range(m)]
                mx = max(zb); eb = [math.exp(z - mx) for z in zb]
                bf[i][c] += sum(eb[j] * Cb[m * (i - 1) + j][c] for j in range(m)) / sum(eb)
    comp = o.compress(Ca, Cb, Za, Zb, Ba, Bb, m)
    assert np.allclose(comp, np.array(bf), atol=1e-12)
    K = g.normal(size=(N, DI)); qi = g.normal(size=(HI, DI)); w = g.normal(size=HI)
    kv = g.normal(size=(n, d)); q = g.normal(size=(H, d)); sink = g.normal(size=H)
    p = n - 1
    V = min(N, (p + 1) // m)
    sc = []
    for i in range(V):
        t = 0.0
        for h in range(HI):
            t += w[h] * max(0.0, sum(qi[h][e] * K[i][e] for e in range(DI)))
        sc.append(t)
    chosen = sorted(sorted(range(V), key=lambda i: (-sc[i], i))[:k])
    rows = [list(comp[i]) for i in chosen] + [list(kv[t]) for t in range(max(0, p - W + 1), p + 1)]
    outs = []
    for h in range(H):
        ls = [sum(q[h][e] * r[e] for e in range(d)) for r in rows]
        mx = max(max(ls), sink[h])
        ex = [math.exp(v - mx) for v in ls]
        Z = math.exp(sink[h] - mx) + sum(ex)
        outs.append([sum(ex[j] * rows[j][e] for j in range(len(rows))) / Z for e in range(d)])
    idx, out, lse, s = o.csa_query(q, qi, w, comp, K, p, N, m, k, o.window_rows(kv, p, W), sink)
    assert np.allclose(s, sc, atol=1e-12)
    assert list(idx) == chosen
    assert np.allclose(out, np.array(outs), atol=1e-12)


# ------------------------------------------------------ MXFP4 query quantiser

_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_values(codes):
    codes = np.asarray(codes, np.int64)
    return np.where(codes & 8, -1.0, 1.0) * _E2M1[codes & 7]


def check_mxfp4_quantize_ties_and_saturation(o):
    """One block whose maximum is 6 (so the scale byte is 127 and the element
    values are the inputs themselves): the OCP rule rounds each tie to the
    even code and saturates beyond 6; the table is the E2M1 grid worked by
    hand."""
    x = np.zeros(32)
    x[:14] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 0.3, -0.1, 2.9, -1.74, 4.9]
    want = [6.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -4.0, 0.5, 0.0, 3.0, -1.5, 4.0]
    q, sc = o.mxfp4_quantize(x[None])
    assert sc.tolist() == [[127]]
    d = o.mxfp4_decode(q, sc)[0]
    assert d[:14].tolist() == want and np.all(d[14:] == 0)
    assert not np.signbit(d[10])  # -0.1 rounds to zero and keeps no sign
    # a block maximum of 7 still has floor(log2) = 2: scale byte 127, 7 saturates to 6
    x2 = np.zeros(32)
    x2[0], x2[1] = 7.0, -0.75
    q, sc = o.mxfp4_quantize(x2[None])
    assert sc.tolist() == [[127]] and o.mxfp4_decode(q, sc)[0][:2].tolist() == [6.0, -1.0]


def check_mxfp4_quantize_round_trip(o):
    """Blocks whose values are E2M1 values times 2^s with the block maximum 6
    or 4 are representable: quantising them gives back the same codes and
    the scale byte 127 + s."""
    g = _rng(41)
    for s_, top in ((-9, 7), (0, 6), (3, 7), (12, 6)):
        codes = g.integers(0, 16, (6, 128)).astype(np.int64)
        codes[codes == 8] = 0                      # -0 quantises to +0
        codes = np.where((codes & 7) > (top & 7), codes & 8 | (top & 7), codes)
        codes[:, 5::32] = top                      # each block holds its maximum
        x = _e2m1_values(codes) * 2.0 ** s_
        q, sc = o.mxfp4_quantize(x)
        assert np.all(sc == 127 + s_), (s_, top)  # max 6 or 4: floor(log2) = 2 + s
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        assert np.array_equal(q, packed), (s_, top)


def check_mxfp4_quantize_nearest(o):
    """Random blocks at several magnitudes: the block maximum lands in
    [4, 8) of the scale, and every element is a nearest point of the E2M1
    grid to x / scale (brute force over the 15 grid values), or 6 where it
    saturates."""
    g = _rng(42)
    grid = np.concatenate([-_E2M1[1:][::-1], _E2M1])
    for mag in (1e-3, 1.0, 37.0, 1e6):
        x = g.standard_normal((16, 64)) * mag
        q, sc = o.mxfp4_quantize(x)
        d = o.mxfp4_decode(q, sc)
        scale = np.repeat(np.exp2(sc.astype(np.float64) - 127.0), 32, axis=-1)
        y, v = x / scale, d / scale
        amax = np.abs(y).reshape(16, 2, 32).max(axis=-1)
        assert np.all((amax >= 4.0) & (amax < 8.0))
        best = np.abs(y[..., None] - grid).min(axis=-1)
        inside = np.abs(y) <= 6.0
        assert np.all(np.abs(y - v)[inside] <= best[inside] + 1e-12)
        assert np.all(np.abs(v[~inside]) == 6.0) and np.all(np.sign(v[~inside]) == np.sign(y[~inside]))


def check_indexer_fp4_query(o):
    """The FP4 QK path: a query whose head rows are already MXFP4 values
    scores exactly as the plain path; a general query scores as the plain
    path on its quantised values, which differ from it."""
    g = _rng(43)
    H, D, V = 4, 64, 40
    codes = g.integers(0, 16, (H, D)).astype(np.int64)
    codes[codes == 8] = 0
    codes[:, ::32] = 7
    q_rep = _e2m1_values(codes) * 2.0 ** -3
    k = g.standard_normal((V, D))
    w = g.uniform(0, 1, H)
    a = o.indexer_scores(q_rep, w, k, V, q_fp4=True)
    b = o.indexer_scores(q_rep, w, k, V)
    assert np.array_equal(a, b)
    q = g.standard_normal((H, D))
    f = o.indexer_scores(q, w, k, V, q_fp4=True)
    assert not np.allclose(f, o.indexer_scores(q, w, k, V), rtol=1e-3, atol=0)
    # each quantised element errs by less than 2 (saturation; half a grid step
    # below 6) block scales, a scale at most amax / 4, so by amax / 2 of its
    # head row; ReLU is 1-Lipschitz, which bounds the score change
    err = np.abs(f - o.indexer_scores(q, w, k, V))
    bound = np.abs(k).sum(axis=1) * np.sum(w * 0.5 * np.abs(q).max(axis=1))
    assert np.all(err <= bound + 1e-12)


ALL_CHECKS = [v for k_, v in sorted(globals().items()) if k_.startswith("check_")]
