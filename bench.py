"""Benchmark of the CSA/HCA attention hot path on one MI355X.

Default workload (the configuration the headline metric is quoted on): CSA
decode in the V4-Flash shape -- 32 sequences of 131072 tokens (32768
compressed entries of dim 512), 64 indexer heads x 128, top-k 512, 64 query
heads x 512, a 128-token window and a sink, bf16. One step is one decode token
per sequence through the whole path:
    csa_compress   (entry N-1 completes at this token: n is a multiple of m)
    indexer_score  (the dominant HBM stream)
    indexer_topk
    sparse_mqa_decode (split attention + combine)
Inputs are synthetic (seeded generator), resident in HBM before timing, and
rotated over several device replicas so that no step reads cache-resident
data from the previous one.

Other workloads: c5 (1M context, E4M3 indexer keys), c2x (c2 with MXFP4
indexer keys), c4 (HCA decode 1M), c3 (CSA prefill 64K), c6 (HCA prefill 64K),
c4f / c2f / c3f (c4 / c2 / c3 with the main KV rows in E4M3 + bf16 RoPE dims),
c2r (c2 with the query RMSNorm + RoPE prologue and the output inverse RoPE),
c2m (c2 with two query tokens per sequence and step).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload c2|c5|c4|c3|c2x|c6|c4f|c2f|c3f|c2r|c2m]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA decode tokens/sec + indexer/KV HBM GB/s at 128K–1M ctx; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2",
                    choices=["c2", "c5", "c4", "c3", "c2x", "c6", "c4f", "c2f", "c3f", "c2r", "c2m"])
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain 1 GiB device-to-device copies: the known-size reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def _src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_attention_06_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_file: str, src_files):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(p):
        return None
    vals = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != _src_hash(src_files):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    a = _args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_attention_06_amd as L
    from synth import gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                          "copies": 3}), flush=True)
        return
    if a.workload in ("c3", "c3f"):
        return bench_prefill(a, torch, L, gen, dev, gen.C3F if a.workload == "c3f" else gen.C3)
    if a.workload == "c6":
        return bench_hca_prefill(a, torch, L, gen, dev)
    cfg = {"c2": gen.C2, "c5": gen.C5, "c4": gen.C4, "c2x": gen.C2X, "c4f": gen.C4F, "c2f": gen.C2F,
           "c2r": gen.C2R, "c2m": gen.C2M}[a.workload]
    t0 = time.time()
    x = gen.gen_decode(cfg, with_compress=True)
    print(f"[bench] generated {cfg.name} inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def bf(v):
        return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(dev)

    def td(v):
        return torch.from_numpy(np.ascontiguousarray(v)).to(dev)

    B, N, H, D, W, m = cfg.B, cfg.N, cfg.H, cfg.D, cfg.W, cfg.m
    kvt = td if cfg.kv_dtype == "fp8" else bf  # mixed-precision rows travel as bytes
    rowb = D + 64 if cfg.kv_dtype == "fp8" else 2 * D  # bytes per main-KV row
    base = {"q": bf(x["q"]), "kv_comp": kvt(x["kv_comp"]), "kv_win": kvt(x["kv_win"])}
    Tq = cfg.Tq  # query tokens per sequence and step
    if cfg.kind == "csa_decode":
        base["q_idx"] = bf(x["q_idx"] if Tq > 1 else x["q_idx"][:, None])
        base["w"] = td(x["w"] if Tq > 1 else x["w"][:, None])
        if cfg.k_dtype == "fp8":
            base["k_idx"] = td(x["k_idx_codes"])
            base["k_scale"] = td(x["k_scale"])
        elif cfg.k_dtype == "mxfp4":
            base["k_idx"] = td(x["k_idx_codes"]).view(torch.float4_e2m1fn_x2)
            base["k_scale"] = td(x["k_scale"])
        else:
            base["k_idx"] = bf(x["k_idx"])
        for nm in ("Ca", "Cb", "Za", "Zb"):
            base[nm] = bf(x[nm])
    else:
        for nm in ("Ca", "Za"):
            base[nm] = bf(x[nm])
    shared = {"sink": td(x["sink"]), "Ba": td(x["Ba"]), "Bb": td(x["Bb"]),
              "q_pos": td(np.tile(np.arange(cfg.n - Tq, cfg.n, dtype=np.int32), (B, 1))),
              "n_comp": td(np.full((B,), N, np.int32)),
              "win_len": td(np.full((B,), min(W + Tq - 1, cfg.n), np.int32))}
    if cfg.qk_rope:
        shared["q_gamma"] = td(x["q_gamma"])
        shared["pos"] = td(np.full((B,), cfg.n - 1, np.int32))
    att_scale = 1.0 / math.sqrt(D) if cfg.qk_rope else 1.0
    reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(a.replicas - 1)]
    out = torch.empty(((B, Tq, H, D) if Tq > 1 else (B, H, D)), dtype=torch.bfloat16, device=dev)
    qn = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    if cfg.kind == "csa_decode":
        k = cfg.top_k
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=dev)
        idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
        ws_t = torch.empty(max(1, L.indexer_topk_workspace_bytes(B, Tq, N, k)), dtype=torch.uint8, device=dev)
        ws_a = torch.empty(max(1, L.sparse_mqa_decode_multi_workspace_bytes(B, Tq, H, D, k, W)), dtype=torch.uint8,
                           device=dev)
    else:
        ws_a = torch.empty(max(1, L.hca_dense_mqa_workspace_bytes(B, H, D, N, W)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def rec(ev, i):
        if ev is not None:
            ev[i].record(stream)

    def step(r, ev=None):
        rec(ev, 0)
        q_att = r["q"]
        if cfg.qk_rope:  # prologue: RMSNorm + RoPE of the raw queries at their position
            L.qk_norm_rope(r["q"], qn, shared["pos"], shared["q_gamma"], norm=True, rope=True, stream=s)
            q_att = qn
        if cfg.kind == "csa_decode":
            # the completed block's entry and the indexer scan, one call (one launch for bf16 keys)
            L.csa_compress_indexer_score(r["Ca"], r["Cb"], r["Za"], r["Zb"], shared["Ba"], shared["Bb"], r["kv_comp"],
                                         r["q_idx"], r["w"], r["k_idx"], r.get("k_scale"), shared["q_pos"],
                                         shared["n_comp"], scores, m_c=m, m=m, tok_begin=cfg.n - 2 * m,
                                         blk_begin=N - 1, blk_end=N, stream=s)
            rec(ev, 1)
            rec(ev, 2)
            L.indexer_topk(scores, shared["q_pos"], shared["n_comp"], idx, m=m, ws=ws_t, stream=s)
            rec(ev, 3)
            if Tq > 1:
                L.sparse_mqa_decode_multi(q_att, r["kv_comp"], idx, r["kv_win"], shared["win_len"], shared["sink"],
                                          out, scale=att_scale, ws=ws_a, stream=s)
            else:
                L.sparse_mqa_decode(q_att, r["kv_comp"], idx.view(B, k), r["kv_win"], shared["win_len"],
                                    shared["sink"], out, scale=att_scale, ws=ws_a, stream=s)
            if cfg.qk_rope:  # epilogue: the output's rotated dims turned back
                L.qk_norm_rope(out, out, shared["pos"], inverse=True, stream=s)
        else:
            # HCA: the token completes block N-1 (m' divides n): one branch, no overlap
            L.csa_compress(r["Ca"], None, r["Za"], None, shared["Ba"], None, r["kv_comp"], m=m,
                           tok_begin=cfg.n - m, blk_begin=N - 1, blk_end=N, overlap=False, stream=s)
            rec(ev, 1)
            rec(ev, 2)
            rec(ev, 3)
            L.hca_dense_mqa(r["q"], r["kv_comp"], shared["n_comp"], shared["q_pos"].view(B), r["kv_win"],
                            shared["win_len"], shared["sink"], out, m=m, ws=ws_a, stream=s)

    for i in range(a.warmup):
        step(reps[i % len(reps)])
    torch.cuda.synchronize()
    # (1) the headline: K plain steps between two events
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record(stream)
    t_wall = time.perf_counter()
    for i in range(a.steps):
        step(reps[i % len(reps)])
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = e_start.elapsed_time(e_end) / a.steps
    # (2) the same K steps with an event at every phase boundary:
    # [0] compress [1] indexer scan [2] top-k [3] attention [next 0]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    e_fin = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for i in range(a.steps):
        step(reps[i % len(reps)], evs[i])
    e_fin.record(stream)
    torch.cuda.synchronize()
    nxt = [evs[i + 1][0] for i in range(a.steps - 1)] + [e_fin]
    ph = np.array([[evs[i][0].elapsed_time(evs[i][1]), evs[i][1].elapsed_time(evs[i][2]),
                    evs[i][2].elapsed_time(evs[i][3]), evs[i][3].elapsed_time(nxt[i])] for i in range(a.steps)])
    ph_mean = ph.mean(axis=0)
    attn_avg = float(ph_mean[3])
    # (3) the dominant kernel alone, K back-to-back launches between two events
    # on the stream it runs on: its average launch duration for the roofline
    e3a, e3b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e3a.record(stream)
    for i in range(a.steps):
        r = reps[i % len(reps)]
        if cfg.kind == "csa_decode":
            L.indexer_score(r["q_idx"], r["w"], r["k_idx"], r.get("k_scale"), shared["q_pos"], shared["n_comp"],
                            scores, m=m, stream=s)
        else:
            L.hca_dense_mqa(r["q"], r["kv_comp"], shared["n_comp"], shared["q_pos"].view(B), r["kv_win"],
                            shared["win_len"], shared["sink"], out, m=m, ws=ws_a, stream=s)
    e3b.record(stream)
    torch.cuda.synchronize()
    kern_avg = e3a.elapsed_time(e3b) / a.steps
    scan_avg = kern_avg

    tokens_per_s = B * Tq / (ms_step * 1e-3)
    res = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
    }
    if cfg.kind == "csa_decode":
        kbytes = {"fp8": N * (cfg.D_I + 4), "mxfp4": N * (cfg.D_I // 2 + cfg.D_I // 32)}.get(cfg.k_dtype, N * cfg.D_I * 2)
        # keys (+scales) once per sequence (what the method needs), q_idx and w per query
        scan_bytes = B * (kbytes + Tq * (cfg.H_I * cfg.D_I * 2 + cfg.H_I * 4))
        step_bytes = B * (kbytes + Tq * (cfg.H_I * cfg.D_I * 2 + cfg.H_I * 4 + (k + W) * rowb + H * D * 2 * 2 + k * 4))
        res["config"] = {"workload": cfg.name, "batch": B, "context_tokens": cfg.n, "compressed_entries": N,
                         "m": m, "top_k": k, "indexer_heads": cfg.H_I, "indexer_dim": cfg.D_I,
                         "heads": H, "head_dim": D, "window": W, "indexer_key_dtype": cfg.k_dtype,
                         "kv_dtype": cfg.kv_dtype, "qk_norm_rope": cfg.qk_rope, "query_tokens_per_sequence": Tq}
        # the scan alone (the step's launch also carries the compression: <.., 1|4>)
        kname = {"fp8": "idx_scan_lp_kernel<2, 0> (E4M3 keys)", "mxfp4": "idx_scan_lp_kernel<3, 0> (MXFP4 keys)"}.get(
            cfg.k_dtype, "idx_scan_bf16_kernel<2, 0> (two query rows per workgroup)" if Tq % 2 == 0
            else "idx_scan_bf16_kernel<1, 0>")
        res["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": round(scan_bytes / (scan_avg * 1e-3) / 1e9, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(scan_bytes / (scan_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "traffic": _traffic(f"idx_scan_{a.workload}_traffic.txt", ["indexer.hip", "common.h"]),
                           "algorithmic_bytes_per_launch": scan_bytes, "avg_launch_ms": round(scan_avg, 4)}
        res["phases_ms"] = {"compress_and_indexer_scan": round(float(ph_mean[0] + ph_mean[1]), 4),
                            "topk": round(float(ph_mean[2]), 4), "attention": round(attn_avg, 4)}
        res["step_hbm_gbs"] = round(step_bytes / (ms_step * 1e-3) / 1e9, 1)
        res["indexer_kv_hbm_gbs"] = res["roofline"]["achieved"]
    else:
        hbytes = B * ((N + W) * rowb + H * D * 2 * 2)
        res["config"] = {"workload": cfg.name, "batch": B, "context_tokens": cfg.n, "compressed_entries": N,
                         "m": m, "heads": H, "head_dim": D, "window": W, "kv_dtype": cfg.kv_dtype}
        res["phases_ms"] = {"compress": round(float(ph_mean[0]), 4), "attention": round(attn_avg, 4)}
        res["roofline"] = {"bound": "hbm", "kernel": "hca_dense_mqa (attn_bf16_kernel<1, %s> HCA splits + combine)"
                           % ("true" if cfg.kv_dtype == "fp8" else "false"),
                           "achieved": round(hbytes / (kern_avg * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(hbytes / (kern_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "traffic": None, "algorithmic_bytes_per_launch": hbytes, "avg_launch_ms": round(kern_avg, 4)}
    res["wall_s_timed"] = round(wall, 3)

    if not a.no_cpu:
        res["cpu_baseline"] = cpu_baseline(cfg, x, a.cpu_seconds)
    print(json.dumps(res), flush=True)


def prefill_flops(cfg, pos):
    """Algorithmic FLOPs of a prefill chunk: indexer over visible pairs,
    sparse MQA over min(k, V) selected rows and the window rows."""
    V = np.minimum(cfg.N, (pos.astype(np.int64) + 1) // cfg.m)
    win = np.minimum(cfg.W, pos.astype(np.int64) + 1)
    idx = float(V.sum()) * cfg.H_I * cfg.D_I * 2
    mqa = float((np.minimum(cfg.top_k, V) + win).sum()) * cfg.H * cfg.D * 4
    return idx, mqa


def bench_prefill(a, torch, L, gen, dev, cfg):
    """CSA prefill of one 65536-token sequence: compression of all tokens, then
    16 chunks of 4096 queries through scores, top-k and sparse MQA (main KV
    rows in bf16, or E4M3 + bf16 RoPE dims)."""
    t0 = time.time()
    tok = gen.gen_prefill_tokens(cfg)
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(dev)
    td = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    N, m, D, H, k, W = cfg.N, cfg.m, cfg.D, cfg.H, cfg.top_k, cfg.W
    Ca, Cb, Za, Zb = (bf(tok[nm][None]) for nm in ("Ca", "Cb", "Za", "Zb"))
    Ba, Bb, sink = td(tok["Ba"]), td(tok["Bb"]), td(tok["sink"])
    fp8 = cfg.kv_dtype == "fp8"
    kv_tok, k_idx = (td if fp8 else bf)(tok["kv_tok"]), bf(tok["k_idx"][None])
    comp = (torch.empty((1, N, D + 64), dtype=torch.uint8, device=dev) if fp8
            else torch.empty((1, N, D), dtype=torch.bfloat16, device=dev))
    nch = gen.num_chunks(cfg)
    chunks = []
    for c in range(nch):
        qs = gen.gen_prefill_queries(cfg, c)
        chunks.append({"q": bf(qs["q"]), "q_idx": bf(qs["q_idx"][None]), "w": td(qs["w"][None]),
                       "q_pos": td(qs["q_pos"][None]), "pos_np": qs["q_pos"]})
    print(f"[bench] generated {cfg.name} inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    T = gen.QCHUNK
    n_comp = td(np.array([N], np.int32))
    scores = torch.empty((1, T, N), dtype=torch.float32, device=dev)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=dev)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    ws_t = torch.empty(max(1, L.indexer_topk_workspace_bytes(1, T, N, k)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def run(ev=None):
        if ev is not None: ev[0].record(stream)
        L.csa_compress(Ca, Cb, Za, Zb, Ba, Bb, comp, m=m, stream=s)
        if ev is not None: ev[1].record(stream)
        for c, ch in enumerate(chunks):
            L.indexer_score(ch["q_idx"], ch["w"], k_idx, None, ch["q_pos"], n_comp, scores, m=m, stream=s)
            if ev is not None: ev[2 + 3 * c].record(stream)
            L.indexer_topk(scores, ch["q_pos"], n_comp, idx, m=m, ws=ws_t, stream=s)
            if ev is not None: ev[3 + 3 * c].record(stream)
            L.sparse_mqa_prefill(ch["q"], comp[0], idx[0], kv_tok, ch["q_pos"][0], sink, out, W=W, stream=s)
            if ev is not None: ev[4 + 3 * c].record(stream)

    for _ in range(max(1, a.warmup)):
        run()
    torch.cuda.synchronize()
    steps = max(1, min(a.steps, 5))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 + 3 * nch)]
    run(ev)
    torch.cuda.synchronize()
    comp_ms = ev[0].elapsed_time(ev[1])
    prev = [ev[1]] + [ev[4 + 3 * c] for c in range(nch - 1)]
    idx_ms = [prev[c].elapsed_time(ev[2 + 3 * c]) for c in range(nch)]
    topk_ms = [ev[2 + 3 * c].elapsed_time(ev[3 + 3 * c]) for c in range(nch)]
    attn_ms = [ev[3 + 3 * c].elapsed_time(ev[4 + 3 * c]) for c in range(nch)]
    fl = [prefill_flops(cfg, ch["pos_np"]) for ch in chunks]
    idx_fl, mqa_fl = sum(f[0] for f in fl), sum(f[1] for f in fl)
    total_fl = idx_fl + mqa_fl
    idx_tfs = idx_fl / (sum(idx_ms) * 1e-3) / 1e12
    mqa_tfs = mqa_fl / (sum(attn_ms) * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(cfg.n / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": max(1, a.warmup), "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.n, "query_chunk": T, "compressed_entries": N, "m": m,
                   "top_k": k, "indexer_heads": cfg.H_I, "indexer_dim": cfg.D_I, "heads": H, "head_dim": D,
                   "window": W, "kv_dtype": cfg.kv_dtype},
        "prefill_tflops": round(total_fl / (ms * 1e-3) / 1e12, 2),
        "algorithmic_tflop": round(total_fl / 1e12, 3),
        "roofline": {"bound": "mfma", "kernel": "attn_prs_kernel<2, %s> (sparse prefill)" % ("true" if fp8 else "false"),
                     "achieved": round(mqa_tfs, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(mqa_tfs / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_all_launches": mqa_fl,
                     "avg_launch_ms": round(float(np.mean(attn_ms)), 4)},
        "roofline_indexer": {"bound": "mfma", "kernel": "idx_prefill_kernel", "achieved": round(idx_tfs, 1),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(idx_tfs / BF16_PEAK_TFLOPS, 4),
                             "algorithmic_flops_all_launches": idx_fl, "avg_launch_ms": round(float(np.mean(idx_ms)), 4)},
        "phases_ms": {"compress": round(comp_ms, 4), "indexer_total": round(sum(idx_ms), 4),
                      "topk_total": round(sum(topk_ms), 4), "attention_total": round(sum(attn_ms), 4)},
    }
    if not a.no_cpu:
        res["cpu_baseline"] = cpu_prefill_baseline(cfg, tok, a.cpu_seconds)
    print(json.dumps(res), flush=True)


def hca_prefill_rows(cfg, pos):
    """Rows each query attends in HCA prefill: V(p) entries plus its window."""
    pos = pos.astype(np.int64)
    return np.minimum(cfg.N, (pos + 1) // cfg.m) + np.minimum(cfg.W, pos + 1)


def bench_hca_prefill(a, torch, L, gen, dev):
    """HCA prefill of one 65536-token sequence: single-branch compression of
    all tokens at m' = 128, then 16 chunks of 4096 queries through hca_prefill
    (every visible entry plus the window and the sink)."""
    cfg = gen.C6
    t0 = time.time()
    tok = gen.gen_prefill_tokens(cfg)
    bf = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(dev)
    td = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    N, m, D, H, W = cfg.N, cfg.m, cfg.D, cfg.H, cfg.W
    Ca, Za, Ba, sink = bf(tok["Ca"][None]), bf(tok["Za"][None]), td(tok["Ba"]), td(tok["sink"])
    kv_tok = bf(tok["kv_tok"])
    comp = torch.empty((1, N, D), dtype=torch.bfloat16, device=dev)
    nch = gen.num_chunks(cfg)
    chunks = []
    for c in range(nch):
        qs = gen.gen_prefill_queries(cfg, c)
        chunks.append({"q": bf(qs["q"]), "q_pos": td(qs["q_pos"]), "pos_np": qs["q_pos"]})
    print(f"[bench] generated {cfg.name} inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    T = gen.QCHUNK
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def run(ev=None):
        if ev is not None: ev[0].record(stream)
        L.csa_compress(Ca, None, Za, None, Ba, None, comp, m=m, overlap=False, stream=s)
        if ev is not None: ev[1].record(stream)
        for c, ch in enumerate(chunks):
            L.hca_prefill(ch["q"], comp[0], kv_tok, ch["q_pos"], sink, out, m=m, W=W, stream=s)
            if ev is not None: ev[2 + c].record(stream)

    for _ in range(max(1, a.warmup)):
        run()
    torch.cuda.synchronize()
    steps = max(1, min(a.steps, 5))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 + nch)]
    run(ev)
    torch.cuda.synchronize()
    comp_ms = ev[0].elapsed_time(ev[1])
    attn_ms = [ev[1 + c].elapsed_time(ev[2 + c]) for c in range(nch)]
    rows = [float(hca_prefill_rows(cfg, ch["pos_np"]).sum()) for ch in chunks]
    mqa_fl = sum(rows) * H * D * 4
    mqa_tfs = mqa_fl / (sum(attn_ms) * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(cfg.n / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": max(1, a.warmup), "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.n, "query_chunk": T, "compressed_entries": N, "m": m,
                   "heads": H, "head_dim": D, "window": W},
        "prefill_tflops": round(mqa_fl / (ms * 1e-3) / 1e12, 2),
        "algorithmic_tflop": round(mqa_fl / 1e12, 3),
        "roofline": {"bound": "mfma", "kernel": "attn_prs_kernel<3> (HCA prefill)", "achieved": round(mqa_tfs, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(mqa_tfs / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_all_launches": mqa_fl,
                     "avg_launch_ms": round(float(np.mean(attn_ms)), 4)},
        "phases_ms": {"compress": round(comp_ms, 4), "attention_total": round(sum(attn_ms), 4)},
    }
    if not a.no_cpu:
        res["cpu_baseline"] = cpu_hca_prefill_baseline(cfg, tok, a.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_hca_prefill_baseline(cfg, tok, budget_s: float):
    """The oracle on the host: single-branch compression of the whole
    sequence, then queries of the last chunk one by one until the budget is
    spent; extrapolated to all queries by attended-row counts."""
    import oracle
    from synth import gen
    t0 = time.perf_counter()
    comp = oracle.compress(tok["Ca"], None, tok["Za"], None, tok["Ba"], None, cfg.m, overlap=False)
    t_comp = time.perf_counter() - t0
    qs = gen.gen_prefill_queries(cfg, gen.num_chunks(cfg) - 1)
    t1 = time.perf_counter()
    done, rows = 0, 0.0
    while done < len(qs["q_pos"]) and (done == 0 or time.perf_counter() - t1 < budget_s):
        i = len(qs["q_pos"]) - 1 - done
        p = int(qs["q_pos"][i])
        oracle.hca_query(qs["q"][i], comp, p, cfg.N, cfg.m, oracle.window_rows(tok["kv_tok"], p, cfg.W), tok["sink"])
        rows += float(hca_prefill_rows(cfg, np.array([p]))[0])
        done += 1
    t_q = time.perf_counter() - t1
    all_rows = float(hca_prefill_rows(cfg, gen.query_positions(cfg)).sum())
    est = t_comp + t_q * all_rows / max(rows, 1.0)
    return {"value": round(cfg.n / est, 3), "unit": "tokens/s", "cores": _threads(), "kind": "oracle",
            "sample": f"compression of all {cfg.n} tokens ({t_comp:.1f}s) + {done} queries of the last chunk "
                      f"({t_q:.1f}s), extrapolated to all queries by attended-row counts"}


def cpu_prefill_baseline(cfg, tok, budget_s: float):
    """The oracle on the host: compression of the whole sequence is timed,
    then queries of the last chunk one by one until the budget is spent; the
    rate is extrapolated to all queries by visible-pair counts."""
    import oracle
    from synth import gen
    t0 = time.perf_counter()
    comp = oracle.compress(tok["Ca"], tok["Cb"], tok["Za"], tok["Zb"], tok["Ba"], tok["Bb"], cfg.m)
    kv_tok = tok["kv_tok"]
    if cfg.kv_dtype == "fp8":  # the entries as stored, and the token rows' values
        comp = oracle.kv_fp8_decode(gen.kv_fp8_rows(comp), cfg.D)
        kv_tok = oracle.kv_fp8_decode(kv_tok, cfg.D)
    t_comp = time.perf_counter() - t0
    qs = gen.gen_prefill_queries(cfg, gen.num_chunks(cfg) - 1)
    t1 = time.perf_counter()
    done, pairs = 0, 0
    while done < len(qs["q_pos"]) and (done == 0 or time.perf_counter() - t1 < budget_s):
        i = len(qs["q_pos"]) - 1 - done
        p = int(qs["q_pos"][i])
        oracle.csa_query(qs["q"][i], qs["q_idx"][i], qs["w"][i], comp, tok["k_idx"], p, cfg.N, cfg.m, cfg.top_k,
                         oracle.window_rows(kv_tok, p, cfg.W), tok["sink"])
        pairs += min(cfg.N, (p + 1) // cfg.m)
        done += 1
    t_q = time.perf_counter() - t1
    all_pairs = float(np.minimum(cfg.N, (np.arange(cfg.n, dtype=np.int64) + 1) // cfg.m).sum())
    est = t_comp + t_q * all_pairs / max(pairs, 1)
    return {"value": round(cfg.n / est, 3), "unit": "tokens/s", "cores": _threads(), "kind": "oracle",
            "sample": f"compression of all {cfg.n} tokens ({t_comp:.1f}s) + {done} queries of the last chunk "
                      f"({t_q:.1f}s), extrapolated to all queries by visible-pair counts"}


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(cfg, x, budget_s: float):
    """The float64 oracle on the host cores, on whole sequences of the same
    workload, cycling over the step's sequences until the time budget is
    used (at least one sequence)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    from synth import gen
    fp8 = cfg.kv_dtype == "fp8"
    kvd = (lambda r: oracle.kv_fp8_decode(r, cfg.D)) if fp8 else (lambda r: np.asarray(r, np.float64))
    stored = (lambda e: oracle.kv_fp8_decode(gen.kv_fp8_rows(e), cfg.D)) if fp8 else (lambda e: e)
    done = 0
    t0 = time.perf_counter()
    m = cfg.m
    while done == 0 or time.perf_counter() - t0 < budget_s:
        b = done % cfg.B
        if cfg.kind == "csa_decode":
            ent = oracle.compress(x["Ca"][b], x["Cb"][b], x["Za"][b], x["Zb"][b], x["Ba"], x["Bb"], m,
                                  blocks=range(1, 2))[0]
            comp = kvd(x["kv_comp"][b])
            comp[cfg.N - 1] = stored(ent)
            if cfg.k_dtype == "fp8":
                keys, sc = oracle.e4m3_decode(x["k_idx_codes"][b]), x["k_scale"][b]
            elif cfg.k_dtype == "mxfp4":
                keys, sc = oracle.mxfp4_decode(x["k_idx_codes"][b], x["k_scale"][b]), None
            else:
                keys, sc = x["k_idx"][b], None
            win = kvd(x["kv_win"][b])
            for t in range(cfg.Tq):  # query token t at position n - Tq + t, its window ending at its token
                p = cfg.n - cfg.Tq + t
                q, qi_, w_ = ((x["q"][b][t], x["q_idx"][b][t], x["w"][b][t]) if cfg.Tq > 1
                              else (x["q"][b], x["q_idx"][b], x["w"][b]))
                tau = 1.0
                if cfg.qk_rope:
                    q = oracle.rope_rotate(oracle.rms_norm(q[None], x["q_gamma"], 1e-6), [p])[0]
                    tau = 1.0 / math.sqrt(cfg.D)
                hi = len(win) - cfg.Tq + t
                _, o, _, _ = oracle.csa_query(q, qi_, w_, comp, keys, p, cfg.N, m, cfg.top_k,
                                              win[max(0, hi - cfg.W + 1):hi + 1], x["sink"], k_scale=sc, tau=tau)
                if cfg.qk_rope:
                    oracle.rope_rotate(o[None], [p], inverse=True)
        else:
            ent = oracle.compress(x["Ca"][b], None, x["Za"][b], None, x["Ba"], None, m, overlap=False)[0]
            comp = kvd(x["kv_comp"][b])
            comp[cfg.N - 1] = stored(ent)
            oracle.hca_query(x["q"][b], comp, cfg.n - 1, cfg.N, m, kvd(x["kv_win"][b]), x["sink"])
        done += 1
    dt = time.perf_counter() - t0
    return {"value": round(done * cfg.Tq / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} sequences ({cfg.Tq} query token(s) each; the step's {cfg.B} taken in turn, "
                      f"{done / cfg.B:.1f} steps) of a decode step ({cfg.name}), float64 NumPy, {dt:.1f}s"}


if __name__ == "__main__":
    main()
