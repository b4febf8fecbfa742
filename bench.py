"""Benchmark of the CSA/HCA attention hot path on one MI355X.

Default workload (the configuration the headline metric is quoted on): CSA
decode in the V4-Flash shape -- 32 sequences of 131072 tokens (32768
compressed entries of dim 512), 64 indexer heads x 128, top-k 512, 64 query
heads x 512, a 128-token window and a sink, bf16. One step is one decode token
per sequence through the whole path:
    csa_compress   (entry N-1 completes at this token: n is a multiple of m)
    indexer_score  (the dominant HBM stream; one launch with the compression)
    top-k, sparse MQA and the merge of its splits (three launches)
as one csa_decode_step call. Inputs are synthetic (seeded generator),
resident in HBM before timing, and rotated over several device replicas so
that no step reads cache-resident data from the previous one. The default
line also carries c5, c4, c3 and c2q (below), each timed the same way, under
"workloads".

Other workloads: c5 (1M context, E4M3 indexer keys), c2x (c2 with MXFP4
indexer keys), c4 (HCA decode 1M), c3 (CSA prefill 64K), c6 (HCA prefill 64K),
c4f / c2f / c3f (c4 / c2 / c3 with the main KV rows in E4M3 + bf16 RoPE dims),
c2r (c2 with the query RMSNorm + RoPE prologue and the output inverse RoPE),
c2m (c2 with two query tokens per sequence and step), c2q (c2x with the
indexer query quantised to MXFP4 in the call: FP4 x FP4 on the scaled MFMA).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
                       [--workload c2|c5|c4|c3|c2x|c6|c4f|c2f|c3f|c2r|c2m|c2q]
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
                    choices=["c2", "c5", "c4", "c3", "c2x", "c6", "c4f", "c2f", "c3f", "c2r", "c2m", "c2q"])
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--extra-cpu-seconds", type=float, default=4.0,
                    help="budget of the CPU baseline of each secondary workload")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="with the default workload, skip the secondary workloads (c5, c4, c3, c2q)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain 1 GiB device-to-device copies: the known-size reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


EXTRAS = ("c5", "c4", "c3", "c2q")  # secondary workloads carried by the default line


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


def _roofline(bound, kernel, work, ms, peak, unit, traffic=None, copy_gbs=None):
    """achieved = algorithmic work per launch / average launch duration."""
    ach = work / (ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
    r = {"bound": bound, "kernel": kernel, "achieved": round(ach, 1), "peak": peak, "unit": unit,
         "frac": round(ach / peak, 4), "traffic": traffic,
         ("algorithmic_bytes_per_launch" if unit == "GB/s" else "algorithmic_flops_per_launch"): work,
         "avg_launch_ms": round(ms, 4)}
    if copy_gbs and unit == "GB/s":
        r["frac_of_copy"] = round(ach / copy_gbs, 4)  # against the on-box device copy rate
    return r


def measure_copy(torch, dev):
    """On-box rate of a plain 1 GiB device-to-device copy (read + write bytes
    per second): the practical ceiling the HBM fractions are also quoted against."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def _graph_loop_ms(torch, fn, steps):
    """Average duration of fn(i), i < steps, launched back to back: captured
    in one HIP graph so no host work sits between the launches, replayed once
    between two events on the current stream."""
    side = torch.cuda.Stream()  # default priority, as every stream here
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    return ms


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
    copy_gbs = measure_copy(torch, dev)
    res = run_workload(a.workload, a, torch, L, gen, dev, a.steps, a.warmup,
                       None if a.no_cpu else a.cpu_seconds, copy_gbs)
    res["copy_gbs"] = copy_gbs
    if a.workload == "c2" and not a.no_extras:
        # the other headline configurations, each timed the same way (fewer
        # steps, a shorter CPU baseline), under "workloads"
        res["workloads"] = {}
        for w in EXTRAS:
            torch.cuda.empty_cache()
            r = run_workload(w, a, torch, L, gen, dev, min(a.steps, 20), min(a.warmup, 3),
                             None if a.no_cpu else a.extra_cpu_seconds, copy_gbs)
            res["workloads"][w] = {k: v for k, v in r.items() if k not in (
                "metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "dtype", "data")}
    print(json.dumps(res), flush=True)


def run_workload(w, a, torch, L, gen, dev, steps, warmup, cpu_s, copy_gbs):
    if w in ("c3", "c3f"):
        return bench_prefill(a, torch, L, gen, dev, gen.C3F if w == "c3f" else gen.C3, steps, warmup, cpu_s, w)
    if w == "c6":
        return bench_hca_prefill(a, torch, L, gen, dev, steps, warmup, cpu_s)
    cfg = {"c2": gen.C2, "c5": gen.C5, "c4": gen.C4, "c2x": gen.C2X, "c4f": gen.C4F, "c2f": gen.C2F,
           "c2r": gen.C2R, "c2m": gen.C2M, "c2q": gen.C2Q}[w]
    return bench_decode(a, torch, L, gen, dev, cfg, steps, warmup, cpu_s, copy_gbs, w)


def _base(steps, warmup):
    return {"metric": METRIC, "n_gpus": 1, "steps": steps, "warmup": warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}


def bench_decode(a, torch, L, gen, dev, cfg, steps, warmup, cpu_s, copy_gbs, wname):
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
    att_scale = 1.0 / math.sqrt(D) if cfg.qk_rope else 1.0
    reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(a.replicas - 1)]
    out = torch.empty(((B, Tq, H, D) if Tq > 1 else (B, H, D)), dtype=torch.bfloat16, device=dev)
    if cfg.kind == "csa_decode":
        k = cfg.top_k
        idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
        # scores, digit histograms, top-k and attention scratch; zero-filled
        # once, as the step leaves it (its histograms cleared after use)
        wsb = (L.csa_decode_step_qk_workspace_bytes if cfg.qk_rope else L.csa_decode_step_workspace_bytes)
        ws_t = torch.zeros(wsb(B, Tq, N, k, H, D, W), dtype=torch.uint8, device=dev)
        ws_a = None
    else:
        ws_a = torch.zeros(max(1, L.hca_decode_step_workspace_bytes(B, H, D, N, W)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream

    def step(r, pre=None):
        if pre is not None:
            pre.record(stream)
        if cfg.kind == "csa_decode" and cfg.qk_rope:
            # raw queries: the step applies RMSNorm + RoPE before the attention
            # and the inverse rotation to its output
            L.csa_decode_step_qk(r["Ca"], r["Cb"], r["Za"], r["Zb"], shared["Ba"], shared["Bb"], r["q_idx"], r["w"],
                                 r["k_idx"], r.get("k_scale"), shared["q_pos"], shared["n_comp"],
                                 r["q"].view(B, 1, H, D), r["kv_comp"], r["kv_win"], shared["win_len"],
                                 shared["sink"], idx, out.view(B, 1, H, D), q_gamma=shared["q_gamma"], m_c=m, m=m,
                                 tok_begin=cfg.n - 2 * m, blk_begin=N - 1, blk_end=N, scale=att_scale, ws=ws_t,
                                 stream=s)
        elif cfg.kind == "csa_decode":
            # the whole step in one call: the completed block's entry with the
            # indexer scan, then top-k, attention and split merge
            L.csa_decode_step(r["Ca"], r["Cb"], r["Za"], r["Zb"], shared["Ba"], shared["Bb"], r["q_idx"], r["w"],
                              r["k_idx"], r.get("k_scale"), shared["q_pos"], shared["n_comp"],
                              r["q"] if Tq > 1 else r["q"].view(B, 1, H, D), r["kv_comp"], r["kv_win"],
                              shared["win_len"], shared["sink"], idx, out if Tq > 1 else out.view(B, 1, H, D),
                              m_c=m, m=m, tok_begin=cfg.n - 2 * m, blk_begin=N - 1, blk_end=N, scale=att_scale,
                              ws=ws_t, q_fp4=cfg.q_fp4, stream=s)
        else:
            # HCA: the token completes block N-1 (m' divides n): its single-
            # branch entry, the dense attention and the split merge in one call
            L.hca_decode_step(r["Ca"], r["Za"], shared["Ba"], r["q"], r["kv_comp"], shared["n_comp"],
                              shared["q_pos"].view(B), r["kv_win"], shared["win_len"], shared["sink"], out, m_c=m, m=m,
                              tok_begin=cfg.n - m, blk_begin=N - 1, blk_end=N, ws=ws_a, stream=s)

    for i in range(warmup):
        step(reps[i % len(reps)])
    torch.cuda.synchronize()
    # (1) the headline: K plain steps between two events; then four more
    # such runs, for the median over runs
    runs = []
    for rep in range(5):
        e_start = torch.cuda.Event(enable_timing=True)
        e_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e_start.record(stream)
        t_wall = time.perf_counter()
        for i in range(steps):
            step(reps[i % len(reps)])
        e_end.record(stream)
        torch.cuda.synchronize()
        if rep == 0:
            wall = time.perf_counter() - t_wall
        runs.append(e_start.elapsed_time(e_end) / steps)
    ms_step = runs[0]
    # (2) the same K steps with the library's phase events (csa_trace_phases):
    # [0] call start [1] scan launched [2] top-k / fused tail [3] attention
    # kernel [4] call end, plus an event before each step
    pre = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for e in pre + [e for es in evs for e in es]:
        e.record(stream)  # creates the event, so its handle exists
    torch.cuda.synchronize()
    for i in range(steps):
        L.trace_phases(evs[i])
        step(reps[i % len(reps)], pre[i])
    L.trace_phases(None)
    pre[steps].record(stream)
    torch.cuda.synchronize()
    ph = np.array([[pre[i].elapsed_time(evs[i][0])] + [evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)]
                   + [evs[i][4].elapsed_time(pre[i + 1])] for i in range(steps)])
    ph_mean = ph.mean(axis=0)

    res = _base(steps, warmup)
    res.update({"value": round(B * Tq / (ms_step * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms_step, 4),
                "ms_per_step_median_of_5_runs": round(float(np.median(runs)), 4)})
    if cfg.kind == "csa_decode":
        kbytes = {"fp8": N * (cfg.D_I + 4), "mxfp4": N * (cfg.D_I // 2 + cfg.D_I // 32)}.get(cfg.k_dtype, N * cfg.D_I * 2)
        # the scan launch: keys (+scales) once per sequence, q_idx and w per
        # query, the scores it writes, and the compression it carries (the
        # a-branch block and the overlapping b-branch block, four tensors of m
        # rows, in; the entry out)
        comp_bytes = B * (4 * m * D * 2 + rowb)
        scan_bytes = B * (kbytes + Tq * (cfg.H_I * cfg.D_I * 2 + cfg.H_I * 4 + N * 4)) + comp_bytes
        step_bytes = B * (kbytes + Tq * (cfg.H_I * cfg.D_I * 2 + cfg.H_I * 4 + (k + W) * rowb + H * D * 2 * 2 + k * 4))
        res["config"] = {"workload": cfg.name, "batch": B, "context_tokens": cfg.n, "compressed_entries": N,
                         "m": m, "top_k": k, "indexer_heads": cfg.H_I, "indexer_dim": cfg.D_I,
                         "heads": H, "head_dim": D, "window": W, "indexer_key_dtype": cfg.k_dtype,
                         "kv_dtype": cfg.kv_dtype, "qk_norm_rope": cfg.qk_rope, "query_tokens_per_sequence": Tq,
                         "indexer_query": "mxfp4 (quantised in the call)" if cfg.q_fp4 else "bf16"}
        kname = {"fp8": "idx_scan_reg_kernel<2, false, 1> (E4M3 keys, with the entry's compression)",
                 "mxfp4": "idx_scan_reg_kernel<3, true, 1> (MXFP4 keys and the FP4-quantised query on the scaled "
                          "FP4 MFMA, with the entry's compression)" if cfg.q_fp4 else
                          "idx_scan_reg_kernel<3, false, 1> (MXFP4 keys, with the entry's compression)"}.get(
            cfg.k_dtype, "idx_scan_bf16_kernel<2, 1> (two query rows per workgroup, with the entry's compression)"
            if Tq % 2 == 0 else "idx_scan_bf16_kernel<1, 1> (with the entry's compression)")
        # (3) the step's first launch (compression + scan, the same kernel
        # instance) K times back to back, as csa_compress_indexer_score runs
        # it: the step's launch also accumulates the top-k's digit histogram,
        # which this one skips
        scores = ws_t[:B * Tq * N * 4].view(torch.float32).view(B, Tq, N)

        def scan(i):
            r = reps[i % len(reps)]
            L.csa_compress_indexer_score(r["Ca"], r["Cb"], r["Za"], r["Zb"], shared["Ba"], shared["Bb"],
                                         r["kv_comp"], r["q_idx"], r["w"], r["k_idx"], r.get("k_scale"),
                                         shared["q_pos"], shared["n_comp"], scores, m_c=m, m=m,
                                         tok_begin=cfg.n - 2 * m, blk_begin=N - 1, blk_end=N, q_fp4=cfg.q_fp4)

        scan_ms = _graph_loop_ms(torch, scan, steps)
        res["roofline"] = _roofline("hbm", kname, scan_bytes, scan_ms, HBM_PEAK_GBS, "GB/s",
                                    _traffic(f"idx_scan_{wname}_traffic.txt",
                                             ["indexer.hip", "common.h", "compress_entry.h"]), copy_gbs)
        # the same launch inside the traced step, between the library's phase
        # events (which add their own 1-3 us)
        res["roofline"]["in_step_ms"] = round(float(ph_mean[1]), 4)
        res["phases_ms"] = {"before_call": round(float(ph_mean[0]), 4), "compress_and_scan": round(float(ph_mean[1]), 4),
                            "topk": round(float(ph_mean[2]), 4),
                            "attention": round(float(ph_mean[3]), 4), "merge": round(float(ph_mean[4]), 4),
                            "after_call": round(float(ph_mean[5]), 4)}
        res["step_hbm_gbs"] = round(step_bytes / (ms_step * 1e-3) / 1e9, 1)
        res["step_algorithmic_bytes"] = step_bytes
        res["indexer_kv_hbm_gbs"] = res["roofline"]["achieved"]
    else:
        # the step's two launches: the appended entry (m tokens of Ca and Za
        # in, the entry out), every row once, q in, the output out
        abytes = B * ((N + W) * rowb + H * D * 2 * 2 + 2 * m * D * 2 + rowb)
        res["config"] = {"workload": cfg.name, "batch": B, "context_tokens": cfg.n, "compressed_entries": N,
                         "m": m, "heads": H, "head_dim": D, "window": W, "kv_dtype": cfg.kv_dtype}
        res["phases_ms"] = {"before_call": round(float(ph_mean[0]), 4),
                            "append_and_attention": round(float(ph_mean[1] + ph_mean[2] + ph_mean[3]), 4),
                            "merge": round(float(ph_mean[4]), 4)}

        def hca(i):
            r = reps[i % len(reps)]
            L.hca_decode_step(r["Ca"], r["Za"], shared["Ba"], r["q"], r["kv_comp"], shared["n_comp"],
                              shared["q_pos"].view(B), r["kv_win"], shared["win_len"], shared["sink"], out, m_c=m, m=m,
                              tok_begin=cfg.n - m, blk_begin=N - 1, blk_end=N, ws=ws_a)

        attn_ms = _graph_loop_ms(torch, hca, steps)
        fp8 = cfg.kv_dtype == "fp8"
        res["roofline"] = _roofline("hbm", "hca_decode_step: attn_bf16_kernel<1, %s> (append + HCA decode splits) + "
                                    "attn_combine_kernel" % ("true" if fp8 else "false"),
                                    abytes, attn_ms, HBM_PEAK_GBS, "GB/s",
                                    _traffic(f"hca_step_{wname}_traffic.txt",
                                             ["attn.hip", "attn_core.h", "compress_entry.h", "common.h"]),
                                    copy_gbs)
        res["step_hbm_gbs"] = round(abytes / (ms_step * 1e-3) / 1e9, 1)
    res["wall_s_timed"] = round(wall, 3)
    if cpu_s is not None:
        res["cpu_baseline"] = cpu_baseline(cfg, x, cpu_s)
    del reps, base
    return res


def prefill_flops(cfg, pos):
    """Algorithmic FLOPs of a prefill chunk: indexer over visible pairs,
    sparse MQA over min(k, V) selected rows and the window rows."""
    V = np.minimum(cfg.N, (pos.astype(np.int64) + 1) // cfg.m)
    win = np.minimum(cfg.W, pos.astype(np.int64) + 1)
    idx = float(V.sum()) * cfg.H_I * cfg.D_I * 2
    mqa = float((np.minimum(cfg.top_k, V) + win).sum()) * cfg.H * cfg.D * 4
    return idx, mqa


def bench_prefill(a, torch, L, gen, dev, cfg, steps, warmup, cpu_s, wname):
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
    idx = torch.empty((1, T, k), dtype=torch.int32, device=dev)
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    ws_t = torch.zeros(L.indexer_score_topk_workspace_bytes(1, T, N, k), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    ev = None

    def run(trace=False):
        if trace: ev["pre"].record(stream)
        L.csa_compress(Ca, Cb, Za, Zb, Ba, Bb, comp, m=m, stream=s)
        for c, ch in enumerate(chunks):
            if trace: L.trace_phases(ev["idx"][c])  # [0] start [1] scan launched [2..4] top-k done
            L.indexer_score_topk(ch["q_idx"], ch["w"], k_idx, None, ch["q_pos"], n_comp, idx, m=m, ws=ws_t,
                                 stream=s)
            L.sparse_mqa_prefill(ch["q"], comp[0], idx[0], kv_tok, ch["q_pos"][0], sink, out, W=W, stream=s)
            if trace: ev["attn"][c].record(stream)
        if trace: L.trace_phases(None)

    for _ in range(max(1, warmup)):
        run()
    torch.cuda.synchronize()
    steps = max(1, min(steps, 5))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = {"pre": mk(), "idx": [[mk() for _ in range(5)] for _ in range(nch)], "attn": [mk() for _ in range(nch)]}
    for e in [ev["pre"]] + ev["attn"] + [e for es in ev["idx"] for e in es]:
        e.record(stream)
    torch.cuda.synchronize()
    run(trace=True)
    torch.cuda.synchronize()
    comp_ms = ev["pre"].elapsed_time(ev["idx"][0][0])
    idx_ms = [ev["idx"][c][0].elapsed_time(ev["idx"][c][1]) for c in range(nch)]
    topk_ms = [ev["idx"][c][1].elapsed_time(ev["idx"][c][4]) for c in range(nch)]
    attn_ms = [ev["idx"][c][4].elapsed_time(ev["attn"][c]) for c in range(nch)]
    fl = [prefill_flops(cfg, ch["pos_np"]) for ch in chunks]
    idx_fl, mqa_fl = sum(f[0] for f in fl), sum(f[1] for f in fl)
    total_fl = idx_fl + mqa_fl
    res = _base(steps, max(1, warmup))
    res.update({
        "value": round(cfg.n / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "config": {"workload": cfg.name, "tokens": cfg.n, "query_chunk": T, "compressed_entries": N, "m": m,
                   "top_k": k, "indexer_heads": cfg.H_I, "indexer_dim": cfg.D_I, "heads": H, "head_dim": D,
                   "window": W, "kv_dtype": cfg.kv_dtype},
        "prefill_tflops": round(total_fl / (ms * 1e-3) / 1e12, 2),
        "algorithmic_tflop": round(total_fl / 1e12, 3),
        # per launch: a 4096-query chunk (all chunks' flops over all chunks' time)
        "roofline": _roofline("mfma", "attn_prs_kernel<2, %s> (sparse prefill, per 4096-query chunk)"
                              % ("true" if fp8 else "false"), mqa_fl / nch, float(np.mean(attn_ms)),
                              BF16_PEAK_TFLOPS, "TFLOP/s",
                              _traffic(f"attn_prefill_{wname}_traffic.txt",
                                       ["attn.hip", "attn_core.h", "compress_entry.h", "common.h"])),
        "roofline_indexer": _roofline("mfma", "idx_prefill_kernel (per 4096-query chunk)", idx_fl / nch,
                                      float(np.mean(idx_ms)), BF16_PEAK_TFLOPS, "TFLOP/s",
                                      _traffic(f"idx_prefill_{wname}_traffic.txt",
                                               ["indexer.hip", "common.h", "compress_entry.h"])),
        "phases_ms": {"compress": round(comp_ms, 4), "indexer_total": round(sum(idx_ms), 4),
                      "topk_total": round(sum(topk_ms), 4), "attention_total": round(sum(attn_ms), 4)},
    })
    if cpu_s is not None:
        res["cpu_baseline"] = cpu_prefill_baseline(cfg, tok, cpu_s)
    return res


def hca_prefill_rows(cfg, pos):
    """Rows each query attends in HCA prefill: V(p) entries plus its window."""
    pos = pos.astype(np.int64)
    return np.minimum(cfg.N, (pos + 1) // cfg.m) + np.minimum(cfg.W, pos + 1)


def bench_hca_prefill(a, torch, L, gen, dev, steps, warmup, cpu_s):
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

    for _ in range(max(1, warmup)):
        run()
    torch.cuda.synchronize()
    steps = max(1, min(steps, 5))
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
    res = _base(steps, max(1, warmup))
    res.update({
        "value": round(cfg.n / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "config": {"workload": cfg.name, "tokens": cfg.n, "query_chunk": T, "compressed_entries": N, "m": m,
                   "heads": H, "head_dim": D, "window": W},
        "prefill_tflops": round(mqa_fl / (ms * 1e-3) / 1e12, 2),
        "algorithmic_tflop": round(mqa_fl / 1e12, 3),
        "roofline": _roofline("mfma", "attn_prs_kernel<3> (HCA prefill, per 4096-query chunk)", mqa_fl / nch,
                              float(np.mean(attn_ms)), BF16_PEAK_TFLOPS, "TFLOP/s"),
        "phases_ms": {"compress": round(comp_ms, 4), "attention_total": round(sum(attn_ms), 4)},
    })
    if cpu_s is not None:
        res["cpu_baseline"] = cpu_hca_prefill_baseline(cfg, tok, cpu_s)
    return res


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
                                              win[max(0, hi - cfg.W + 1):hi + 1], x["sink"], k_scale=sc, tau=tau,
                                              q_fp4=cfg.q_fp4)
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
