#!/usr/bin/env python3
"""Throughput of the DFlash / DFlash2 draft block step on one MI355X.

One step is one pass of the whole hot path over one block of synthetic
input: inject 16 accepted tokens' target features (fc + RMSNorm + Wk/Wv into
the cache), the DFlash2 grouped dynamic conv, non-causal block attention over
the injected context plus the block, the LM head with top-K and unary
scores, the selector edges with their best path, and the accept length.

Default workload (the 32k-context setting, Qwen-27B-shaped bf16 layer): the
cache holds 32768 injected rows (written by a timed 32768-token prefill
injection, reported on its own as MFMA TFLOP/s), each step re-injects the last
16 context rows and drafts one B = 16 block over 32768 + 16 keys.

    python bench.py [--steps K] [--warmup W] [--workload c2|c1|c3|c4] [--no-cpu]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA
METRIC = "draft block steps/s + drafted tok/s at 32k ctx; % HBM / MFMA peak"
WORKLOADS = {"c1": "c1_qwen27b_1k", "c2": "c2_prefill_32k", "c3": "c3_decode_64k", "c4": "c4_q8_0_32k"}
COUNTERS = os.path.join(ROOT, "profiles", "lmhead_topk_c2_counters.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--kv", default="act", choices=["act", "q8_0"],
                    help="KV cache in the activation type or Q8_0 (codes + fp16 block scales)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU-baseline leg")
    ap.add_argument("--prefill-reps", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the batched-conv, per-kernel and streaming-ceiling measurements "
                         "(for runs under an external profiler)")
    ap.add_argument("--inject-sweep", action="store_true",
                    help="only time dflash_inject for 1..64 stashed blocks of B accepted tokens "
                         "(deferred, batched injection) and print that sweep")
    ap.add_argument("--topk-rows", action="store_true",
                    help="only time the row-wise top-K call against torch.topk and a full sort "
                         "over a grid of shapes and print that")
    ap.add_argument("--site-lines", action="store_true",
                    help="only time the batched conv (2048 blocks) and the feed-forward site and "
                         "print those two lines (for counter runs under an external profiler)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    return ap.parse_args()


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_diffusion_drafter_step_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_counters(cfg):
    """HBM bytes per LM-head launch from the committed rocprofv3 counter
    summary, or None when there is none, the kernel source changed since, or
    the summary was taken on an LM head of another shape or weight type."""
    try:
        c = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if c.get("source_hash") != src_hash("topk.hip", "merge.h", "common.h", "stream.h", "dflash_abi.cpp"):
        return None
    if c.get("lm_head_shape") != {"V": cfg.V, "d": cfg.d, "B": cfg.B, "K": cfg.K, "weights": cfg.weight}:
        return None
    return c.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calib_copy:
        n = 1 << 28                     # 2^28 floats = 1 GiB read + 1 GiB written per copy
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": 4 * n, "calib_copy_bytes_written": 4 * n, "reps": 5}))
        return

    from block_diffusion_drafter_step_amd import configs, pipeline, synth, workmodel
    from block_diffusion_drafter_step_amd import dflash as D

    D.load()
    if args.topk_rows:
        print(json.dumps({"topk_rows": topk_rows_sweep()}), flush=True)
        return
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = configs.get(WORKLOADS[args.workload])
    decode64 = cfg.prefill_kv > 0
    inj_n = 16
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + cfg.seed)
    adt = pipeline.act_dtype(cfg.act)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(adt)

    host = synth.Workload(cfg)
    W = pipeline.DeviceWeights(host, drop_host=args.no_cpu or args.inject_sweep)
    kvq = args.kv == "q8_0"
    kvt = "q8_0" if kvq else None
    cache = pipeline.new_cache(cfg, kv=kvt)
    if args.inject_sweep:
        print(json.dumps({"workload": cfg.name, "inject_sweep": inject_sweep(cfg, W, cache, randn)}),
              flush=True)
        return
    if args.site_lines:
        print(json.dumps({"workload": cfg.name, "conv_batched": conv_batched(cfg, W, randn),
                          "ffn_block": ffn_block_line(cfg, randn)}), flush=True)
        return
    prefill = None
    if decode64:
        # long-context decode: the cache already holds prefill_kv seeded rows
        if kvq:   # codes uniform in [-127, 127], scales of N(0, 1) rows (max |x| ~ 3.5 over 32 values)
            p = cfg.prefill_kv
            for t in (cache.k[:, :p], cache.v[:, :p // 32]):
                t.copy_(torch.randint(-127, 128, t.shape, generator=gen, device=dev, dtype=torch.int32)
                        .to(torch.int8))
            for t in (cache.k_scales[:, :p], cache.v_scales[:, :p]):
                t.copy_((torch.rand(t.shape, generator=gen, device=dev) * 0.01 + 0.022).half())
        else:
            cache.k[:, :cfg.prefill_kv].copy_(randn(cfg.Hkv, cfg.prefill_kv, cfg.hd))
            cache.v[:, :cfg.prefill_kv // 32].copy_(randn(cfg.Hkv, cfg.prefill_kv // 32, cfg.hd, 32))
        n_ctx0 = cfg.prefill_kv
    else:
        # prefill injection of n_ctx tokens (the MFMA-bound tile GEMM path)
        n = cfg.n_ctx
        hid = [randn(n, cfg.d_t) for _ in range(cfg.L_t)]
        ws = D.workspace(D.dflash_inject_workspace(cfg.L_t, n, cfg.d_t, cfg.d, cfg.kv, cfg.act))
        for _ in range(2):   # untimed: the first calls also ramp the clocks up
            D.dflash_inject(hid, W.fc, None, cfg.eps, W.wk, W.wv, cache, 0, ws)
        torch.cuda.synchronize()
        times = []
        for _ in range(args.prefill_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            D.dflash_inject(hid, W.fc, None, cfg.eps, W.wk, W.wv, cache, 0, ws)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
        fl = workmodel.inject_flops(n, cfg.L_t, cfg.d_t, cfg.d, cfg.kv)
        t = float(np.median(times))
        prefill = {"tokens": n, "ms": round(t * 1e3, 3), "tflop": round(fl / 1e12, 3),
                   "achieved_tflops": round(fl / t / 1e12, 1), "peak_tflops": MFMA_BF16_PEAK_TFS,
                   "frac": round(fl / t / 1e12 / MFMA_BF16_PEAK_TFS, 4), "bound": "mfma"}
        del hid, ws
        n_ctx0 = cfg.n_ctx
        torch.cuda.empty_cache()

    step = pipeline.BlockStep(cfg, W, cache, inject_n=inj_n)
    hid16 = [randn(inj_n, cfg.d_t) for _ in range(cfg.L_t)]
    x = randn(1, cfg.B, cfg.d)
    anchor = int(host.anchor()[0])
    target = torch.randint(0, cfg.V, (1, cfg.B), generator=gen, device=dev, dtype=torch.int32)

    def positions(i):
        """(pos0 of the 16 injected rows, context rows attended) for step i."""
        if decode64:
            s = i % cfg.steps
            return n_ctx0 + inj_n * s, n_ctx0 + inj_n * (s + 1)
        return n_ctx0 - inj_n, n_ctx0

    # the LM head's top-K, the selector and the accept length against the
    # target tokens in one call (dflash_topk_select)
    names = ["inject", "conv", "attn", "topk+select+accept"]
    calls = [lambda i: step.inject(hid16, positions(i)[0]),
             lambda i: step.conv(x),
             lambda i: step.attn(x, positions(i)[1]),
             lambda i: step.topk_select(anchor, target)]

    def whole_step(i):
        """One step as BlockStep.run enqueues it, in one stream."""
        pos0, n_ctx = positions(i)
        step.run(x, n_ctx, anchor, target, hidden=hid16, pos0=pos0)

    for i in range(args.warmup):
        whole_step(i)
    torch.cuda.synchronize()

    # timed region: whole steps, wall clock between two device synchronisations
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        whole_step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / K
    steps_s = K / (t1 - t0)

    # the dominant kernel's launch duration: a pass of LM_CALLS LM-head calls
    # after the timed region, each bracketed by HIP events on the stream it is
    # launched on (the current stream)
    LM_CALLS = 64
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(LM_CALLS)]
    for e0, e1 in ev:
        e0.record()
        step.topk()   # dflash_topk_unary: the LM-head kernel and its merge
        e1.record()
    torch.cuda.synchronize()
    topk_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    # per-call breakdown: a separate pass after the timed region, events around every call
    nb = min(K, 100)
    evc = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
           for _ in range(nb)]
    for i in range(nb):
        for j, c in enumerate(calls):
            evc[i][j][0].record()
            c(i)
            evc[i][j][1].record()
    torch.cuda.synchronize()
    per = {n: float(np.mean([evc[i][j][0].elapsed_time(evc[i][j][1]) for i in range(nb)]))
           for j, n in enumerate(names)}

    extras = {}
    if not args.no_extras:
        extras["conv_batched"] = conv_batched(cfg, W, randn)
        extras["ffn_block"] = ffn_block_line(cfg, randn)
        ctx_prof = int(np.mean([positions(i)[1] for i in range(20)]))
        extras["kernels"] = kernel_profile(cfg, calls, ctx_prof, kvt)
        extras["hbm_ceiling"] = stream_ceiling()

    if decode64:
        ctx_mean = float(np.mean([positions(i)[1] for i in range(cfg.steps)]))
    else:
        ctx_mean = n_ctx0
    step_bytes = workmodel.step_bytes(cfg, int(ctx_mean), inject_n=inj_n, kv=kvt)
    lm_bytes = workmodel.lmhead_bytes(cfg)
    lm_gbs = lm_bytes / (topk_ms * 1e-3) / 1e9
    attn_bytes = workmodel.attn_bytes(cfg, int(ctx_mean), kv=kvt)
    roofline = {"bound": "hbm", "kernel": "dflash_topk_unary (LM-head top-K kernel + topk_merge_kernel)",
                "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(lm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic_from_counters(cfg),
                "bytes_per_launch": lm_bytes, "launch_ms": round(topk_ms, 4),
                "launch_samples": len(ev)}

    out = {"metric": METRIC, "value": round(steps_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": K,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if cfg.weight == "bf16" else "bf16 x q8_0",
           "data": "synthetic (seeded; random weights of the workload's shapes)",
           "config": {"workload": f"{cfg.name}: decode step at {int(ctx_mean)}-row context"
                                  + (", Q8_0 KV cache" if kvq else ""),
                      "B": cfg.B, "n_ctx": int(ctx_mean), "inject_per_step": inj_n, "d": cfg.d,
                      "L_t": cfg.L_t, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "hd": cfg.hd, "C": cfg.C, "G": cfg.G,
                      "T": cfg.T, "V": cfg.V, "K": cfg.K, "r": cfg.r, "weights": cfg.weight,
                      "kv_cache": "q8_0" if kvq else cfg.act},
           "drafted_tok_per_s": round(steps_s * cfg.B, 1),
           "step_bytes": step_bytes,
           "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "roofline": roofline,
           "per_call_ms": {k: round(v, 4) for k, v in per.items()},
           "per_call_note": "separate pass after the timed region, HIP events around each call",
           "attn_gbs": round(attn_bytes / (per["attn"] * 1e-3) / 1e9, 1)}
    if prefill:
        out["prefill"] = prefill
    out.update(extras)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, host, int(ctx_mean), inj_n, kvq)
    print(json.dumps(out), flush=True)


def topk_rows_sweep(rows=(2, 64, 4096), cols=(128, 4096, 200000), ks=(64, 1024), reps=10):
    """dflash_topk_rows on seeded N(0,1) fp32 rows against torch.topk and a
    full stable descending torch.sort on the same GPU (HIP events, mean of
    `reps` calls after 2 untimed ones).  HBM roofline: the matrix read once."""
    import torch
    from block_diffusion_drafter_step_amd import dflash as D
    g = torch.Generator(device="cuda")
    g.manual_seed(20)

    def timed(f):
        for _ in range(2):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    res = []
    for r in rows:
        for c in cols:
            x = torch.randn(r, c, generator=g, device="cuda")
            for k in ks:
                if k > c:
                    continue
                idx = torch.empty(r, k, dtype=torch.int32, device="cuda")
                val = torch.empty(r, k, dtype=torch.float32, device="cuda")
                ws = D.workspace(D.dflash_topk_rows_workspace(r, c, k))
                us = timed(lambda: D.dflash_topk_rows(x, k, idx, val, ws))
                us_topk = timed(lambda: torch.topk(x, k, dim=1, largest=True, sorted=True))
                us_sort = timed(lambda: torch.sort(x, dim=1, descending=True, stable=True))
                by = r * c * 4
                res.append({"rows": r, "cols": c, "K": k, "us": round(us, 1), "torch_topk_us": round(us_topk, 1),
                            "full_sort_us": round(us_sort, 1), "vs_sort": round(us_sort / us, 2),
                            "gbs": round(by / us / 1e3, 1), "hbm_frac": round(by / us / 1e3 / HBM_PEAK_GBS, 4)})
                print(json.dumps(res[-1]), file=sys.stderr, flush=True)
                del ws, idx, val
            del x
            torch.cuda.empty_cache()
    return res


def inject_sweep(cfg, W, cache, randn, blocks=(1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128)):
    """dflash_inject of 16 k rows: the accepted tokens of k blocks stashed and
    injected at once (deferred injection), k up to 64 and past it.  Each size
    is timed with HIP events on the current stream (median of 5 after 2
    untimed calls).  Bytes: features + fc + Wk + Wv + cache rows; FLOPs:
    fc + Wk + Wv."""
    import numpy as np
    import torch
    from block_diffusion_drafter_step_amd import dflash as D, workmodel
    res = []
    for k in blocks:
        n = cfg.B * k
        hid = [randn(n, cfg.d_t) for _ in range(cfg.L_t)]
        ws = D.workspace(D.dflash_inject_workspace(cfg.L_t, n, cfg.d_t, cfg.d, cfg.kv, cfg.act))
        for _ in range(2):
            D.dflash_inject(hid, W.fc, None, cfg.eps, W.wk, W.wv, cache, 0, ws)
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            D.dflash_inject(hid, W.fc, None, cfg.eps, W.wk, W.wv, cache, 0, ws)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = float(np.median(ts))
        by = workmodel.inject_bytes(cfg, n)
        fl = workmodel.inject_flops(n, cfg.L_t, cfg.d_t, cfg.d, cfg.kv)
        # the roofline is whichever of HBM and MFMA takes longer for these bytes and flops
        t_roof = max(by / (HBM_PEAK_GBS * 1e9), fl / (MFMA_BF16_PEAK_TFS * 1e12))
        res.append({"blocks": k, "tokens": n, "us": round(t * 1e6, 1), "us_per_token": round(t * 1e6 / n, 3),
                    "gbs": round(by / t / 1e9, 1), "tflops": round(fl / t / 1e12, 1),
                    "roofline_us": round(t_roof * 1e6, 1), "frac_of_roofline": round(t_roof / t, 4)})
        del hid, ws
        torch.cuda.empty_cache()
    return res


def conv_batched(cfg, W, randn, tokens=32768, reps=20):
    """The conv call over a batch of blocks holding `tokens` positions (2048
    blocks of 16 at the 32k setting's token count), HBM bytes = x in + u out
    + base + W_delta over the call time (HIP events on the current stream)."""
    import torch
    from block_diffusion_drafter_step_amd import dflash as D, workmodel
    nb = tokens // cfg.B
    x = randn(nb, cfg.B, cfg.C)
    u = torch.empty_like(x)
    ws = D.workspace(D.dflash_conv_workspace(nb, cfg.B, cfg.C, cfg.G, cfg.T))
    for _ in range(3):
        D.dflash_conv(x, cfg.G, W.base, W.w_delta, u, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        D.dflash_conv(x, cfg.G, W.base, W.w_delta, u, ws)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    b = workmodel.conv_bytes(cfg, nb)
    del x, u, ws
    torch.cuda.empty_cache()
    return {"blocks": nb, "B": cfg.B, "us": round(t * 1e6, 1), "bytes": b,
            "achieved": round(b / t / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}


def ffn_block_line(cfg, randn, reps=20):
    """The feed-forward site (dflash_ffn_block: its conv pair, the gated SiLU
    MLP and the residual) on one block of B rows, with random weights of the
    workload's shapes (Q8_0 codes and scales for the quantised workload); HBM
    bytes = h in, out, the conv pair and the three MLP weights over the call
    time (HIP events on the current stream)."""
    import torch
    from block_diffusion_drafter_step_amd import dflash as D, workmodel
    d, F = cfg.d, cfg.d_ff

    def weight(rows, cols, dtype):
        if dtype == "q8_0":
            q = torch.randint(-127, 128, (rows, cols), dtype=torch.int8, device="cuda")
            s = (torch.rand(rows, cols // 32, device="cuda") * 0.019 + 0.001).half()
            return D.Weight("q8_0", q, s)
        return D.Weight(dtype, randn(rows, cols) * cols ** -0.5)

    h = randn(1, cfg.B, d)
    out = torch.empty_like(h)
    base = randn(cfg.T, d) * 0.7
    wd = weight(cfg.T * cfg.G, d, cfg.act)
    wg, wu, wn = weight(F, d, cfg.weight), weight(F, d, cfg.weight), weight(d, F, cfg.weight)
    ws = D.workspace(D.dflash_ffn_block_workspace(1, cfg.B, d, cfg.G, cfg.T, F))
    for _ in range(3):
        D.dflash_ffn_block(h, cfg.G, base, wd, wg, wu, wn, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        D.dflash_ffn_block(h, cfg.G, base, wd, wg, wu, wn, out, ws)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    b = workmodel.ffn_bytes(cfg, 1)
    del wg, wu, wn, ws
    torch.cuda.empty_cache()
    return {"B": cfg.B, "d": d, "d_ff": F, "weights": cfg.weight, "us": round(t * 1e6, 1), "bytes": b,
            "achieved": round(b / t / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}


def kernel_profile(cfg, calls, n_ctx, kvt=None, steps=20):
    """Average device time of every kernel over `steps` whole steps, from a
    torch.profiler device trace (it records every dispatch of the process,
    libdflash's included), and the HBM fractions of the kernels it names:
    attention = KV bytes over (split + combine), LM head = its bytes over
    (top-K kernel + merge)."""
    import torch
    from block_diffusion_drafter_step_amd import workmodel
    try:
        from torch.profiler import ProfilerActivity, profile
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for i in range(steps):
                for c in calls:
                    c(i)
            torch.cuda.synchronize()
        avg = {}
        for e in prof.key_averages():
            tot = getattr(e, "device_time_total", None)
            if tot is None:
                tot = getattr(e, "cuda_time_total", 0.0)
            if e.count and tot and ("dfl" in e.key):
                avg[e.key] = (e.count, tot / e.count)
    except Exception as ex:   # a profiler that cannot trace here leaves the rest of the line intact
        return {"error": f"{type(ex).__name__}: {ex}"}

    def us(sub):
        return sum(v[1] for k, v in avg.items() if sub in k)

    out = {"steps": steps, "avg_us": {k[:90]: round(v[1], 2) for k, v in sorted(avg.items(), key=lambda kv: -kv[1][1] * kv[1][0])}}
    split, comb = us("attn_split_kernel"), us("attn_combine_kernel")
    # in the step the LM head's merge runs inside the top-K + selector kernel
    lm, merge = us("lmhead_topk"), us("topk_merge_kernel") + us("topk_select_kernel")
    if split + comb > 0:
        kv = workmodel.attn_kv_bytes(cfg, n_ctx, kvt)
        out["attention_kv"] = {"n_ctx": n_ctx, "bytes": kv, "split_us": round(split, 2),
                               "combine_us": round(comb, 2),
                               "achieved": round(kv / ((split + comb) * 1e-6) / 1e9, 1),
                               "frac": round(kv / ((split + comb) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                               "split_only_frac": round(kv / (split * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if lm > 0:
        b = workmodel.lmhead_bytes(cfg)
        out["lm_head"] = {"bytes": b, "kernel_us": round(lm, 2),
                          "kernel_frac": round(b / (lm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "merge_and_selector_us": round(merge, 2)}
    return out


def stream_ceiling(reps=10):
    """Measured streaming rates of plain device kernels on 1 GiB: a copy (read +
    write) and a sum (read)."""
    import torch
    n = 1 << 28
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    r = {}
    for name, fn, nbytes in [("copy", lambda: b.copy_(a), 8 * n), ("sum", lambda: a.sum(), 4 * n)]:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        r[name + "_gbs"] = round(nbytes / t / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return r


def cpu_baseline(cfg, host, n_ctx, inj_n, kvq=False, reps=3):
    """The oracle (fp64 numpy, untuned) running whole block steps of the same
    workload on the host cores: injection of 16 rows, conv, attention over
    n_ctx + B keys, LM head over V, selector, accept.  Each stage is timed
    (median of `reps` steps), and the 32k prefill injection of the prefill
    workloads is timed on 512 of its rows and extrapolated to all of them."""
    import numpy as np
    import threadpoolctl

    import oracle as O
    from block_diffusion_drafter_step_amd import synth

    t_setup = time.perf_counter()
    f = O.weight_to_f64
    a = lambda t: O.act_to_f64(t, cfg.act)
    bp = cfg.act == "bf16"
    # the context rows the step attends are drawn on the host (same distribution)
    shp = (cfg.Hkv, n_ctx, cfg.hd)
    if kvq:
        ck = O.kv_dequant_q8_0(*O.kv_quant_q8_0(synth.normal(cfg.seed, "cpu.ck", shp, 1.0, "f32")), bp)
        cv = O.kv_dequant_q8_0(*O.kv_quant_q8_0(synth.normal(cfg.seed, "cpu.cv", shp, 1.0, "f32")), bp)
    else:
        ck = a(synth.normal(cfg.seed, "cpu.ck", shp, 1.0, cfg.act))
        cv = a(synth.normal(cfg.seed, "cpu.cv", shp, 1.0, cfg.act))
    hid = [a(synth.normal(cfg.seed, f"cpu.hid.{l}", (inj_n, cfg.d_t), 1.0, cfg.act)) for l in range(cfg.L_t)]
    x = a(host.x())[0]
    A, Bc = host.codebooks()
    A, Bc = a(A), a(Bc)
    anchor = int(host.anchor()[0])
    fc, wk, wv, wq, wo = f(host.fc()), f(host.wk()), f(host.wv()), f(host.wq()), f(host.wo())
    base, wd, P, wl = a(host.conv_base()), f(host.w_delta()), f(host.sel_proj()), host.w_lm()
    setup = time.perf_counter() - t_setup
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    rows = lambda m: m.reshape(inj_n, cfg.Hkv, cfg.hd).transpose(1, 0, 2)

    def one_step():
        t = {}
        t0 = time.perf_counter()
        if kvq:   # the cache keeps codes of the unrounded projections
            z = O.encode(hid, fc, None, cfg.eps, bp)["z"]
            ck[:, n_ctx - inj_n:] = O.kv_dequant_q8_0(*O.kv_quant_q8_0(rows(z @ wk.T)), bp)
            cv[:, n_ctx - inj_n:] = O.kv_dequant_q8_0(*O.kv_quant_q8_0(rows(z @ wv.T)), bp)
        else:
            inj = O.inject(hid, fc, None, cfg.eps, wk, wv, bp)
            ck[:, n_ctx - inj_n:] = rows(inj["k"])
            cv[:, n_ctx - inj_n:] = rows(inj["v"])
        t["inject"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        c = O.conv(x[None], base, wd, cfg.G, bp)
        t["conv"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        at = O.block_attn(c["u"][0], x, wq, wk, wv, wo, ck, cv, n_ctx, cfg.Hq, 0.0, bp)
        t["attn"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        tk = O.topk_unary_from_logits(O.lm_logits_stored(at["out"], wl), cfg.K)
        t["topk"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        sel = O.selector(at["out"], P, A, Bc, tk["idx"], tk["unary"], anchor)
        t["select"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.accept_len(sel["path"][None, :], sel["path"][None, :])
        t["accept"] = time.perf_counter() - t0
        return t

    runs = [one_step() for _ in range(reps)]
    stages = {k: float(np.median([r[k] for r in runs])) for k in runs[0]}
    step_s = float(np.median([sum(r.values()) for r in runs]))
    out = {"value": round(1.0 / step_s, 5), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
           "sample": f"median of {reps} whole oracle block steps of the same workload ({step_s:.2f} s each; "
                     f"fp64 numpy, untuned; input staging {setup:.1f} s not counted)",
           "stage_s": {k: round(v, 4) for k, v in stages.items()},
           "affinity_cpus": len(os.sched_getaffinity(0))}
    if cfg.n_ctx >= 4096 and not cfg.prefill_kv:
        # the prefill injection on 512 seeded rows, extrapolated to n_ctx rows
        m = 512
        ph = [a(synth.normal(cfg.seed, f"cpu.pf.{l}", (m, cfg.d_t), 1.0, cfg.act)) for l in range(cfg.L_t)]
        t0 = time.perf_counter()
        O.inject(ph, fc, None, cfg.eps, wk, wv, bp)
        tp = time.perf_counter() - t0
        out["prefill_sample"] = {"rows": m, "s": round(tp, 3), "tokens": cfg.n_ctx,
                                 "extrapolated_s": round(tp * cfg.n_ctx / m, 2),
                                 "note": "extrapolated from 512 rows (rows are independent)"}
    return out


if __name__ == "__main__":
    main()
