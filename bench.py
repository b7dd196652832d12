#!/usr/bin/env python3
"""Benchmark of the self-conditioning soft embedding on one MI355X.

A step is one pass of the whole hot path over one canvas batch: se_row_stats over
the full-width fp32 logits, then the rank's slice contraction, both on one stream.
The contraction path is chosen with --path:
  step     se_soft_embed_step (default): statistics and the slice embedding in one
           call, outputs bitwise those of se_row_stats + se_soft_embed_fused
  unfused  se_row_stats, then se_probs_bf16 + se_soft_embed (bitwise the fused call)
  staged   se_row_stats, then se_soft_embed_staged (bitwise the fused call)
  fused    se_row_stats, then se_soft_embed_fused (probabilities rebuilt in the GEMM
           prologue)
  step_onepass  se_soft_embed_step_onepass: the whole step from one read of the
           logits (equal to the step up to rounding)
  onepass  se_soft_embed_onepass, which forms the row statistics from the same read
           of the logits (whole-vocabulary workloads only; no se_row_stats call)
Inputs are seeded synthetic data already resident in HBM when the timed region starts.

Default workload: one tensor-parallel rank's share at its real shape (L_c = 256
canvas positions, full-width logits over V = 262,144, slice [65536, 131072) of a
bf16 table padded to 262,400 rows, d = 2,816, gamma = sqrt(2816)).

Prints ONE JSON line.  ``value`` is soft-embed GFLOP/s over the whole step
(2 L (e - s) d FLOP per step / step time); the same line carries steps/s, per-call
times, the roofline of the timed call (the whole step for step, step_onepass and
onepass; the contraction call otherwise), every other path timed on the same inputs,
the vendor GEMM at the same shape, and the fp64 oracle timed on this host as a CPU
baseline.
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

METRIC = "soft-embed GFLOP/s + steps/s at L_c=256,V=262144,d=2816; % of roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
KERNEL_SOURCES = ["soft_embed.hip", "row_stats.hip", "probs.hip", "onepass.hip", "se_device.h",
                  "se_launch.h", "api.cpp"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "diffusion_self_conditioning_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def fused_call_bytes(w) -> int:
    """Algorithmic HBM bytes of one fused call: the bf16 shard slice once, the fp32 logits
    slice once, the fp32 output once."""
    return 2 * w.k * w.d + 4 * w.rows * w.k + 4 * w.rows * w.d


def fp8_call_bytes(w) -> int:
    """Algorithmic HBM bytes of one fused call on the e4m3 table: the codes and row scales of
    the slice once, the fp32 logits slice once, the fp32 output once."""
    return w.k * w.d + 4 * w.k + 4 * w.rows * w.k + 4 * w.rows * w.d


def event_time_us(fn, K: int, warmup: int) -> float:
    """Average time of fn() over K back-to-back calls, from events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for k in range(K):
        fn()
        ev[k + 1].record()
    torch.cuda.synchronize()
    return sum(ev[k].elapsed_time(ev[k + 1]) for k in range(K)) * 1e3 / K


def row_stats_bytes(w) -> int:
    return 4 * w.rows * w.vocab + 16 * w.rows


def measured_traffic(path: str, workload: str):
    """HBM bytes per call of the step's contraction path from the committed rocprofv3 counter
    summary of this workload, if it was taken on the current kernel sources; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", f"traffic_soft_embed_{path}_{workload}.json")) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("bytes_per_call")


def cpu_baseline(w, x_np, bits, budget_s: float = 12.0):
    """The fp64 oracle (row stats + slice contraction) on a bounded row sample of the same
    workload, on this host's cores; scaled to GFLOP/s of the soft embedding."""
    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    shard = bits[w.vocab_start:w.vocab_end]
    rows = max(1, cores)
    t0 = time.perf_counter()
    oracle.row_stats(x_np[:rows])
    oracle.soft_embed(x_np[:rows], w.vocab_start, w.vocab_end, shard, w.gamma)
    dt = time.perf_counter() - t0
    if dt < budget_s / 3:
        rows = min(w.rows, max(rows, int(rows * budget_s / max(dt, 1e-3))) // cores * cores or cores)
        t0 = time.perf_counter()
        oracle.row_stats(x_np[:rows])
        oracle.soft_embed(x_np[:rows], w.vocab_start, w.vocab_end, shard, w.gamma)
        dt = time.perf_counter() - t0
    flops = 2 * rows * w.k * w.d
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    return {"value": round(flops / dt / 1e9, 4), "unit": "GFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows} of {w.rows} rows of the {w.name} workload (row stats over "
                      f"V={w.vocab} + fp64 contraction over the {w.k}-row slice), {dt:.2f} s "
                      f"on {model}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU needs tens of milliseconds of this work before its kernels run at their
    # steady-state speed (measured: 5 warmup steps leave the rank step about 6% slow)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="rank", choices=["rank", "full", "conv", "batch", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="step",
                    choices=["unfused", "fused", "staged", "step", "step_onepass", "onepass"],
                    help="how the step runs: se_soft_embed_step (default, one call, bitwise the "
                         "separate calls), se_soft_embed_step_onepass (one call, one read of the "
                         "logits), or se_row_stats followed by the unfused, staged or fused "
                         "contraction, or se_soft_embed_onepass (whole-vocabulary workloads; "
                         "softmax statistics from the same read of the logits)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (the "
                         "reference for scaling the HBM byte counters), then exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration // 4
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 4 * n, "launches": 5}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the soft embedding of one tensor-parallel rank needs no second GPU; the "
              "cross-rank all-reduce is not part of this library.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    from diffusion_self_conditioning_amd import _binding as B
    from diffusion_self_conditioning_amd import api
    from diffusion_self_conditioning_amd import workloads as wl

    w = wl.get(args.workload)
    whole = w.vocab_start == 0 and w.vocab_end == w.vocab
    if args.path == "onepass" and not whole:
        print("--path onepass needs a workload whose slice is the whole vocabulary (its row "
              "statistics are those of the slice)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    x_np = wl.make_logits(w)
    bits, _ = wl.make_table(w)
    x = torch.from_numpy(x_np).to(dev)
    table = torch.from_numpy(bits).to(dev)
    shard = table[w.vocab_start:w.vocab_end]
    L, d = w.rows, w.d
    mx = torch.empty(L, device=dev)
    lse = torch.empty(L, device=dev)
    ent = torch.empty(L, device=dev)
    am = torch.empty(L, device=dev, dtype=torch.int32)
    out = torch.empty((L, d), device=dev)
    ws = api.workspace(L, w.vocab_start, w.vocab_end, d, dev)
    probs = torch.empty((L, w.vocab), device=dev, dtype=torch.bfloat16)
    wso = api.onepass_workspace(L, w.vocab_start, w.vocab_end, d, dev)
    wss = api.staged_workspace(L, w.vocab_start, w.vocab_end, d, dev)
    ws1 = api.step_onepass_workspace(L, w.vocab, w.vocab_start, w.vocab_end, d, dev)

    def stats():
        B.se_row_stats(x, mx, lse, ent, am)

    def call_unfused(o):
        B.se_probs_bf16(x, lse, w.vocab_start, w.vocab_end, probs)
        B.se_soft_embed(probs, w.vocab_start, w.vocab_end, shard, w.gamma, o, ws)

    def call_fused(o):
        B.se_soft_embed_fused(x, lse, w.vocab_start, w.vocab_end, shard, w.gamma, o, ws)

    def call_staged(o):
        B.se_soft_embed_staged(x, lse, w.vocab_start, w.vocab_end, shard, w.gamma, o, wss)

    def call_step(o):
        B.se_soft_embed_step(x, w.vocab_start, w.vocab_end, shard, w.gamma, o, mx, lse, ent, am,
                             wss)

    def call_step_onepass(o):
        B.se_soft_embed_step_onepass(x, w.vocab_start, w.vocab_end, shard, w.gamma, o, mx, lse,
                                     ent, am, ws1)

    def call_onepass(o):
        B.se_soft_embed_onepass(x, w.vocab_start, w.vocab_end, shard, w.gamma, o, mx, lse, ent,
                                am, wso)

    calls = {"unfused": call_unfused, "fused": call_fused, "staged": call_staged,
             "step": call_step, "step_onepass": call_step_onepass, "onepass": call_onepass}
    call_names = {"unfused": "se_probs_bf16 + se_soft_embed", "fused": "se_soft_embed_fused",
                  "staged": "se_soft_embed_staged", "step": "se_soft_embed_step",
                  "step_onepass": "se_soft_embed_step_onepass",
                  "onepass": "se_soft_embed_onepass"}
    embed = calls[args.path]
    # the one-pass and whole-step calls form the statistics themselves
    with_stats = args.path not in ("onepass", "step", "step_onepass")

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        if with_stats:
            stats()
        embed(out)
    torch.cuda.synchronize()

    # timed region: K whole steps, events around each call on the launch stream
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    for k in range(K):
        ev[k][0].record()
        if with_stats:
            stats()
        ev[k][1].record()
        embed(out)
        ev[k][2].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / K
    us_stats = [ev[k][0].elapsed_time(ev[k][1]) * 1e3 for k in range(K)]
    us_embed = [ev[k][1].elapsed_time(ev[k][2]) * 1e3 for k in range(K)]
    us_stats_avg = sum(us_stats) / K
    us_embed_avg = sum(us_embed) / K
    us_step_sorted = sorted(a + b for a, b in zip(us_stats, us_embed))

    flops = w.flops()
    gflops_step = flops / (ms_step * 1e-3) / 1e9
    gflops_call = flops / (us_embed_avg * 1e-6) / 1e9
    call_bytes = fused_call_bytes(w)
    if args.path == "onepass":          # plus the statistics it writes
        call_bytes += 16 * L
    elif args.path in ("step", "step_onepass"):   # the whole step: every logit once, table, outputs
        call_bytes = row_stats_bytes(w) + 2 * w.k * w.d + 4 * L * w.d
    achieved_gbs = call_bytes / (us_embed_avg * 1e-6) / 1e9
    t_roof_call_us = max(flops / (PEAK_BF16_TFLOPS * 1e12), call_bytes / (PEAK_HBM_GBS * 1e9)) * 1e6
    stats_bytes = row_stats_bytes(w) if with_stats else 0
    step_bytes = call_bytes + stats_bytes
    t_roof_step_us = (stats_bytes / (PEAK_HBM_GBS * 1e9) + t_roof_call_us * 1e-6) * 1e6
    mfma_bound = flops / (PEAK_BF16_TFLOPS * 1e12) > call_bytes / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(args.path, w.name)
    roof = {"bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(gflops_call / 1e3 if mfma_bound else achieved_gbs, 2),
            "peak": PEAK_BF16_TFLOPS if mfma_bound else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "traffic": traffic}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = call_names[args.path] + " call"
    roof["algorithmic_bytes"] = call_bytes

    # side measurements (not part of `value`): every contraction path on the same inputs,
    # each event-timed as one call; the unfused and fused outputs are compared bitwise
    side = {}
    ref_out = out.clone()
    exact = args.path in ("unfused", "fused", "staged", "step")
    for name in ("unfused", "fused", "staged"):
        o = torch.empty_like(out)
        side[name + "_call_us"] = round(event_time_us(lambda: calls[name](o), K, args.warmup), 2)
        if exact:
            side[name + "_equals_step_output"] = bool(torch.equal(o, ref_out))
        del o
    # the two whole-step calls (statistics included), and how far apart their outputs are
    o1, o2 = torch.empty_like(out), torch.empty_like(out)
    side["step_call_us"] = round(event_time_us(lambda: call_step(o1), K, args.warmup), 2)
    side["step_onepass_call_us"] = round(event_time_us(lambda: call_step_onepass(o2), K,
                                                       args.warmup), 2)
    side["step_onepass_rel_diff_vs_step"] = float(
        (o2.double() - o1.double()).norm() / o1.double().norm())
    del o1, o2
    side["gflops_unfused_call"] = round(flops / (side["unfused_call_us"] * 1e-6) / 1e9, 2)
    side["gflops_fused_call"] = round(flops / (side["fused_call_us"] * 1e-6) / 1e9, 2)
    side["gflops_staged_call"] = round(flops / (side["staged_call_us"] * 1e-6) / 1e9, 2)

    # side measurement: the sampler's acceptance / convergence step on this step's row
    # statistics (canvases of 256 positions)
    acc_side = None
    if L % 256 == 0:
        nc = L // 256
        st = {"acc": torch.zeros(L, dtype=torch.uint8, device=dev),
              "prev": torch.full((L,), -1, dtype=torch.int32, device=dev),
              "sc": torch.zeros(nc, dtype=torch.int32, device=dev),
              "stc": torch.zeros(nc, dtype=torch.int32, device=dev),
              "new": torch.empty(L, dtype=torch.uint8, device=dev),
              "conv": torch.empty(nc, dtype=torch.uint8, device=dev)}

        def accept_step():
            B.se_accept_converge(ent, am, 256, 8.0, 3, 0.05, 64, st["acc"], st["prev"], st["sc"],
                                 st["stc"], st["new"], st["conv"])

        acc_side = {"accept_converge_us": round(event_time_us(accept_step, K, args.warmup), 2),
                    "canvases": nc, "accepted_last_step": int(st["new"].sum().item())}

    # side measurement: the on-device sum of 4 per-rank partials of this output shape,
    # written as fp32 and bf16
    parts4 = torch.randn((4, L, d), device=dev)
    red_f = torch.empty((L, d), device=dev)
    red_b = torch.empty((L, d), dtype=torch.bfloat16, device=dev)
    red_us = event_time_us(lambda: B.se_reduce_partials(parts4, out=red_f, out_bf16=red_b), K,
                           args.warmup)
    red_side = {"reduce_partials_us": round(red_us, 2), "parts": 4,
                "gbs": round((4 * 4 + 4 + 2) * L * d / (red_us * 1e-6) / 1e9, 1)}
    del parts4, red_f, red_b

    # side measurement: the same calls on the e4m3 form of the shard (quantized once on the
    # GPU, untimed), fused and unfused, with the fused call's HBM roofline
    codes = torch.empty((w.k, d), dtype=torch.uint8, device=dev)
    wscale = torch.empty(w.k, device=dev)
    B.se_quantize_table_fp8(shard, codes, wscale)
    out8 = torch.empty_like(out)
    pr8 = torch.empty((L, w.vocab), device=dev, dtype=torch.bfloat16)
    B.se_probs_bf16(x, lse, w.vocab_start, w.vocab_end, pr8)
    us_f8 = event_time_us(lambda: B.se_soft_embed_fp8_fused(
        x, lse, w.vocab_start, w.vocab_end, codes, wscale, w.gamma, out8, ws), K, args.warmup)
    us_u8 = event_time_us(lambda: B.se_soft_embed_fp8(
        pr8, w.vocab_start, w.vocab_end, codes, wscale, w.gamma, out8, ws), K, args.warmup)
    # the whole step against the e4m3 table (statistics + staged probabilities + contraction)
    mx8, lse8, ent8 = torch.empty(L, device=dev), torch.empty(L, device=dev), torch.empty(L, device=dev)
    am8 = torch.empty(L, device=dev, dtype=torch.int32)
    us_s8 = event_time_us(lambda: B.se_soft_embed_step_fp8(
        x, w.vocab_start, w.vocab_end, codes, wscale, w.gamma, out8, mx8, lse8, ent8, am8, wss),
        K, args.warmup)
    s8_bytes = row_stats_bytes(w) + w.k * d + 4 * w.k + 4 * L * d
    us_q = event_time_us(lambda: B.se_quantize_table_fp8(shard, codes, wscale), 3, 1)
    f8_bytes = fp8_call_bytes(w)
    fp8_side = {"fused_call_us": round(us_f8, 2),
                "gflops_fused_call": round(flops / (us_f8 * 1e-6) / 1e9, 2),
                "unfused_gemm_only_us": round(us_u8, 2),
                "roofline_fused_call": {"bound": "hbm", "algorithmic_bytes": f8_bytes,
                                        "achieved": round(f8_bytes / (us_f8 * 1e-6) / 1e9, 2),
                                        "peak": PEAK_HBM_GBS,
                                        "frac": round(f8_bytes / (us_f8 * 1e-6) / 1e9
                                                      / PEAK_HBM_GBS, 4)},
                "step_us": round(us_s8, 2),
                "gflops_step": round(flops / (us_s8 * 1e-6) / 1e9, 2),
                "roofline_step": {"bound": "hbm", "algorithmic_bytes": s8_bytes,
                                  "achieved": round(s8_bytes / (us_s8 * 1e-6) / 1e9, 2),
                                  "peak": PEAK_HBM_GBS,
                                  "frac": round(s8_bytes / (us_s8 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
                "quantize_shard_us": round(us_q, 2)}
    del codes, wscale, out8, pr8, mx8, lse8, ent8, am8

    # side measurement: the one-pass call over the same slice (softmax over the slice, row
    # statistics from the same read of the logits), and the merge of 4 slice results.  For
    # a slice that is the whole vocabulary the one-pass call is a whole step.
    oo = torch.empty((L, d), device=dev)
    so = [torch.empty(L, device=dev) for _ in range(3)]
    ao = torch.empty(L, device=dev, dtype=torch.int32)
    us_o = event_time_us(lambda: B.se_soft_embed_onepass(
        x, w.vocab_start, w.vocab_end, shard, w.gamma, oo, so[0], so[1], so[2], ao, wso), K,
        args.warmup)
    outs4 = torch.randn((4, L, d), device=dev)
    st4 = [torch.randn((4, L), device=dev) for _ in range(3)]
    am4 = torch.zeros((4, L), device=dev, dtype=torch.int32)
    us_m = event_time_us(lambda: B.se_merge_slices(outs4, st4[0], st4[1], st4[2], am4, oo, so[0],
                                                   so[1], so[2], ao), K, args.warmup)
    o_bytes = fused_call_bytes(w) + 16 * L
    onepass_side = {"call_us": round(us_o, 2),
                    "gflops_call": round(flops / (us_o * 1e-6) / 1e9, 2),
                    "roofline_call": {"bound": "hbm", "algorithmic_bytes": o_bytes,
                                      "achieved": round(o_bytes / (us_o * 1e-6) / 1e9, 2),
                                      "peak": PEAK_HBM_GBS,
                                      "frac": round(o_bytes / (us_o * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                                    4)},
                    "merge_4_slices_us": round(us_m, 2)}
    del oo, so, ao, outs4, st4, am4

    # cold step: a 1 GiB write between steps evicts L2 and the 256 MB MALL first; and the
    # achievable HBM rate of a plain 1 GiB device-to-device copy, beside the 8 TB/s peak
    scrub = torch.empty(1 << 28, device=dev)
    cold = []
    for k in range(5):
        scrub.fill_(float(k))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if with_stats:
            stats()
        embed(out)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    src = torch.ones(1 << 28, device=dev)
    copy_us = event_time_us(lambda: scrub.copy_(src), 10, 3)
    del scrub, src
    # achievable dense bf16 matrix-core rate on this machine: the vendor GEMM (torch.mm, contiguous
    # operands) on an 8192-cube, beside the 2.5 PFLOP/s peak
    ga = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)
    gb = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)
    mm_us = event_time_us(lambda: torch.mm(ga, gb), 10, 5)
    del ga, gb
    # the vendor GEMM at this call's own shape: the slice's bf16 probabilities [rows, K]
    # (row-major, contiguous) times the bf16 shard [K, d], fp32 output, beside the library's
    # contraction of the same operands (se_soft_embed on the probabilities se_probs_bf16 wrote)
    B.se_probs_bf16(x, lse, w.vocab_start, w.vocab_end, probs)
    pa = probs[:, w.vocab_start:w.vocab_end].contiguous()
    pb = shard.view(torch.bfloat16)
    og = torch.empty_like(out)
    vend_us = event_time_us(lambda: torch.mm(pa, pb, out_dtype=torch.float32), 10, 5)
    ours_us = event_time_us(lambda: B.se_soft_embed(probs, w.vocab_start, w.vocab_end, shard,
                                                    w.gamma, og, ws), 10, 5)
    del pa, pb, og
    ceilings = {"cold_step_us_median": round(sorted(cold)[len(cold) // 2], 2),
                "hbm_copy_gbs": round(2 * (1 << 28) * 4 / (copy_us * 1e-6) / 1e9, 1),
                "bf16_gemm_8192_tflops": round(2 * 8192 ** 3 / (mm_us * 1e-6) / 1e12, 1),
                "vendor_gemm_same_shape_us": round(vend_us, 2),
                "vendor_gemm_same_shape_tflops": round(flops / (vend_us * 1e-6) / 1e12, 1),
                "library_contraction_same_shape_us": round(ours_us, 2),
                "library_contraction_same_shape_tflops": round(flops / (ours_us * 1e-6) / 1e12, 1)}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, x_np, bits)

    line = {
        "metric": METRIC, "value": round(gflops_step, 2), "unit": "GFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: L_c={L} rows, full-width fp32 logits V={w.vocab}, "
                               f"slice [{w.vocab_start},{w.vocab_end}) of a bf16 table "
                               f"[{w.table_rows}, {d}], gamma={w.gamma:.6g}"
                               + f" ({args.path})",
                   "rows": L, "vocab": w.vocab, "vocab_start": w.vocab_start,
                   "vocab_end": w.vocab_end, "d": d, "seed": w.seed},
        "steps_per_s": round(1e3 / ms_step, 2),
        "canvas_steps_per_s": round(1e3 / ms_step * (L / 256), 2),
        "gflops_call": round(gflops_call, 2),
        "kernel_us": {"se_row_stats": round(us_stats_avg, 2) if with_stats else None,
                      call_names[args.path]: round(us_embed_avg, 2)},
        "step_us_median": round(us_step_sorted[K // 2], 2),
        "step_us_min": round(us_step_sorted[0], 2),
        "roofline": roof,
        "roofline_step": {"t_roof_us": round(t_roof_step_us, 2),
                          "frac": round(t_roof_step_us / (ms_step * 1e3), 4),
                          "algorithmic_bytes": step_bytes},
        "roofline_call_t_roof_us": round(t_roof_call_us, 2),
        "wall_s_timed": round(wall, 4),
        "paths": side,
        "accept_converge": acc_side,
        "reduce_partials": red_side,
        "fp8_table": fp8_side,
        "onepass": onepass_side,
        "cold_and_ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
