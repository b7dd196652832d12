#!/usr/bin/env python3
"""Benchmark of the self-conditioning soft embedding on one MI355X.

A step is one pass of the whole hot path over one canvas batch: the softmax
statistics of the full-width fp32 logits (max, log-sum-exp, entropy, argmax) and the
soft embedding gamma * P[:, s:e] W_shard of the step's vocabulary slice.

Default workload: the whole vocabulary, one canvas (L_c = 256 positions, V = 262,144,
slice [0, 262144), d = 2,816, gamma = sqrt(2816); 378 GFLOP of soft embedding per step),
timed on its fastest whole-step path, se_soft_embed_step_onepass (statistics and
embedding from one read of the logits).  --path picks another way to run the step:
  step          se_soft_embed_step: statistics then the slice embedding, one call, bitwise
                se_row_stats + se_soft_embed_fused
  step_onepass  se_soft_embed_step_onepass (one read of the logits; equal to step up to
                rounding)
  onepass       se_soft_embed_onepass (whole-vocabulary workloads: the slice statistics are
                the row statistics)
  unfused       se_row_stats, then se_probs_bf16 + se_soft_embed
  staged        se_row_stats, then se_soft_embed_staged
  fused         se_row_stats, then se_soft_embed_fused
Inputs are seeded synthetic data, resident in HBM before the timed region starts.  Before
anything is timed the step runs back to back for 60 ms: after an idle gap of a few
milliseconds the GPU's power control drops below its sustained clock for tens of
milliseconds, and a sampler runs its steps back to back.  Then --warmup W steps and
--steps K timed steps, back to back with nothing recorded between them.

Prints ONE JSON line.  ``value`` is soft-embed GFLOP/s over whole steps (2 L (e - s) d
FLOP per step / ms_per_step).  The line also carries: steps/s; the duration of each
kernel of one step, from start and end events that the dispatch stamps for the library's
launches (se_set_launch_events), and the gaps between them; ``roofline`` of the dominant
kernel (the contraction) and
``roofline_step`` of the whole step, both on measured times; ``parity`` of the timed
step's outputs against the fp64 oracle on every row (the rows the CPU baseline
computes); ``cpu_baseline`` (that oracle's time on this host's cores); every other path
on the same inputs; and ``workloads``: the one-rank shard (65,536-position slice), the
near-converged canvas and the 2,048-row batch, each timed on its fastest path with its
own rooflines and sampled oracle parity.
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
                  "se_launch.h", "se_dispatch.h", "api.cpp"]
# fastest whole-step path of each workload (measured on MI355X)
BEST_PATH = {"tiny": "step", "rank": "step", "full": "step_onepass", "conv": "step_onepass",
             "batch": "step_onepass"}
# kernel launches of one call, in order
LAUNCHES = {
    "step": ["row_stats_kernel<stats + staged slice>", "soft_embed_pp_kernel",
             "splitk_reduce_kernel"],
    "step_onepass": ["step_sweep_kernel", "soft_embed_pp_kernel", "merge_ranges_kernel",
                     "scaled_reduce_kernel"],
    "onepass": ["step_sweep_kernel", "soft_embed_pp_kernel", "merge_ranges_kernel",
                "scaled_reduce_kernel"],
    "step_onepass_fp8": ["step_sweep_kernel<scaled>", "soft_embed_pp_kernel<e4m3 in place>",
                         "merge_ranges_kernel", "scaled_reduce_kernel"],
    "staged": ["row_stats_kernel", "probs_bf16_kernel<tiled>", "soft_embed_pp_kernel",
               "splitk_reduce_kernel"],
    "fused": ["row_stats_kernel", "soft_embed_kernel<fused>", "splitk_reduce_kernel"],
    "unfused": ["row_stats_kernel", "probs_bf16_kernel", "soft_embed_pp_kernel",
                "splitk_reduce_kernel"],
}
GATE_REL_FRO, ENTROPY_TOL, LSE_REL_TOL = 5e-3, 1e-4, 2e-6


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "diffusion_self_conditioning_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def event_time_us(fn, K: int, warmup: int, settle_ms: float = 0.0) -> float:
    """Average time of fn() over K back-to-back calls, from two events on the current stream
    around them (nothing recorded in between), after `warmup` calls (and, with settle_ms,
    after running fn back to back for that long)."""
    import torch
    if settle_ms > 0:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        spent = 0.0
        while spent < settle_ms:
            e0.record()
            for _ in range(10):
                fn()
            e1.record()
            e1.synchronize()
            spent += e0.elapsed_time(e1)
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / K


def step_bytes_logits_once(w) -> int:
    """Algorithmic HBM bytes of a whole step that reads every logit once: the full-width
    fp32 logits, the bf16 table slice, the fp32 output and the four statistics per row."""
    return 4 * w.rows * w.vocab + 2 * w.k * w.d + 4 * w.rows * w.d + 16 * w.rows


def step_bytes_two_pass(w) -> int:
    """The step's bytes as the two-pass design counts them: statistics over the full width
    (4 L V + 16 L) plus the fused call (table slice, logits slice, output)."""
    return (4 * w.rows * w.vocab + 16 * w.rows) + (2 * w.k * w.d + 4 * w.rows * w.k
                                                   + 4 * w.rows * w.d)


def contraction_bytes(w, fused: bool, table_elem_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one contraction launch: the table slice once (bf16, or e4m3
    codes: table_elem_bytes 1) and the probability operand once (staged bf16, or fp32 logits
    for the fused kernel).  The split partials are implementation traffic, not counted."""
    return table_elem_bytes * w.k * w.d + (4 if fused else 2) * w.rows * w.k


def roofline(flops: int, nbytes: int, us: float, traffic=None) -> dict:
    mfma = flops / (PEAK_BF16_TFLOPS * 1e12) > nbytes / (PEAK_HBM_GBS * 1e9)
    achieved = flops / (us * 1e-6) / 1e12 if mfma else nbytes / (us * 1e-6) / 1e9
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS
    return {"bound": "mfma" if mfma else "hbm", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s" if mfma else "GB/s", "frac": round(achieved / peak, 4),
            "traffic": traffic}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary of this
    workload, if it was taken on the current kernel sources; else (None, reason)."""
    name = f"profiles/traffic_{kernel}_{workload}.json"
    try:
        with open(os.path.join(ROOT, name)) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None, f"no counter summary {name}"
    if t.get("kernel_hash") != kernel_hash():
        return None, f"{name} was taken on kernel sources {t.get('kernel_hash')}, not these"
    return t.get("bytes_per_launch"), f"{t.get('source', name)} (kernel sources {t['kernel_hash']})"


class Step:
    """Device buffers of one workload and the calls that run its step."""

    def __init__(self, w, x_np, bits, dev):
        import torch
        from diffusion_self_conditioning_amd import api
        self.w, self.dev = w, dev
        self.x = torch.from_numpy(x_np).to(dev)
        self.table = torch.from_numpy(bits).to(dev)
        self.shard = self.table[w.vocab_start:w.vocab_end]
        L, d = w.rows, w.d
        f = dict(device=dev, dtype=torch.float32)
        self.mx, self.lse, self.ent = torch.empty(L, **f), torch.empty(L, **f), torch.empty(L, **f)
        self.am = torch.empty(L, device=dev, dtype=torch.int32)
        self.out = torch.empty((L, d), **f)
        self.ws = api.workspace(L, w.vocab_start, w.vocab_end, d, dev)
        self.wss = api.staged_workspace(L, w.vocab_start, w.vocab_end, d, dev)
        self.ws1 = api.step_onepass_workspace(L, w.vocab, w.vocab_start, w.vocab_end, d, dev)
        self.wso = None
        self.probs = None
        self.codes = self.wscale = None

    def quantized(self):
        """The e4m3 codes and power-of-two row scales of the shard (quantized once)."""
        if self.codes is None:
            import torch
            from diffusion_self_conditioning_amd import _binding as B
            self.codes = torch.empty(tuple(self.shard.shape), dtype=torch.uint8, device=self.dev)
            self.wscale = torch.empty(self.shard.shape[0], device=self.dev)
            B.se_quantize_table_fp8(self.shard, self.codes, self.wscale)
        return self.codes, self.wscale

    def call(self, path: str, out=None):
        from diffusion_self_conditioning_amd import _binding as B
        from diffusion_self_conditioning_amd import api
        w, o = self.w, (self.out if out is None else out)
        s, e = w.vocab_start, w.vocab_end
        stats = (self.mx, self.lse, self.ent, self.am)
        if path == "step":
            B.se_soft_embed_step(self.x, s, e, self.shard, w.gamma, o, *stats, self.wss)
        elif path == "step_onepass":
            B.se_soft_embed_step_onepass(self.x, s, e, self.shard, w.gamma, o, *stats, self.ws1)
        elif path == "step_onepass_fp8":
            codes, wscale = self.quantized()
            B.se_soft_embed_step_onepass_fp8(self.x, s, e, codes, wscale, w.gamma, o, *stats,
                                             self.ws1)
        elif path == "onepass":
            if self.wso is None:
                self.wso = api.onepass_workspace(w.rows, s, e, w.d, self.dev)
            B.se_soft_embed_onepass(self.x, s, e, self.shard, w.gamma, o, *stats, self.wso)
        else:
            B.se_row_stats(self.x, *stats)
            if path == "unfused":
                if self.probs is None:
                    import torch
                    self.probs = torch.empty((w.rows, w.vocab), device=self.dev,
                                             dtype=torch.bfloat16)
                B.se_probs_bf16(self.x, self.lse, s, e, self.probs)
                B.se_soft_embed(self.probs, s, e, self.shard, w.gamma, o, self.ws)
            elif path == "staged":
                B.se_soft_embed_staged(self.x, self.lse, s, e, self.shard, w.gamma, o, self.wss)
            elif path == "fused":
                B.se_soft_embed_fused(self.x, self.lse, s, e, self.shard, w.gamma, o, self.ws)
            else:
                raise ValueError(path)


def condition(st: Step, path: str, min_ms: float = 60.0, min_calls: int = 20):
    """Run the step back to back for at least `min_ms` of GPU time before anything is timed.
    After an idle gap of a few milliseconds the GPU starts a burst at a high clock and then,
    a few steps in, drops below its sustained clock for tens of milliseconds while its power
    control settles (measured: the first 60 whole-vocabulary steps after a 10 ms gap average
    467 us, against 430 us back to back); this brings every measurement that follows to the
    sustained state a serving loop runs in."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, spent = 0, 0.0
    while n < min_calls or spent < min_ms:
        e0.record()
        for _ in range(10):
            st.call(path)
        e1.record()
        e1.synchronize()
        spent += e0.elapsed_time(e1)
        n += 10


def timed_steps(st: Step, path: str, K: int, W: int):
    """W warmup steps, then K timed steps back to back, bracketed by synchronisations and by
    two events on the launch stream (nothing is recorded between the steps: an event between
    two steps delays the next one by several µs).  Then K more steps with an event after each,
    for the spread of single steps.  Returns (ms_per_step, per-step µs list, wall seconds of
    the timed steps)."""
    import torch
    for _ in range(W):
        st.call(path)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for k in range(K):
        st.call(path)
    ev[K].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[K]) / K
    ev[0].record()
    for k in range(K):
        st.call(path)
        ev[k + 1].record()
    torch.cuda.synchronize()
    per = [ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(K)]
    return ms, per, wall


class HipEvents:
    """Timing events of the HIP runtime this process already runs (the one torch loaded and
    the library uses), created with hipEventDisableSystemFence: completing one performs no
    system-scope cache writeback and invalidation, which would slow the kernel after it."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        import torch
        torch.cuda.init()
        path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln)
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.live = []

    def create(self, n: int) -> list:
        out = []
        for _ in range(n):
            h = self.ct.c_void_p()
            if self.hip.hipEventCreateWithFlags(self.ct.byref(h),
                                                self.ct.c_uint(self.DISABLE_SYSTEM_FENCE)):
                raise RuntimeError("hipEventCreateWithFlags failed")
            out.append(h.value)
        self.live += out
        return out

    def record(self, ev: int, stream: int) -> None:
        if self.hip.hipEventRecord(self.ct.c_void_p(ev), self.ct.c_void_p(stream)):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_us(self, a: int, b: int) -> float:
        t = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(t), self.ct.c_void_p(a), self.ct.c_void_p(b)):
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value * 1e3

    def destroy_all(self) -> None:
        for h in self.live:
            self.hip.hipEventDestroy(self.ct.c_void_p(h))
        self.live = []


def kernel_times(st: Step, path: str, K: int):
    """Per-launch kernel durations of one step, averaged over K back-to-back steps: the
    library's launch markers (se_set_launch_events) have the dispatch stamp each kernel's
    start and end into two events, so a duration is the kernel alone and the steps run as
    in the timed region (no command between them, nothing synchronises).  Also the gaps
    between consecutive kernels of a step.  Returns ([(name, µs)], [gap µs])."""
    import torch
    from diffusion_self_conditioning_amd import _binding as B
    n_max = 16
    hev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    steps = [hev.create(n_max) for _ in range(K)]
    bracket = hev.create(2)
    torch.cuda.synchronize()
    used = []
    hev.record(bracket[0], stream)
    for marks in steps:
        B.se_set_launch_events(marks)
        st.call(path)
        used.append(B.se_launch_events_used())
        B.se_set_launch_events([])
    hev.record(bracket[1], stream)
    torch.cuda.synchronize()
    n_used = used[0] // 2
    if any(u != 2 * n_used for u in used) or n_used == 0:
        hev.destroy_all()
        raise RuntimeError("launch count changed between steps")
    sums, gaps = [0.0] * n_used, [0.0] * max(0, n_used - 1)
    for marks in steps:
        t = [hev.elapsed_us(marks[2 * j], marks[2 * j + 1]) for j in range(n_used)]
        g = [hev.elapsed_us(marks[2 * j - 1], marks[2 * j]) for j in range(1, n_used)]
        sums = [a + b for a, b in zip(sums, t)]
        gaps = [a + b for a, b in zip(gaps, g)]
    marked_us = hev.elapsed_us(bracket[0], bracket[1]) / K
    hev.destroy_all()
    names = LAUNCHES.get(path, [])
    if path in ("step_onepass", "onepass", "step_onepass_fp8") and n_used == 3:
        from diffusion_self_conditioning_amd import _binding as B
        w = st.w
        two_pass = path != "onepass" and (
            B.se_soft_embed_step_onepass_workspace_bytes(w.rows, w.vocab, w.vocab_start,
                                                         w.vocab_end, w.d)
            == B.se_soft_embed_staged_workspace_bytes(w.rows, w.vocab_start, w.vocab_end, w.d))
        one = LAUNCHES[path]
        names = ([] if two_pass and path.endswith("_fp8")   # the two-pass e4m3 step: unnamed
                 else LAUNCHES["step"] if two_pass          # the one-read call ran the two-pass step
                 else [one[0], one[1], one[3]])
    if len(names) != n_used:
        names = [f"launch_{j}" for j in range(n_used)]
    return [(names[j], sums[j] / K) for j in range(n_used)], [v / K for v in gaps], marked_us


def step_report(st: Step, path: str, K: int, W: int) -> dict:
    """Timed steps, per-kernel times and rooflines of one workload on one path."""
    w = st.w
    condition(st, path)
    ms, per, wall = timed_steps(st, path, K, W)
    kt, gaps, marked_us = kernel_times(st, path, K)
    flops = w.flops()
    dom_i = max(range(len(kt)), key=lambda j: kt[j][1] if "soft_embed" in kt[j][0] else -1)
    dom_name, dom_us = kt[dom_i]
    fused = "fused" in dom_name
    e4m3 = path.endswith("_fp8")
    traffic, source = measured_traffic("soft_embed_kernel_fused" if fused else
                                       "soft_embed_pp_kernel_e4m3" if e4m3 else
                                       "soft_embed_pp_kernel", w.name)
    nbytes = contraction_bytes(w, fused, 1 if e4m3 else 2)
    roof = roofline(flops, nbytes, dom_us, traffic)
    roof.update({"kernel": dom_name, "kernel_us": round(dom_us, 2),
                 "algorithmic_bytes": nbytes,
                 "algorithmic_flops": flops, "traffic_source": source,
                 "basis": "algorithmic bytes (table slice + staged bf16 probabilities) "
                          "or FLOP of one launch / its duration between the start and end "
                          "events the dispatch stamps"})
    once, two = step_bytes_logits_once(w), step_bytes_two_pass(w)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12) * 1e6

    def step_roof(nbytes):
        t_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e6
        # the statistics pass is HBM work that cannot hide under an MFMA-bound contraction
        stats_us = (4 * w.rows * w.vocab + 16 * w.rows) / (PEAK_HBM_GBS * 1e9) * 1e6
        t_roof = max(t_hbm, stats_us + t_mfma)
        return {"algorithmic_bytes": nbytes, "t_roof_us": round(t_roof, 2),
                "frac": round(t_roof / (ms * 1e3), 4)}

    srt = sorted(per)
    return {
        "path": path, "ms_per_step": round(ms, 5), "steps_per_s": round(1e3 / ms, 2),
        "canvas_steps_per_s": round(1e3 / ms * (w.rows / 256), 2),
        "gflops": round(flops / (ms * 1e-3) / 1e9, 2),
        "step_us_median": round(srt[len(srt) // 2], 2), "step_us_min": round(srt[0], 2),
        "wall_s_timed": round(wall, 4),
        "kernel_us": {name: round(us, 2) for name, us in kt},
        "gaps_between_kernels_us": [round(g, 2) for g in gaps],
        "marked_step_us": round(marked_us, 2),
        "roofline": roof,
        "roofline_step": {
            "basis": "whole-step algorithmic bytes (or the statistics pass plus the MFMA "
                     "time, if longer) / ms_per_step",
            "logits_once": step_roof(once),
            "two_pass_design": step_roof(two)},
    }


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            return next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                        "unknown CPU")
    except OSError:
        return "unknown CPU"


def parity(w, got: dict, ref_stats: dict, ref_out, rows) -> dict:
    """The GPU step's outputs against the fp64 oracle on `rows`: argmax and row max exact,
    lse within 2e-6 relative, entropy within 1e-4 nats, the soft embedding within 5e-3
    relative Frobenius (the oracle takes exact p)."""
    import numpy as np
    r = np.asarray(rows)
    am_bad = int(np.sum(got["argmax"][r] != ref_stats["argmax"][r]))
    d_max = float(np.max(np.abs(got["max"][r].astype(np.float64) - ref_stats["max"][r])))
    lse_rel = float(np.max(np.abs(got["lse"][r] - ref_stats["lse"][r])
                           / np.maximum(1.0, np.abs(ref_stats["lse"][r]))))
    d_h = float(np.max(np.abs(got["entropy"][r] - ref_stats["entropy"][r])))
    o = got["out"][r].astype(np.float64)
    rel = float(np.linalg.norm(o - ref_out) / max(np.linalg.norm(ref_out), 1e-300))
    row_rel = np.linalg.norm(o - ref_out, axis=1) / np.maximum(
        np.linalg.norm(ref_out, axis=1), 1e-300)
    ok = am_bad == 0 and d_max == 0.0 and lse_rel <= LSE_REL_TOL and d_h <= ENTROPY_TOL \
        and rel <= GATE_REL_FRO
    return {"rows_checked": int(r.size), "rows_total": w.rows,
            "argmax_mismatches": am_bad, "max_abs_d_row_max": d_max,
            "max_rel_d_lse": lse_rel, "max_abs_d_entropy_nats": d_h,
            "rel_fro": rel, "max_row_rel_fro": float(np.max(row_rel)),
            "tolerances": {"argmax": "exact", "row_max": "exact", "lse_rel": LSE_REL_TOL,
                           "entropy_nats": ENTROPY_TOL, "rel_fro": GATE_REL_FRO},
            "pass": bool(ok)}


def fetch(st: Step) -> dict:
    return {"out": st.out.cpu().numpy(), "max": st.mx.cpu().numpy(),
            "lse": st.lse.cpu().numpy(), "entropy": st.ent.cpu().numpy(),
            "argmax": st.am.cpu().numpy()}


def cpu_baseline_and_parity(w, x_np, bits, got, budget_s: float = 30.0):
    """The fp64 oracle (statistics over the full width + slice contraction) on this host's
    cores: every row when it fits the time budget, else an even sample; its time is the
    CPU baseline, its results the parity reference."""
    import numpy as np
    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    shard = bits[w.vocab_start:w.vocab_end]
    probe = min(w.rows, max(1, cores))
    t0 = time.perf_counter()
    oracle.soft_embed(x_np[:probe], w.vocab_start, w.vocab_end, shard, w.gamma)
    per_row = (time.perf_counter() - t0) / probe
    n = w.rows if per_row * w.rows <= budget_s else max(probe, int(budget_s / per_row))
    rows = np.unique(np.linspace(0, w.rows - 1, n).round().astype(np.int64))
    xs = np.ascontiguousarray(x_np[rows])
    t0 = time.perf_counter()
    ref_stats_s = oracle.row_stats(xs)
    ref_out = oracle.soft_embed(xs, w.vocab_start, w.vocab_end, shard, w.gamma)
    dt = time.perf_counter() - t0
    ref_stats = {k: np.zeros(w.rows, v.dtype) for k, v in ref_stats_s.items()}
    for k, v in ref_stats_s.items():
        ref_stats[k][rows] = v
    par = parity(w, got, ref_stats, ref_out, rows)
    base = {"value": round(2 * rows.size * w.k * w.d / dt / 1e9, 4), "unit": "GFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{rows.size} of {w.rows} rows of the {w.name} workload (statistics over "
                      f"V={w.vocab} + fp64 contraction over the {w.k}-position slice), "
                      f"{dt:.2f} s on {host_cpu()}"}
    return base, par


def sampled_parity(w, x_np, bits, got, seed: int = 11):
    """Oracle parity on two seeded rows of every 256-row tile plus the first and last row;
    statistics on every row."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(seed)
    rows = {0, w.rows - 1}
    for t0 in range(0, w.rows, 256):
        n = min(256, w.rows - t0)
        rows.update(int(t0 + v) for v in rng.choice(n, size=min(2, n), replace=False))
    rows = np.array(sorted(rows))
    ref_stats = oracle.row_stats(x_np)
    ref_out = oracle.soft_embed(np.ascontiguousarray(x_np[rows]), w.vocab_start, w.vocab_end,
                                bits[w.vocab_start:w.vocab_end], w.gamma)
    par = parity(w, got, ref_stats, ref_out, rows)
    # statistics of every row
    am_bad = int(np.sum(got["argmax"] != ref_stats["argmax"]))
    d_h = float(np.max(np.abs(got["entropy"] - ref_stats["entropy"])))
    par["stats_all_rows"] = {"argmax_mismatches": am_bad, "max_abs_d_entropy_nats": d_h,
                             "max_abs_d_row_max": float(np.max(np.abs(
                                 got["max"].astype(np.float64) - ref_stats["max"])))}
    par["pass"] = bool(par["pass"] and am_bad == 0 and d_h <= ENTROPY_TOL)
    return par


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="full", choices=["full", "rank", "conv", "batch", "tiny"])
    ap.add_argument("--path", default="auto",
                    choices=["auto", "step", "step_onepass", "onepass", "unfused", "staged",
                             "fused", "step_onepass_fp8"],
                    help="how the step runs (auto: the workload's fastest whole-step path; "
                         "step_onepass_fp8, the e4m3-table step, with --minimal only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--side-workloads", default="rank,conv,batch",
                    help="comma-separated workloads timed beside the main one on their fastest "
                         "paths ('' for none)")
    ap.add_argument("--minimal", action="store_true",
                    help="only the headline steps (warmup, timed steps, per-kernel times): for "
                         "profiling runs; no side paths, side workloads or CPU baseline")
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
    from diffusion_self_conditioning_amd import workloads as wl

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    w = wl.get(args.workload)
    path = BEST_PATH[w.name] if args.path == "auto" else args.path
    whole = w.vocab_start == 0 and w.vocab_end == w.vocab
    if path == "step_onepass_fp8" and not args.minimal:
        print("--path step_onepass_fp8 (another numerical contract: the e4m3 table) runs with "
              "--minimal only; the full run reports it under fp8_table", file=sys.stderr)
        sys.exit(2)
    if path == "onepass" and not whole:
        print("--path onepass needs a workload whose slice is the whole vocabulary (its row "
              "statistics are those of the slice)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    say(f"generating {w.name} inputs")
    x_np = wl.make_logits(w)
    bits, _ = wl.make_table(w)
    st = Step(w, x_np, bits, dev)
    L, d = w.rows, w.d
    flops = w.flops()

    if args.minimal:
        say(f"warmup {W}, {K} timed steps ({path})")
        rep = step_report(st, path, K, W)
        print(json.dumps({"metric": METRIC, "value": rep["gflops"], "unit": "GFLOP/s",
                          "n_gpus": 1, "steps": K, "warmup": W,
                          "ms_per_step": rep["ms_per_step"], "minimal": True,
                          "config": {"workload": w.name, "path": path,
                                     "table": "e4m3" if path.endswith("_fp8") else "bf16"},
                          "kernel_us": rep["kernel_us"],
                          "gaps_between_kernels_us": rep["gaps_between_kernels_us"],
                          "marked_step_us": rep["marked_step_us"], "roofline": rep["roofline"]}),
              flush=True)
        return

    # every path on the same inputs, event-timed as whole steps, after the GPU has been
    # brought to its sustained state under this load
    say("paths")
    condition(st, path)
    side = {}
    outs = {}
    for p in ("step", "step_onepass", "unfused", "staged", "fused") + (("onepass",) if whole
                                                                       else ()):
        o = torch.empty_like(st.out)
        side[p + "_step_us"] = round(event_time_us(lambda: st.call(p, o), K, W), 2)
        outs[p] = o
    ref = outs["step"]
    for p in ("unfused", "staged", "fused"):
        side[p + "_equals_step_output"] = bool(torch.equal(outs[p], ref))
    side["step_onepass_rel_diff_vs_step"] = float(
        (outs["step_onepass"].double() - ref.double()).norm() / ref.double().norm())
    del outs, o

    # the headline: W warmup steps, K timed steps of the chosen path
    say(f"warmup {W}, {K} timed steps ({path})")
    main_rep = step_report(st, path, K, W)
    got = fetch(st)           # the last timed step's outputs (the marker pass repeats it)

    # side measurements on the same inputs
    say("side measurements")
    acc_side = None
    if L % 256 == 0:
        nc = L // 256
        acc = {"acc": torch.zeros(L, dtype=torch.uint8, device=dev),
               "prev": torch.full((L,), -1, dtype=torch.int32, device=dev),
               "sc": torch.zeros(nc, dtype=torch.int32, device=dev),
               "stc": torch.zeros(nc, dtype=torch.int32, device=dev),
               "new": torch.empty(L, dtype=torch.uint8, device=dev),
               "conv": torch.empty(nc, dtype=torch.uint8, device=dev)}

        def accept_step():
            B.se_accept_converge(st.ent, st.am, 256, 8.0, 3, 0.05, 64, acc["acc"], acc["prev"],
                                 acc["sc"], acc["stc"], acc["new"], acc["conv"])

        acc_side = {"accept_converge_us": round(event_time_us(accept_step, K, W), 2),
                    "canvases": nc, "accepted_last_step": int(acc["new"].sum().item())}
        del acc
    parts4 = torch.randn((4, L, d), device=dev)
    red_f = torch.empty((L, d), device=dev)
    red_b = torch.empty((L, d), dtype=torch.bfloat16, device=dev)
    red_us = event_time_us(lambda: B.se_reduce_partials(parts4, out=red_f, out_bf16=red_b), K, W)
    red_side = {"reduce_partials_us": round(red_us, 2), "parts": 4,
                "gbs": round((4 * 4 + 4 + 2) * L * d / (red_us * 1e-6) / 1e9, 1)}
    del parts4, red_f, red_b

    # the e4m3 form of the shard (quantized once, untimed): the whole step against it
    codes = torch.empty((w.k, d), dtype=torch.uint8, device=dev)
    wscale = torch.empty(w.k, device=dev)
    B.se_quantize_table_fp8(st.shard, codes, wscale)
    out8 = torch.empty_like(st.out)
    s8 = [torch.empty(L, device=dev) for _ in range(3)] + [
        torch.empty(L, device=dev, dtype=torch.int32)]
    us_s8 = event_time_us(lambda: B.se_soft_embed_step_fp8(
        st.x, w.vocab_start, w.vocab_end, codes, wscale, w.gamma, out8, *s8, st.wss), K, W,
        settle_ms=60.0)
    out8o = torch.empty_like(st.out)
    s8o = [torch.empty(L, device=dev) for _ in range(3)] + [
        torch.empty(L, device=dev, dtype=torch.int32)]
    us_s8o = event_time_us(lambda: B.se_soft_embed_step_onepass_fp8(
        st.x, w.vocab_start, w.vocab_end, codes, wscale, w.gamma, out8o, *s8o, st.ws1), K, W,
        settle_ms=60.0)
    s8_bytes = 4 * L * w.vocab + w.k * d + 4 * w.k + 4 * L * d + 16 * L
    us_q = event_time_us(lambda: B.se_quantize_table_fp8(st.shard, codes, wscale), 3, 1)

    def fp8_roof(us):
        # whole-step bytes (logits once, codes and scales once, outputs) or FLOP, whichever
        # binds at the nominal peaks (the FLOP, here)
        r = roofline(flops, s8_bytes, us)
        r.update({"algorithmic_bytes": s8_bytes, "algorithmic_flops": flops})
        return r
    fp8_side = {"step_us": round(us_s8, 2), "gflops_step": round(flops / (us_s8 * 1e-6) / 1e9, 2),
                "roofline_step": fp8_roof(us_s8),
                "onepass_step_us": round(us_s8o, 2),
                "onepass_gflops_step": round(flops / (us_s8o * 1e-6) / 1e9, 2),
                "onepass_roofline_step": fp8_roof(us_s8o),
                "quantize_shard_us": round(us_q, 2),
                "note": "a different numerical contract (the dequantized e4m3 table); not value. "
                        "step: se_soft_embed_step_fp8 (two passes over the logits, the codes "
                        "converted to bf16 in LDS); onepass_step: se_soft_embed_step_onepass_fp8 "
                        "(one read, row scales carried by the staged probabilities, codes read "
                        "in place)"}
    del codes, wscale, out8, s8, out8o, s8o

    # cold step, and the box's achievable ceilings beside the peaks
    scrub = torch.empty(1 << 28, device=dev)
    cold = []
    for k in range(5):
        scrub.fill_(float(k))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st.call(path)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    src = torch.ones(1 << 28, device=dev)
    copy_us = event_time_us(lambda: scrub.copy_(src), 10, 3)
    del scrub, src
    ga = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)
    gb = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)
    mm_us = event_time_us(lambda: torch.mm(ga, gb), 10, 5)
    del ga, gb
    # the vendor GEMM at the contraction's own shape: the slice's bf16 probabilities
    # [rows, K] (contiguous) times the bf16 shard [K, d], fp32 output
    B.se_row_stats(st.x, st.mx, st.lse, st.ent, st.am)
    pr = torch.empty((L, w.vocab), device=dev, dtype=torch.bfloat16)
    B.se_probs_bf16(st.x, st.lse, w.vocab_start, w.vocab_end, pr)
    pa = pr[:, w.vocab_start:w.vocab_end].contiguous()
    del pr
    pb = st.shard.view(torch.bfloat16)
    vend_us = event_time_us(lambda: torch.mm(pa, pb, out_dtype=torch.float32), 10, 5)
    del pa, pb
    # a read-only stream: the full-width statistics pass over this workload's logits
    stats_us = event_time_us(lambda: B.se_row_stats(st.x, st.mx, st.lse, st.ent, st.am), K, W,
                             settle_ms=30)
    # the matrix cores alone: one workgroup per CU, 8 chains of 32x32x16 bf16 MFMAs per wave
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    loop_iters = 20000
    loop_out = torch.empty(cus * 256, device=dev)
    loop_us = event_time_us(lambda: B.se_mfma_loop(loop_out, cus, loop_iters), 10, 3,
                            settle_ms=60)
    loop_flop = cus * 4 * 8 * loop_iters * 32 * 32 * 16 * 2
    del loop_out
    ceilings = {"cold_step_us_median": round(sorted(cold)[len(cold) // 2], 2),
                "hbm_copy_gbs": round(2 * (1 << 28) * 4 / (copy_us * 1e-6) / 1e9, 1),
                "hbm_read_gbs": round((4 * L * w.vocab + 16 * L) / (stats_us * 1e-6) / 1e9, 1),
                "mfma_loop_tflops": round(loop_flop / (loop_us * 1e-6) / 1e12, 1),
                "bf16_gemm_8192_tflops": round(2 * 8192 ** 3 / (mm_us * 1e-6) / 1e12, 1),
                "vendor_gemm_same_shape_us": round(vend_us, 2),
                "vendor_gemm_same_shape_tflops": round(flops / (vend_us * 1e-6) / 1e12, 1),
                "note": "achievable rates on this box beside the nominal peaks: a device copy "
                        "(read + write), the statistics pass (read only), se_mfma_loop (bf16 "
                        "MFMA chains, no memory) and the vendor GEMM"}

    cpu, par = None, None
    if not args.no_cpu_baseline:
        say("cpu baseline and parity (fp64 oracle)")
        cpu, par = cpu_baseline_and_parity(w, x_np, bits, got)
    del st
    torch.cuda.empty_cache()

    # the other workloads, each on its fastest path, with sampled oracle parity
    others = {}
    for name in [n for n in args.side_workloads.split(",") if n and n != w.name]:
        ow = wl.get(name)
        say(f"side workload {name}")
        ox = wl.make_logits(ow)
        ob, _ = wl.make_table(ow)
        ost = Step(ow, ox, ob, dev)
        op = BEST_PATH[name]
        rep = step_report(ost, op, K, W)
        rep["config"] = (f"{name}: L_c={ow.rows}, V={ow.vocab}, slice [{ow.vocab_start},"
                         f"{ow.vocab_end}), d={ow.d}, seed {ow.seed}")
        if not args.no_cpu_baseline:
            rep["parity"] = sampled_parity(ow, ox, ob, fetch(ost))
        others[name] = rep
        del ost, ox, ob
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": main_rep["gflops"], "unit": "GFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": main_rep["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: L_c={L} rows, full-width fp32 logits V={w.vocab}, "
                               f"slice [{w.vocab_start},{w.vocab_end}) of a bf16 table "
                               f"[{w.table_rows}, {d}], gamma={w.gamma:.6g}; whole step on "
                               f"{path}",
                   "rows": L, "vocab": w.vocab, "vocab_start": w.vocab_start,
                   "vocab_end": w.vocab_end, "d": d, "seed": w.seed, "path": path,
                   "flops_per_step": flops},
        "steps_per_s": main_rep["steps_per_s"],
        "canvas_steps_per_s": main_rep["canvas_steps_per_s"],
        "step_us_median": main_rep["step_us_median"], "step_us_min": main_rep["step_us_min"],
        "kernel_us": main_rep["kernel_us"],
        "gaps_between_kernels_us": main_rep["gaps_between_kernels_us"],
        "marked_step_us": main_rep["marked_step_us"],
        "roofline": main_rep["roofline"],
        "roofline_step": main_rep["roofline_step"],
        "parity": par,
        "cpu_baseline": cpu,
        "wall_s_timed": main_rep["wall_s_timed"],
        "paths": side,
        "workloads": others,
        "accept_converge": acc_side,
        "reduce_partials": red_side,
        "fp8_table": fp8_side,
        "cold_and_ceilings": ceilings,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
