"""The calls under HIP graph capture (MI355X), through the C ABI.

The library allocates nothing, never synchronises and never reads device data on the
host, so a caller can capture a whole step into a graph (torch.cuda.graph drives the
capture on its own stream); se_soft_embed_step_noalloc, the entry point for callers that
cannot allocate, is captured too.  Every replay here is checked bit for bit against an eager
call on the same inputs; the inputs change between replays (new logits copied into the
captured buffer), with the program's own eager work and synchronisations in between.
"""
import sys

import numpy as np
import pytest
import torch

from diffusion_self_conditioning_amd import workloads as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from diffusion_self_conditioning_amd import _binding as B
    from diffusion_self_conditioning_amd import api

DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("which", ["step", "step_onepass", "staged", "step_held_slice", "step_fp8",
                                   "step_onepass_fp8", "step_noalloc"])
def test_captured_step_replays_match_eager_calls(which):
    L, V, s, e, d = 256, 30000, 8000, 20000, 512
    if which == "step_held_slice":          # two whole 16,384-position groups: kept in registers
        V, s, e = 65536, 16384, 49152
    rng = np.random.default_rng(51)
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s, d)) * 0.02).astype(np.float32))
    w_t = torch.from_numpy(tab).to(DEV)
    x_t = torch.empty((L, V), device=DEV)
    f = dict(device=DEV, dtype=torch.float32)
    out = torch.empty((L, d), **f)
    mx, lse, ent = torch.empty(L, **f), torch.empty(L, **f), torch.empty(L, **f)
    am = torch.empty(L, device=DEV, dtype=torch.int32)
    if which in ("step_onepass", "step_onepass_fp8"):
        ws = api.step_onepass_workspace(L, V, s, e, d, DEV)
    else:
        ws = api.staged_workspace(L, s, e, d, DEV)
    if which.endswith("fp8"):               # e4m3 table, quantized once before the capture
        codes, wscale = api.quantize_table_fp8(w_t)
        torch.cuda.synchronize()

    def call():
        if which in ("step", "step_held_slice"):
            B.se_soft_embed_step(x_t, s, e, w_t, 2.0, out, mx, lse, ent, am, ws)
        elif which == "step_noalloc":           # the library's own workspace: nothing to pass
            B.se_soft_embed_step_noalloc(x_t, s, e, w_t, 2.0, out, mx, lse, ent, am)
        elif which == "step_onepass":
            B.se_soft_embed_step_onepass(x_t, s, e, w_t, 2.0, out, mx, lse, ent, am, ws)
        elif which == "step_fp8":
            B.se_soft_embed_step_fp8(x_t, s, e, codes, wscale, 2.0, out, mx, lse, ent, am, ws)
        elif which == "step_onepass_fp8":
            B.se_soft_embed_step_onepass_fp8(x_t, s, e, codes, wscale, 2.0, out, mx, lse, ent, am,
                                             ws)
        else:                                   # statistics call, then the staged contraction
            B.se_row_stats(x_t, mx, lse, ent, am)
            B.se_soft_embed_staged(x_t, lse, s, e, w_t, 2.0, out, ws)

    def new_logits(seed):
        r = np.random.default_rng(seed)
        x = (r.standard_normal((L, V)) * 3).astype(np.float32)
        x[np.arange(L), r.integers(0, V, L)] += 8.0
        x_t.copy_(torch.from_numpy(x))
        torch.cuda.synchronize()

    new_logits(0)
    call()                                      # eager first (fills the per-device CU cache)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("capture", which)
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(1, 4):
        new_logits(rep)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, mx, lse, ent, am)]
        call()                                  # eager on the same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, (out, mx, lse, ent, am)):
            assert torch.equal(a, b), f"replay {rep} differs from the eager call"
        # some eager work of the program between replays
        torch.cuda.synchronize()
