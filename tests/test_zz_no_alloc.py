"""se_soft_embed_step_noalloc against se_soft_embed_step (MI355X).

The no-allocation entry point runs se_soft_embed_step with the library's own device array as
its workspace, so on the same inputs its outputs must be those of the call with a caller
workspace, bit for bit.  Two calls in a row on one GPU, the second with a smaller input (the
array keeps the first call's contents), then a shape past the array, which is rejected with
nothing launched.
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


def inputs(L, V, s, e, d, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((L, V), dtype=np.float32) * np.float32(3.0))
    x[np.arange(L), rng.integers(0, V, L)] += np.float32(8.0)
    w = wl.fp32_to_bf16_bits(rng.standard_normal((e - s, d), dtype=np.float32)
                             * np.float32(0.02))
    return torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV)


def outputs(L, d):
    f = dict(device=DEV, dtype=torch.float32)
    return (torch.full((L, d), float("nan"), **f), torch.empty(L, **f), torch.empty(L, **f),
            torch.empty(L, **f), torch.empty(L, device=DEV, dtype=torch.int32))


def compare(L, V, s, e, d, seed, gamma):
    say(f"noalloc vs step: L={L} V={V} slice [{s},{e}) d={d}")
    x, w = inputs(L, V, s, e, d, seed)
    ref = outputs(L, d)
    ws = api.staged_workspace(L, s, e, d, DEV)
    B.se_soft_embed_step(x, s, e, w, gamma, *ref, ws)
    got = outputs(L, d)
    B.se_soft_embed_step_noalloc(x, s, e, w, gamma, *got)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    assert torch.isfinite(got[0]).all()


def test_noalloc_equals_step_on_two_calls_then_rejects_past_its_array():
    max_bytes = B.se_soft_embed_step_noalloc_max_bytes()
    # the one-rank shape (about 95 MiB of workspace), then a smaller, ragged one
    assert B.se_soft_embed_staged_workspace_bytes(256, 65536, 131072, 2816) <= max_bytes
    compare(256, 262144, 65536, 131072, 2816, 1, float(wl.SQRT_D))
    compare(300, 20000, 4096, 12296, 520, 2, 5.0)
    # past the array: SE_ERR_WORKSPACE, outputs untouched
    L, V, d = 256, 262144, 2816
    assert B.se_soft_embed_staged_workspace_bytes(L, 0, V, d) > max_bytes
    x = torch.zeros((L, V), device=DEV)
    w = torch.zeros((V, d), device=DEV, dtype=torch.int16)
    out = outputs(L, d)
    out[0].fill_(7.0)
    with pytest.raises(B.SoftEmbedError) as ei:
        B.se_soft_embed_step_noalloc(x, 0, V, w, 1.0, *out)
    assert ei.value.status == B.SE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out[0] == 7.0)
