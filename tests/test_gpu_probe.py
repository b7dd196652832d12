"""The MFMA-rate probe se_mfma_loop on the GPU (MI355X), through the C ABI.

With every operand element equal to u (rounded to bf16 by truncation to its top 16
bits), each MFMA adds 16 u^2 to each of the 16 accumulator elements a lane holds per
chain, so after `iters` MFMAs on each of 8 chains a lane's stored sum is
8 * 16 * iters * 16 u^2 = 2048 iters u^2.  The values below are exact in fp32, so the
check is bit-exact: it pins the probe's arithmetic (and the count of work the rate is
computed from) to the instruction's definition.
"""
import struct
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from diffusion_self_conditioning_amd import _binding as B

DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def bf16_trunc(x: float) -> float:
    bits = struct.unpack("<I", struct.pack("<f", x))[0] & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", bits))[0]


@pytest.mark.parametrize("blocks,iters,unit", [(1, 1, 1.0), (3, 5, 1.0), (7, 9, 0.5),
                                               (2, 7, 3.0), (5, 11, 1.1), (256, 64, -2.0)])
def test_mfma_loop_sums_are_exact(blocks, iters, unit):
    say("mfma loop", blocks, iters, unit)
    out = torch.full((blocks * 256 + 64,), float("nan"), device=DEV)
    B.se_mfma_loop(out, blocks, iters, unit)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    u = bf16_trunc(unit)
    want = np.float32(2048.0 * iters * u * u)
    assert float(want) == 2048.0 * iters * u * u          # exact in fp32
    np.testing.assert_array_equal(got[:blocks * 256], np.full(blocks * 256, want, np.float32))
    assert np.isnan(got[blocks * 256:]).all()             # nothing past the last lane
