"""Oracle of the on-device sum of per-rank partials -- TEST INFRASTRUCTURE (only
tests/, the smoke check and the benchmark's CPU leg use it).

calvarado04.com/tag/vllm, section "The fix": E^sc = gamma * sum_r S^(r), one
all-reduce over the ranks, result in the embedding dtype.  The library adds the
parts in the order r = 0 .. T-1 in fp32, so this oracle does exactly that with
numpy float32 additions (IEEE round to nearest even per add), then rounds the
sum to bfloat16 (nearest even) with the fp64 rounding routine of the oracle.
"""
from __future__ import annotations

import numpy as np

from . import round_bf16


def reduce_partials(parts: np.ndarray):
    """parts: float32 [T, rows, d].  Returns (fp32 sum, bf16 bit patterns as uint16)."""
    p = np.asarray(parts, dtype=np.float32)
    acc = p[0].copy()
    for r in range(1, p.shape[0]):
        acc = np.add(acc, p[r], dtype=np.float32)
    rounded = round_bf16(acc.astype(np.float64)).astype(np.float32)
    bits = (rounded.view(np.uint32) >> 16).astype(np.uint16)
    return acc, bits
