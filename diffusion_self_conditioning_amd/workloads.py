"""Seeded synthetic inputs for the self-conditioning soft embedding.

This module only *draws* inputs: logits rows, planted maxima and the bf16
embedding table.  It holds none of the method's arithmetic (no softmax, no
contraction, no entropy) and is the one piece of Python that both the fp64
oracle and the HIP path are fed from, so that both sides see identical bytes.

Shapes follow the pages (calvarado04.com, "Where the shapes stop agreeing"):
vocabulary V = 262,144, hidden size d = 2,816, canvas length 256, and the
four-way vocab shard of 65,536 rows.  The embedding table is padded to
262,400 rows for the one-rank workload, as a vocab-parallel layout pads its
shards ("The fix", last paragraph: padded rows carry no probability mass).

Randomness: numpy PCG64 via ``SeedSequence(seed).spawn(3)``; child 0 draws
logits, child 1 the planted indices, child 2 the table.  Seeds equal the
workload number so runs are reproducible and recorded.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_logits", "make_table",
           "fp32_to_bf16_bits", "bf16_bits_to_fp32", "one_hot_logits",
           "uniform_logits"]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    rows: int            # L: canvas positions (rows of the logits matrix)
    vocab: int           # V: full logits width (softmax is over all of it)
    d: int               # hidden size
    vocab_start: int     # s: first vocab id of this call's slice
    vocab_end: int       # e: one past the last vocab id of the slice
    table_rows: int      # rows of the (possibly padded) embedding table
    gamma: float         # learned normaliser, passed to both sides as fp32
    logit_std: float     # std-dev of the Gaussian logits
    plant: str           # "margin8" | "value20" | "none"
    table_fp32: bool     # True: the table is fp32 (the GPU gets its bf16 rounding)
    w_std: float = 0.02

    @property
    def k(self) -> int:
        return self.vocab_end - self.vocab_start

    def flops(self) -> int:
        """2 * L * (e - s) * d multiply-add FLOP of one slice contraction."""
        return 2 * self.rows * self.k * self.d

    def diffuse(self) -> "Workload":
        """Same seed and shape with no planted maximum (a diffuse distribution)."""
        return replace(self, name=self.name + "-diffuse", plant="none")

    def with_rows(self, rows: int) -> "Workload":
        return replace(self, name=f"{self.name}-L{rows}", rows=rows)


SQRT_D = float(np.float32(math.sqrt(2816.0)))

# Workload table.  "tiny" is the small case the oracle finishes in seconds;
# "rank" is one tensor-parallel rank's share at its real shape (T = 4, the
# second of four shards); "full" the whole vocabulary; "conv" a near-converged
# canvas; "batch" eight 256-position canvases at once.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 4096, 256, 0, 4096, 4096, 16.0, 3.0,
                     "margin8", True),
    "rank": Workload("rank", 2, 256, 262144, 2816, 65536, 131072, 262400,
                     SQRT_D, 3.0, "margin8", False),
    "full": Workload("full", 3, 256, 262144, 2816, 0, 262144, 262144,
                     SQRT_D, 3.0, "margin8", False),
    "conv": Workload("conv", 4, 256, 262144, 2816, 0, 262144, 262144,
                     SQRT_D, 1.0, "value20", False),
    "batch": Workload("batch", 5, 2048, 262144, 2816, 0, 262144, 262144,
                      SQRT_D, 3.0, "margin8", False),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(3)]


def make_logits(w: Workload, plant: str | None = None) -> np.ndarray:
    """fp32 logits [rows, vocab], row-major, ld = vocab.

    plant "margin8": index k_i (uniform) is set to the largest other value of
    its row plus 8, which makes it the unique row maximum.
    plant "value20": index k_i is set to exactly 20.0 (rest ~ N(0, 1)).
    """
    plant = w.plant if plant is None else plant
    g_logits, g_plant, _ = _streams(w.seed)
    x = g_logits.standard_normal((w.rows, w.vocab), dtype=np.float32)
    if w.logit_std != 1.0:
        x *= np.float32(w.logit_std)
    ks = g_plant.integers(0, w.vocab, size=w.rows)
    if plant == "margin8":
        for i, k in enumerate(ks):
            row = x[i]
            keep = row[k]
            row[k] = -np.inf
            top = row.max() if w.vocab > 1 else np.float32(0.0)
            row[k] = keep
            row[k] = np.float32(top) + np.float32(8.0)
    elif plant == "value20":
        x[np.arange(w.rows), ks] = np.float32(20.0)
    elif plant != "none":
        raise ValueError(plant)
    return x


def planted_index(w: Workload) -> np.ndarray:
    """The indices k_i that make_logits plants (same stream, same order)."""
    _, g_plant, _ = _streams(w.seed)
    return g_plant.integers(0, w.vocab, size=w.rows)


def fp32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); uint16 bits.

    Used only to synthesise the bf16 embedding table from Gaussian draws.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_table(w: Workload, chunk_rows: int = 1 << 16):
    """Embedding table [table_rows, d].

    Returns (bits, f32): ``bits`` is the uint16 bf16 table the GPU reads;
    ``f32`` is the fp32 table for a fp32 workload (else None).  Rows at or past
    ``vocab`` (the padding of a vocab-parallel layout) are zero.
    """
    _, _, g_w = _streams(w.seed)
    bits = np.zeros((w.table_rows, w.d), dtype=np.uint16)
    f32 = np.zeros((w.table_rows, w.d), dtype=np.float32) if w.table_fp32 else None
    real = min(w.vocab, w.table_rows)
    for r0 in range(0, real, chunk_rows):
        r1 = min(real, r0 + chunk_rows)
        blk = g_w.standard_normal((r1 - r0, w.d), dtype=np.float32)
        blk *= np.float32(w.w_std)
        bits[r0:r1] = fp32_to_bf16_bits(blk)
        if f32 is not None:
            f32[r0:r1] = blk
    return bits, f32


def shard(w: Workload, table_bits: np.ndarray) -> np.ndarray:
    """The local shard a rank holds: table rows [vocab_start, table_rows).

    Row 0 of the shard is vocab id ``vocab_start``; rows past ``vocab_end -
    vocab_start`` belong to the next rank or to padding and must never be read
    by a call on [vocab_start, vocab_end).
    """
    return table_bits[w.vocab_start:]


def one_hot_logits(rows: int, vocab: int, ks, hot: float = 0.0,
                   cold: float = -200.0) -> np.ndarray:
    x = np.full((rows, vocab), np.float32(cold), dtype=np.float32)
    x[np.arange(rows), np.asarray(ks)] = np.float32(hot)
    return x


def uniform_logits(rows: int, vocab: int, value: float = 0.5) -> np.ndarray:
    return np.full((rows, vocab), np.float32(value), dtype=np.float32)
