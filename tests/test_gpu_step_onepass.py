"""GPU parity of se_soft_embed_step_onepass (MI355X), through the C ABI.

The call is se_soft_embed_step's step (statistics of the full-width softmax, the slice's
soft embedding against them) from one read of the logits: every range of a row is
normalised against its own maximum and the ranges merge afterwards.  Its oracle is the
full-row oracle: oracle.row_stats over all columns and oracle.soft_embed over [s, e).
Bars as the two-pass path:
  argmax, row max          bit-exact
  log-sum-exp              |d| <= 2e-6 * max(1, |lse|)
  entropy                  |d| <= 1e-4 nats
  soft embedding           relative Frobenius <= 5e-3
Cases: the whole vocabulary as the slice, slices at the start, middle and end of the
row, slices of 1 and 63 positions, vocabularies and slice ends that are not multiples
of 4 (ranges with scalar heads and tails), whole and partial 256-row tiles, a row
maximum in the slice or outside it, one-hot / uniform / wide-range / tied rows, the
empty slice and split ranges too long for the sweep (both the two-pass step, bit for
bit), repeatability, and the one-rank workload at full size.  Two cases run the rows'
range merge inside the contraction (one wave of workgroups; the workgroups of the
splits one block shorter each merge 8 rows): 13 rows on 16 merging waves, and 511 rows
over 2 x 3 output tiles with ragged rows and columns.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from diffusion_self_conditioning_amd import workloads as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from diffusion_self_conditioning_amd import _binding as B
    from diffusion_self_conditioning_amd import api

DEV = "cuda:0"
GATE = 5e-3


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rel_fro(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def table(rows, d, seed):
    rng = np.random.default_rng(seed)
    bits = wl.fp32_to_bf16_bits((rng.standard_normal((rows + 24, d)) * 0.02).astype(np.float32))
    bits[rows:] = 0x7FC0                        # shard rows past the slice: NaN, never read
    return bits


def dev_logits(x):
    """x in a buffer whose row pitch is a multiple of 4, padded with huge values past V."""
    L, V = x.shape
    ld = ((V + 3) // 4) * 4
    buf = np.full((L, ld), np.float32(1e30), np.float32)
    buf[:, :V] = x
    return dev(buf)[:, :V]


def step1(x_t, s, e, w_t, gamma):
    out, mx, lse, ent, am = api.soft_embed_step(x_t, s, e, w_t, gamma, onepass=True)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), dict(max=mx.cpu().numpy(), lse=lse.cpu().numpy(),
                                    entropy=ent.cpu().numpy(), argmax=am.cpu().numpy()))


def check(x, s, e, bits, gamma, rows=None):
    out, g = step1(dev_logits(x), s, e, dev(bits), gamma)
    xr = x if rows is None else np.ascontiguousarray(x[rows])
    if rows is not None:
        out = out[rows]
        g = {k: v[rows] for k, v in g.items()}
    r = oracle.row_stats(xr)
    np.testing.assert_array_equal(g["argmax"], r["argmax"])
    np.testing.assert_array_equal(g["max"].astype(np.float64), r["max"])
    tol = 2e-6 * np.maximum(1.0, np.abs(r["lse"]))
    assert np.all(np.abs(g["lse"] - r["lse"]) <= tol), np.max(np.abs(g["lse"] - r["lse"]) / tol)
    assert np.max(np.abs(g["entropy"] - r["entropy"])) <= 1e-4, \
        np.max(np.abs(g["entropy"] - r["entropy"]))
    if e > s:
        ref = oracle.soft_embed(xr, s, e, bits[:e - s], gamma)
        rf = rel_fro(out, ref)
        say(f"rel_fro {rf:.3e}")
        assert np.all(np.isfinite(out)) and rf <= GATE
    else:
        assert np.count_nonzero(out) == 0
    return out, g


CASES = {
    # name: (L, V, s, e, d, seed)
    "whole-vocab": (16, 4096, 0, 4096, 256, 1),
    "ragged": (17, 20008, 8, 20008, 48, 2),
    "slice-1": (5, 1000, 16, 17, 16, 3),
    "slice-63": (33, 1003, 64, 127, 2816, 4),          # V and e not multiples of 4
    "slice-at-start": (40, 50001, 0, 12345, 64, 5),
    "slice-in-middle": (64, 50000, 12344, 37001, 128, 6),
    "two-row-tiles": (300, 2048, 1024, 2048, 512, 7),
    "many-pre-chunks": (8, 120000, 96000, 100003, 32, 8),
    "whole-tile": (256, 30003, 1000, 13337, 272, 10),   # ping-pong contraction, tail
    "merge-in-contraction": (13, 20008, 8, 20008, 48, 11),
    "merge-row-tiles": (511, 100011, 8, 100008, 520, 12),
    # splits of at least 32 super-steps: three probability stage buffers in the contraction
    "long-splits": (17, 150011, 8, 150003, 2816, 13),
    "long-splits-two-tiles": (300, 160011, 8, 160011, 2816, 14),
    # split ranges of 12,289 .. 16,384 positions: the sweep's 4-wave, 16-group form, with
    # ranges before and after the slice cut at 16,384
    "wide-sweep": (16, 330011, 8, 330008, 2816, 15),
    "wide-sweep-mid-slice": (16, 400011, 40000, 370000, 2816, 16),
}


def merges_in_contraction(L, K, d):
    """Whether the contraction of an L x K x d one-read step carries the range merge: one
    wave of workgroups (256 x 256 tiles times the split count at most the CU count), at
    least two splits, and 8 rows per workgroup of the splits one 128-block shorter."""
    splits = B.se_soft_embed_splits(L, 0, K, d)
    tiles = -(-L // 256) * -(-d // 256)
    kb = -(-K // 128)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if splits < 2 or tiles * splits > cus:
        return False
    longest = -(-kb // splits)
    short = sum(((r + 1) * kb // splits - r * kb // splits) < longest for r in range(splits))
    return short * tiles * 8 >= L


@pytest.mark.parametrize("case", sorted(CASES))
def test_step_onepass_parity(case):
    L, V, s, e, d, seed = CASES[case]
    if case.startswith("merge"):
        assert merges_in_contraction(L, e - s, d), case
    if case.startswith("wide-sweep"):
        bounds = B.se_soft_embed_ranges(L, s, e, d)
        assert 4 * 3072 < max(b - a for a, b in zip(bounds, bounds[1:])) <= 4 * 4096, case
    if case.startswith("long-splits"):
        bounds = B.se_soft_embed_ranges(L, s, e, d)
        assert min((b - a) // 128 for a, b in zip(bounds, bounds[1:])) >= 32, case
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    # half the rows peak inside the slice, half anywhere in the row
    hot = np.where(np.arange(L) % 2 == 0, rng.integers(s, e, L), rng.integers(0, V, L))
    x[np.arange(L), hot] = x.max(axis=1) + 8.0
    say("step_onepass", case, (L, V, s, e, d))
    check(x, s, e, table(e - s, d, seed + 100), 6.5)


@pytest.mark.parametrize("kind", ["one-hot", "uniform", "wide-range", "ramp", "ties"])
def test_step_onepass_special_rows(kind):
    L, V, s, e, d = 8, 30000, 8000, 20003, 64
    rng = np.random.default_rng(21)
    if kind == "one-hot":
        x = wl.one_hot_logits(L, V, rng.integers(0, V, L), hot=30.0, cold=-200.0)
    elif kind == "uniform":
        x = wl.uniform_logits(L, V, 0.75)
    elif kind == "wide-range":
        x = (rng.standard_normal((L, V)) * 1000.0).astype(np.float32)
    elif kind == "ramp":            # the maximum grows across every range; the slice's
        # mass, about e^-40, stays within fp32 range (a slice whose true share of the
        # softmax is below fp32's smallest value has a zero fp32 embedding on any path)
        x = np.tile(np.linspace(-60.0, 60.0, V, dtype=np.float32), (L, 1))
    else:                           # equal maxima in several ranges: the first one wins
        x = np.zeros((L, V), np.float32)
        x[:, [7, 9000, 20001, 29999]] = 4.0
    say("step_onepass special", kind)
    check(x, s, e, table(e - s, d, 22), 3.0)


def test_step_onepass_agrees_with_the_two_pass_step():
    """Argmax and max bitwise the two-pass step's; lse, entropy and the embedding within
    rounding of them."""
    L, V, s, e, d = 48, 40000, 16000, 28000, 256
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 7.0
    x_t, w_t = dev_logits(x), dev(table(e - s, d, 24))
    a = api.soft_embed_step(x_t, s, e, w_t, 2.0, onepass=True)
    b = api.soft_embed_step(x_t, s, e, w_t, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[4], b[4])
    l1, l2 = a[2].cpu().numpy(), b[2].cpu().numpy()
    assert np.all(np.abs(l1 - l2) <= 2e-6 * np.maximum(1.0, np.abs(l2)))
    assert np.max(np.abs(a[3].cpu().numpy() - b[3].cpu().numpy())) <= 1e-4
    assert rel_fro(a[0].cpu().numpy(), b[0].cpu().numpy()) <= GATE


def test_step_onepass_repeatable():
    rng = np.random.default_rng(25)
    x_t = dev((rng.standard_normal((64, 30000)) * 3).astype(np.float32))
    w_t = dev(table(10000, 128, 26))
    a = api.soft_embed_step(x_t, 4000, 14000, w_t, 2.0, onepass=True)
    b = api.soft_embed_step(x_t, 4000, 14000, w_t, 2.0, onepass=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("shape", [(8, 512, 16, 16, 16), (4096, 110000, 0, 110000, 1024)],
                         ids=["empty-slice", "long-split-ranges"])
def test_step_onepass_falls_back_to_the_two_pass_step(shape):
    """An empty slice, or split ranges longer than 24,576 positions (4096 rows x 4
    n-tiles are 64 tiles; 4 splits of 27,520 positions): the call is se_soft_embed_step,
    bit for bit."""
    L, V, s, e, d = shape
    rng = np.random.default_rng(27)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x_t, w_t = dev(x), dev(table(e - s, d, 28))
    nb1 = B.se_soft_embed_step_onepass_workspace_bytes(L, V, s, e, d)
    nb2 = B.se_soft_embed_staged_workspace_bytes(L, s, e, d)
    assert nb1 == nb2
    say("step_onepass fallback", shape)
    a = api.soft_embed_step(x_t, s, e, w_t, 1.5, onepass=True)
    b = api.soft_embed_step(x_t, s, e, w_t, 1.5)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_step_onepass_full_size_rank():
    w = wl.get("rank")
    say("step_onepass full-size rank: inputs")
    x = wl.make_logits(w)
    bits, _ = wl.make_table(w)
    x_t, tab_t = dev(x), dev(bits)
    shard = tab_t[w.vocab_start:]
    say("step_onepass full-size rank: gpu")
    a = api.soft_embed_step(x_t, w.vocab_start, w.vocab_end, shard, w.gamma, onepass=True)
    b = api.soft_embed_step(x_t, w.vocab_start, w.vocab_end, shard, w.gamma, onepass=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    am = a[4].cpu().numpy()
    np.testing.assert_array_equal(am, wl.planted_index(w))
    rows = np.array([0, 1, 128, 255])
    xr = np.ascontiguousarray(x[rows])
    r = oracle.row_stats(xr)
    np.testing.assert_array_equal(a[1].cpu().numpy()[rows].astype(np.float64), r["max"])
    lse = a[2].cpu().numpy()[rows]
    assert np.all(np.abs(lse - r["lse"]) <= 2e-6 * np.maximum(1.0, np.abs(r["lse"])))
    assert np.max(np.abs(a[3].cpu().numpy()[rows] - r["entropy"])) <= 1e-4
    ref = oracle.soft_embed(xr, w.vocab_start, w.vocab_end, bits[w.vocab_start:w.vocab_end],
                            w.gamma)
    rf = rel_fro(a[0].cpu().numpy()[rows], ref)
    say(f"rel_fro {rf:.3e}")
    assert rf <= GATE
