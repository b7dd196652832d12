"""GPU parity of the one-pass soft embedding (se_soft_embed_onepass) and the merge of
slice results (se_merge_slices) against the fp64 oracle, through the C ABI (MI355X).

The one-pass call over [s, e) is the soft embedding and the row statistics of the
softmax over that slice alone, so its oracle is the ordinary oracle applied to the
logits columns [s, e) as a matrix of their own.  Merging the slices of a partition
must give the full-row oracle.  Bars as the two-pass path:
  argmax, row max          bit-exact
  log-sum-exp              |d| <= 2e-6 * max(1, |lse|)
  entropy                  |d| <= 1e-4 nats
  soft embedding           relative Frobenius <= 5e-3
Cases: whole vocabularies and slices of 1, 63 and 4097 positions; ragged rows and
hidden sizes; 1, a few and 256 split ranges; rows whose maximum sits in any range;
one-hot rows, uniform rows, rows with a dynamic range of thousands of nats; a
near-converged canvas; the rows' range merge inside the contraction (one wave of
workgroups, the workgroups of the splits one block shorter merging 8 rows each); and at
full size the whole vocabulary and a four-rank merge.
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


def onepass(x_t, s, e, w_t, gamma):
    out, mx, lse, ent, am = api.soft_embed_onepass(x_t, s, e, w_t, gamma)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), dict(max=mx.cpu().numpy(), lse=lse.cpu().numpy(),
                                    entropy=ent.cpu().numpy(), argmax=am.cpu().numpy()))


def check_stats(g, r, offset=0):
    np.testing.assert_array_equal(g["argmax"], r["argmax"] + offset)
    np.testing.assert_array_equal(g["max"].astype(np.float64), r["max"])
    tol = 2e-6 * np.maximum(1.0, np.abs(r["lse"]))
    assert np.all(np.abs(g["lse"] - r["lse"]) <= tol), np.max(np.abs(g["lse"] - r["lse"]) / tol)
    assert np.max(np.abs(g["entropy"] - r["entropy"])) <= 1e-4, \
        np.max(np.abs(g["entropy"] - r["entropy"]))


def check_slice(x, s, e, shard_bits, gamma, rows=None):
    """GPU one-pass over [s, e) of x against the oracle over the columns [s, e)."""
    x_t = dev(x)
    out, g = onepass(x_t, s, e, dev(shard_bits), gamma)
    xs = np.ascontiguousarray(x[:, s:e] if rows is None else x[rows, s:e])
    if rows is not None:
        out = out[rows]
        g = {k: v[rows] for k, v in g.items()}
    check_stats(g, oracle.row_stats(xs), offset=s)
    ref = oracle.soft_embed(xs, 0, e - s, shard_bits, gamma)
    r = rel_fro(out, ref)
    say(f"rel_fro {r:.3e}")
    assert np.all(np.isfinite(out)) and r <= GATE
    return out, g


def table(rows, d, seed):
    rng = np.random.default_rng(seed)
    return wl.fp32_to_bf16_bits((rng.standard_normal((rows, d)) * 0.02).astype(np.float32))


CASES = {
    # name: (L, V, s, e, d, seed)
    "tiny-full": (16, 4096, 0, 4096, 256, 1),
    "ragged": (17, 20008, 8, 20008, 48, 2),
    "slice-1": (5, 1000, 16, 17, 16, 3),
    "slice-63": (33, 1000, 64, 127, 2816, 4),
    "slice-4097": (255, 8200, 8, 4105, 272, 5),
    "two-row-tiles": (300, 2048, 0, 2048, 512, 6),
    "256-splits": (16, 65536, 0, 65536, 256, 7),
    "whole-tile-ragged": (256, 20008, 8, 12353, 264, 8),  # ping-pong contraction, tail
    "two-whole-tiles": (512, 4104, 0, 4104, 128, 9),
    # the range merge inside the contraction: 13 rows on 16 merging waves; 511 rows over
    # 2 x 3 output tiles with ragged rows and columns
    "merge-in-contraction": (13, 20008, 8, 20008, 48, 11),
    "merge-row-tiles": (511, 100008, 8, 100008, 520, 12),
    # split ranges of 12,289 .. 16,384 positions: the sweep's 4-wave, 16-group form
    "wide-sweep": (16, 330008, 8, 330008, 2816, 13),
}


def merges_in_contraction(L, K, d):
    """Whether the contraction of an L x K x d one-pass call carries the range merge: one
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
def test_onepass_parity(case):
    L, V, s, e, d, seed = CASES[case]
    if case.startswith("merge"):
        assert merges_in_contraction(L, e - s, d), case
    if case == "wide-sweep":
        bounds = B.se_soft_embed_ranges(L, s, e, d)
        assert 4 * 3072 < max(b - a for a, b in zip(bounds, bounds[1:])) <= 4 * 4096, case
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    # plant each row's maximum in a different place (any split range may hold it)
    hot = rng.integers(s, e, L)
    x[np.arange(L), hot] = x.max(axis=1) + 8.0
    say("onepass", case, (L, V, s, e, d))
    check_slice(x, s, e, table(e - s, d, seed + 100), 7.5)


@pytest.mark.parametrize("kind", ["one-hot", "uniform", "wide-range", "ramp", "ties"])
def test_onepass_special_rows(kind):
    L, V, d = 8, 12000, 64
    rng = np.random.default_rng(11)
    if kind == "one-hot":
        x = wl.one_hot_logits(L, V, rng.integers(0, V, L), hot=30.0, cold=-200.0)
    elif kind == "uniform":
        x = wl.uniform_logits(L, V, 0.75)
    elif kind == "wide-range":
        x = (rng.standard_normal((L, V)) * 1000.0).astype(np.float32)
    elif kind == "ramp":            # the maximum grows across every split range
        x = np.tile(np.linspace(-500.0, 500.0, V, dtype=np.float32), (L, 1))
    else:                           # equal maxima in several ranges: the first one wins
        x = np.zeros((L, V), np.float32)
        x[:, [7, 5000, 11999]] = 4.0
    say("onepass special", kind)
    check_slice(x, 0, V, table(V, d, 12), 3.0)


@pytest.mark.parametrize("shape", [(768, 100000, 2816), (4096, 65536, 1024), (4096, 110000, 1024)],
                         ids=["eight-waves-14336", "eight-waves-16384", "read-twice"])
def test_onepass_long_split_ranges(shape):
    """Long split ranges: 768 rows x 11 n-tiles -> 7 splits of 14,336 positions and 4096
    rows x 4 n-tiles -> 4 splits of 16,384 take the register sweep with 8 waves per range;
    110,000 positions over 4096 rows x 4 n-tiles -> 4 splits of 27,520, longer than 8 waves
    hold (24,576), take the workgroup-per-range sweep, whose second pass reads the logits
    again."""
    L, V, d = shape
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 9.0
    say("onepass long ranges", shape)
    check_slice(x, 0, V, table(V, d, 18), 2.5, rows=np.array([0, 1, L // 2, L - 1]))


def test_onepass_agrees_with_the_two_pass_path():
    """Over the whole vocabulary the one-pass statistics are se_row_stats' (argmax and max
    bitwise) and the embedding is within bf16 rounding of the fused call's."""
    w = wl.get("tiny")
    x = wl.make_logits(w)
    bits, _ = wl.make_table(w)
    x_t, w_t = dev(x), dev(bits)
    out1, g = onepass(x_t, 0, w.vocab, w_t, w.gamma)
    mx, lse, ent, am = api.row_stats(x_t)
    out2 = api.soft_embed(x_t, lse, 0, w.vocab, w_t, w.gamma, fused=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g["argmax"], am.cpu().numpy())
    np.testing.assert_array_equal(g["max"], mx.cpu().numpy())
    l2 = lse.cpu().numpy()
    assert np.all(np.abs(g["lse"] - l2) <= 2e-6 * np.maximum(1.0, np.abs(l2)))
    assert np.max(np.abs(g["entropy"] - ent.cpu().numpy())) <= 1e-4
    assert rel_fro(out1, out2.cpu().numpy()) <= GATE


def test_onepass_repeatable():
    rng = np.random.default_rng(13)
    x_t = dev((rng.standard_normal((64, 30000)) * 3).astype(np.float32))
    w_t = dev(table(30000, 128, 14))
    a = api.soft_embed_onepass(x_t, 0, 30000, w_t, 2.0)
    b = api.soft_embed_onepass(x_t, 0, 30000, w_t, 2.0)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def merge(parts):
    """se_merge_slices over a list of one-pass results (torch tensors)."""
    outs = torch.stack([p[0] for p in parts])
    st = [torch.stack([p[k] for p in parts]).contiguous() for k in range(1, 5)]
    n, d = outs.shape[1], outs.shape[2]
    out = torch.full((n, d), float("nan"), device=DEV)
    f = dict(device=DEV, dtype=torch.float32)
    mx, lse, ent = torch.empty(n, **f), torch.empty(n, **f), torch.empty(n, **f)
    am = torch.empty(n, device=DEV, dtype=torch.int32)
    B.se_merge_slices(outs, st[0], st[1], st[2], st[3], out, mx, lse, ent, am)
    torch.cuda.synchronize()
    return out.cpu().numpy(), dict(max=mx.cpu().numpy(), lse=lse.cpu().numpy(),
                                   entropy=ent.cpu().numpy(), argmax=am.cpu().numpy())


@pytest.mark.parametrize("bounds", [[0, 20008], [0, 1000, 5000, 20008], [0, 8, 4096, 19992, 20008]])
def test_merge_of_slices_is_the_full_row(bounds):
    rng = np.random.default_rng(len(bounds))
    L, V, d = 24, 20008, 96
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 12.0
    bits = table(V, d, 15)
    x_t, w_t = dev(x), dev(bits)
    say("merge", bounds)
    parts = [api.soft_embed_onepass(x_t, a, b, w_t[a:b], 4.0) for a, b in zip(bounds, bounds[1:])]
    out, g = merge(parts)
    check_stats(g, oracle.row_stats(x))
    r = rel_fro(out, oracle.soft_embed(x, 0, V, bits, 4.0))
    say(f"rel_fro {r:.3e}")
    assert r <= GATE


def test_full_size_whole_vocabulary_and_four_rank_merge():
    """The full workload (L=256, V=262144, d=2816) in one pass, sampled rows against the
    oracle; then the four 65,536-row slices merged, against the same oracle."""
    w = wl.get("full")
    say("full-size onepass: inputs")
    x = wl.make_logits(w)
    bits, _ = wl.make_table(w)
    x_t, tab_t = dev(x), dev(bits)
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([[0, 255], rng.integers(0, 256, 2)]))
    stat_rows = np.unique(np.concatenate([rows, rng.integers(0, 256, 20)]))
    say("full-size onepass: gpu")
    res = api.soft_embed_onepass(x_t, 0, w.vocab, tab_t, w.gamma)
    torch.cuda.synchronize()
    out = res[0].cpu().numpy()
    g = dict(max=res[1].cpu().numpy(), lse=res[2].cpu().numpy(), entropy=res[3].cpu().numpy(),
             argmax=res[4].cpu().numpy())
    np.testing.assert_array_equal(g["argmax"], wl.planted_index(w))
    say("full-size onepass: oracle rows", list(rows))
    check_stats({k: v[stat_rows] for k, v in g.items()}, oracle.row_stats(x[stat_rows]))
    ref = oracle.soft_embed(x[rows], 0, w.vocab, bits, w.gamma)
    assert rel_fro(out[rows], ref) <= GATE
    say("full-size four-rank merge")
    q = w.vocab // 4
    parts = [api.soft_embed_onepass(x_t, r * q, (r + 1) * q, tab_t[r * q:(r + 1) * q], w.gamma)
             for r in range(4)]
    mout, mg = merge(parts)
    np.testing.assert_array_equal(mg["argmax"], wl.planted_index(w))
    check_stats({k: v[stat_rows] for k, v in mg.items()}, oracle.row_stats(x[stat_rows]))
    assert rel_fro(mout[rows], ref) <= GATE
    assert rel_fro(mout, out) <= GATE


def test_full_size_near_converged_canvas():
    w = wl.get("conv")
    say("conv onepass: inputs")
    x = wl.make_logits(w)
    bits, _ = wl.make_table(w)
    res = api.soft_embed_onepass(dev(x), 0, w.vocab, dev(bits), w.gamma)
    torch.cuda.synchronize()
    ent = res[3].cpu().numpy()
    assert np.all(np.abs(ent - 0.0178) < 0.003)
    rows = np.array([3, 130])
    g = dict(max=res[1].cpu().numpy()[rows], lse=res[2].cpu().numpy()[rows], entropy=ent[rows],
             argmax=res[4].cpu().numpy()[rows])
    check_stats(g, oracle.row_stats(x[rows]))
    assert rel_fro(res[0].cpu().numpy()[rows],
                   oracle.soft_embed(x[rows], 0, w.vocab, bits, w.gamma)) <= GATE
