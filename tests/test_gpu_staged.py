"""GPU parity of se_soft_embed_staged and se_soft_embed_step (MI355X), through the C ABI.

The staged call must return se_soft_embed_fused's output bit for bit: the same bf16
probabilities (same rounding), contracted in the same order; only their trip through
memory differs.  The fused call is itself gated against the fp64 oracle in
test_gpu_parity.py; here the staged output is also gated directly on the small cases.
Cases: whole and partial 256-row tiles (the two contraction kernels), slices of 1 / 63 /
4097 positions and ragged hidden sizes, slices that start mid-vocabulary, shard rows past
the slice holding NaN (never read), one split and many splits, tails of the last split,
and the one-rank workload at full size.
se_soft_embed_step must return se_row_stats' statistics and the fused call's
embedding bit for bit, on the same kinds of cases plus an empty slice.
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


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rel_fro(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / np.linalg.norm(b)


CASES = {
    # name: (L, V, s, e, d, seed)
    "tiny": (16, 4096, 0, 4096, 256, 1),
    "ragged": (17, 20008, 8, 20008, 48, 2),
    "slice-1": (5, 1000, 16, 17, 16, 3),
    "slice-63": (33, 1000, 64, 127, 2816, 4),
    "slice-4097": (255, 8200, 8, 4105, 272, 5),
    "two-row-tiles": (300, 2048, 0, 2048, 512, 6),
    "one-split": (16, 200, 0, 200, 64, 7),
    "mid-vocab": (64, 50000, 12344, 37000, 128, 8),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_staged_equals_fused(case):
    L, V, s, e, d, seed = CASES[case]
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s + 40, d)) * 0.02).astype(np.float32))
    tab[e - s:] = 0x7FC0                                  # rows past the slice: NaN, never read
    say("staged", case, (L, V, s, e, d))
    x_t, w_t = dev(x), dev(tab)
    _, lse, _, _ = api.row_stats(x_t)
    fused = api.soft_embed(x_t, lse, s, e, w_t, 5.0, fused=True)
    staged = api.soft_embed(x_t, lse, s, e, w_t, 5.0, staged=True)
    torch.cuda.synchronize()
    assert torch.equal(staged, fused)
    if L * (e - s) * d <= 5e9:
        ref = oracle.soft_embed(x, s, e, tab[:e - s], 5.0)
        assert rel_fro(staged.cpu().numpy(), ref) <= 5e-3


# Whole 256-row tiles of staged probabilities take the ping-pong contraction (the shapes
# above, with partial row tiles, take the register-staged one): the tail of the last split
# alone (slices of 1 and 63 positions), one super-step with and without a tail, two row
# tiles, many splits with a tail, hidden sizes that are not a multiple of 256, long splits.
TILE_CASES = {
    # name: (L, V, s, e, d, seed)
    "k1": (256, 1000, 8, 9, 64, 61),
    "k63": (256, 1004, 64, 127, 272, 62),
    "k128": (256, 4096, 0, 128, 128, 63),
    "k200-two-tiles": (512, 5000, 40, 240, 256, 64),
    "k4097": (256, 8200, 8, 4105, 2816, 65),
    "k12345": (512, 50000, 12344, 24689, 520, 66),
    "k65553": (256, 70000, 0, 65553, 256, 67),
    "d16": (256, 5000, 0, 4097, 16, 68),          # one n-tile of 16 columns: clamped loads
    # splits of at least 32 super-steps take three probability stage buffers, the loop
    # unrolled over their cycle: split lengths of every remainder mod 3 (50/51, 113/114,
    # 48/49 super-steps), ragged tails, two row tiles, 64 splits
    "long-splits": (256, 150012, 8, 150003, 2816, 69),
    "long-splits-two-tiles": (512, 160012, 8, 160011, 2816, 70),
    "long-splits-64-splits": (256, 400012, 8, 400011, 512, 71),
    # splits of one to five super-steps (two stage buffers): the stage load past a split's
    # end clamped to its last stage, several splits per tile, two row tiles
    "short-splits-1-2": (256, 1500, 8, 1011, 2816, 72),
    "short-splits-2-3": (256, 3500, 8, 3011, 2816, 73),
    "short-splits-4-5": (512, 5600, 8, 5011, 2816, 74),
}


def split_super_steps(L, s, e, d):
    """The whole super-steps (of 128 positions) of each split of this contraction."""
    bounds = B.se_soft_embed_ranges(L, s, e, d)
    return [(b - a) // 128 for a, b in zip(bounds, bounds[1:])]


@pytest.mark.parametrize("case", sorted(TILE_CASES))
def test_staged_whole_tiles_equals_fused(case):
    L, V, s, e, d, seed = TILE_CASES[case]
    if case.startswith("long-splits"):
        assert min(split_super_steps(L, s, e, d)) >= 32, case
    if case.startswith("short-splits"):
        n = split_super_steps(L, s, e, d)
        assert 1 <= min(n) <= max(n) <= 5, case
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s + 40, d)) * 0.02).astype(np.float32))
    tab[e - s:] = 0x7FC0                                  # rows past the slice: NaN, never read
    say("staged whole tiles", case, (L, V, s, e, d))
    x_t, w_t = dev(x), dev(tab)
    _, lse, _, _ = api.row_stats(x_t)
    fused = api.soft_embed(x_t, lse, s, e, w_t, 5.0, fused=True)
    staged = api.soft_embed(x_t, lse, s, e, w_t, 5.0, staged=True)
    again = api.soft_embed(x_t, lse, s, e, w_t, 5.0, staged=True)
    # row-major bf16 probabilities (pitch rounded up to 8 elements) through se_soft_embed
    probs = torch.empty((L, (V + 7) // 8 * 8), device=DEV, dtype=torch.bfloat16)[:, :V]
    api.se_probs_bf16(x_t, lse, s, e, probs)
    unfused = torch.empty((L, d), device=DEV)
    api.se_soft_embed(probs, s, e, w_t, 5.0, unfused, api.workspace(L, s, e, d, DEV))
    torch.cuda.synchronize()
    assert torch.equal(staged, fused)
    assert torch.equal(again, staged)
    assert torch.equal(unfused, fused)
    ref = oracle.soft_embed(x, s, e, tab[:e - s], 5.0)
    assert rel_fro(staged.cpu().numpy(), ref) <= 5e-3


def test_whole_tiles_with_row_pitches():
    """Whole 256-row tiles with every row pitch wider than its row: logits and row-major
    probabilities (V + 8), table (d + 72, so the table loads skip columns), output (d + 4,
    columns past d untouched).  Staged and unfused equal fused and the step equals the
    separate calls, bit for bit; all meet the oracle."""
    L, V, s, e, d = 256, 20000, 8, 12353, 264
    rng = np.random.default_rng(71)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    xb = np.full((L, V + 8), np.float32(1e30), np.float32)
    xb[:, :V] = x
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s, d)) * 0.02).astype(np.float32))
    tb = np.full((e - s, d + 72), 0x7FC0, np.uint16)          # padding columns: NaN, never read
    tb[:, :d] = tab
    x_t, w_t = dev(xb)[:, :V], dev(tb)[:, :d]
    assert x_t.stride(0) == V + 8 and w_t.stride(0) == d + 72
    say("whole tiles with row pitches")
    mx, lse, ent, am = api.row_stats(x_t)
    outs = {}
    probs = torch.empty((L, V + 8), device=DEV, dtype=torch.bfloat16)[:, :V]   # pitch V + 8
    api.se_probs_bf16(x_t, lse, s, e, probs)
    for name in ("fused", "staged", "step", "unfused"):
        buf = torch.full((L, d + 4), -7.0, device=DEV)
        o = buf[:, :d]
        if name == "fused":
            api.se_soft_embed_fused(x_t, lse, s, e, w_t, 5.0, o, api.workspace(L, s, e, d, DEV))
        elif name == "staged":
            api.se_soft_embed_staged(x_t, lse, s, e, w_t, 5.0, o, api.staged_workspace(L, s, e, d, DEV))
        elif name == "unfused":
            api.se_soft_embed(probs, s, e, w_t, 5.0, o, api.workspace(L, s, e, d, DEV))
        else:
            st = [torch.empty(L, device=DEV) for _ in range(3)] + [torch.empty(L, device=DEV, dtype=torch.int32)]
            api.se_soft_embed_step(x_t, s, e, w_t, 5.0, o, *st, api.staged_workspace(L, s, e, d, DEV))
            for a, b in zip(st, (mx, lse, ent, am)):
                outs.setdefault("stats_equal", True)
                outs["stats_equal"] &= bool(torch.equal(a, b))
        outs[name] = buf
    torch.cuda.synchronize()
    assert outs["stats_equal"]
    assert torch.equal(outs["staged"], outs["fused"]) and torch.equal(outs["step"], outs["fused"])
    assert torch.equal(outs["unfused"], outs["fused"])
    assert bool((outs["staged"][:, d:] == -7.0).all())
    ref = oracle.soft_embed(x, s, e, tab, 5.0)
    assert rel_fro(outs["staged"][:, :d].cpu().numpy(), ref) <= 5e-3


@pytest.mark.parametrize("shape", [(256, 262144, 65536, 131072, 2816), (2048, 20480, 0, 16384, 2816)],
                         ids=["rank-shape", "eight-row-tiles"])
def test_staged_repeated_calls_stay_bitwise(shape):
    """The ping-pong contraction's hand-written wait counts and barriers, exercised back to
    back: 60 staged calls on one stream, each output equal to the fused call's bit for bit."""
    L, V, s, e, d = shape
    rng = np.random.default_rng(81)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s, d)) * 0.02).astype(np.float32))
    x_t, w_t = dev(x), dev(tab)
    say("repeated staged calls", shape)
    _, lse, _, _ = api.row_stats(x_t)
    ref = api.soft_embed(x_t, lse, s, e, w_t, 3.0, fused=True)
    ws = api.staged_workspace(L, s, e, d, DEV)
    outs = [torch.empty_like(ref) for _ in range(60)]
    for o in outs:
        api.soft_embed(x_t, lse, s, e, w_t, 3.0, staged=True, out=o, ws=ws)
    torch.cuda.synchronize()
    assert all(torch.equal(o, ref) for o in outs)


def test_staged_empty_slice_writes_zeros():
    x_t = dev(np.zeros((4, 64), np.float32))
    _, lse, _, _ = api.row_stats(x_t)
    out = torch.full((4, 16), float("nan"), device=DEV)
    api.se_soft_embed_staged(x_t, lse, 8, 8, dev(np.zeros((8, 16), np.uint16)), 1.0, out, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0


def test_staged_full_size_rank():
    w = wl.get("rank")
    say("staged full-size rank: inputs")
    x = wl.make_logits(w)
    bits, _ = wl.make_table(w)
    x_t, tab_t = dev(x), dev(bits)
    _, lse, _, _ = api.row_stats(x_t)
    shard = tab_t[w.vocab_start:]
    say("staged full-size rank: gpu")
    fused = api.soft_embed(x_t, lse, w.vocab_start, w.vocab_end, shard, w.gamma, fused=True)
    staged = api.soft_embed(x_t, lse, w.vocab_start, w.vocab_end, shard, w.gamma, staged=True)
    again = api.soft_embed(x_t, lse, w.vocab_start, w.vocab_end, shard, w.gamma, staged=True)
    torch.cuda.synchronize()
    assert torch.equal(staged, fused)
    assert torch.equal(again, staged)
    rows = np.array([0, 255])
    ref = oracle.soft_embed(x[rows], w.vocab_start, w.vocab_end,
                            bits[w.vocab_start:w.vocab_end], w.gamma)
    assert rel_fro(staged.cpu().numpy()[rows], ref) <= 5e-3


STEP_CASES = {
    # name: (L, V, s, e, d, seed)
    "tiny": (16, 4096, 0, 4096, 256, 21),
    "ragged": (17, 20008, 8, 20008, 48, 22),
    "slice-63": (33, 1003, 64, 127, 2816, 23),        # V not a multiple of 4
    "two-row-tiles": (300, 2048, 1024, 2048, 512, 24),
    "empty-slice": (8, 512, 16, 16, 16, 25),
    "whole-tile": (256, 20003, 4000, 8097, 512, 26),   # the ping-pong contraction
    # slices within 1 to 4 groups of 16,384 positions: the statistics kernel keeps those
    # groups in registers instead of reading the slice twice; a longer slice keeps its first
    # 4 groups and reads the rest again
    "held-1-group": (16, 65536, 16384, 32768, 64, 27),
    "held-4-groups": (16, 65536, 0, 65536, 64, 28),
    "held-2-groups-at-end": (8, 81920, 49152, 81920, 128, 29),
    "five-groups-four-held": (8, 81920, 0, 81920, 64, 30),     # the fifth is read again
    # unaligned slices within at most 4 groups are held too (only [s, e) is written)
    "held-unaligned-4-groups": (16, 65536, 8, 50001, 64, 31),
    "held-unaligned-2-groups": (8, 81920, 20008, 45011, 128, 32),
}


@pytest.mark.parametrize("case", sorted(STEP_CASES))
def test_step_equals_row_stats_then_fused(case):
    """se_soft_embed_step: statistics bitwise se_row_stats', embedding bitwise the fused call's."""
    L, V, s, e, d, seed = STEP_CASES[case]
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s + 24, d)) * 0.02).astype(np.float32))
    tab[e - s:] = 0x7FC0
    ld = ((V + 3) // 4) * 4
    buf = np.full((L, ld), np.float32(1e30), np.float32)
    buf[:, :V] = x
    say("step", case, (L, V, s, e, d))
    x_t, w_t = dev(buf)[:, :V], dev(tab)
    out, mx, lse, ent, am = api.soft_embed_step(x_t, s, e, w_t, 5.0)
    mx2, lse2, ent2, am2 = api.row_stats(x_t)
    ref = api.soft_embed(x_t, lse2, s, e, w_t, 5.0, fused=True)
    torch.cuda.synchronize()
    for a, b in ((mx, mx2), (lse, lse2), (ent, ent2), (am, am2), (out, ref)):
        assert torch.equal(a, b)
    st = oracle.row_stats(x)
    np.testing.assert_array_equal(am.cpu().numpy(), st["argmax"])
    if e > s:
        assert rel_fro(out.cpu().numpy(), oracle.soft_embed(x, s, e, tab[:e - s], 5.0)) <= 5e-3
    else:
        assert torch.count_nonzero(out) == 0


def test_step_full_size_rank():
    w = wl.get("rank")
    say("step full-size rank: inputs")
    x = wl.make_logits(w)
    bits, _ = wl.make_table(w)
    x_t, tab_t = dev(x), dev(bits)
    shard = tab_t[w.vocab_start:]
    say("step full-size rank: gpu")
    out, mx, lse, ent, am = api.soft_embed_step(x_t, w.vocab_start, w.vocab_end, shard, w.gamma)
    mx2, lse2, ent2, am2 = api.row_stats(x_t)
    ref = api.soft_embed(x_t, lse2, w.vocab_start, w.vocab_end, shard, w.gamma, fused=True)
    torch.cuda.synchronize()
    for a, b in ((mx, mx2), (lse, lse2), (ent, ent2), (am, am2), (out, ref)):
        assert torch.equal(a, b)
    np.testing.assert_array_equal(am.cpu().numpy(), wl.planted_index(w))


def test_step_from_two_threads_on_two_streams():
    """Calls are reentrant: two host threads, each with its own stream, buffers and
    workspace, run the whole step concurrently and get the serial call's result bit for
    bit (the library keeps no per-call state of its own)."""
    import threading
    L, V, s, e, d = 64, 20000, 4000, 12000, 256
    rng = np.random.default_rng(31)
    xs = [(rng.standard_normal((L, V)) * 3).astype(np.float32) for _ in range(2)]
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s, d)) * 0.02).astype(np.float32))
    w_t = dev(tab)
    x_ts = [dev(x) for x in xs]
    ref = [api.soft_embed_step(x_t, s, e, w_t, 2.0) for x_t in x_ts]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    errs = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                outs = None
                for _ in range(20):
                    outs = api.soft_embed_step(x_ts[i], s, e, w_t, 2.0,
                                               stream=streams[i].cuda_stream)
                streams[i].synchronize()
                got[i] = outs
        except Exception as ex:          # reported after join
            errs.append(ex)
    say("step from two threads")
    ts = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errs, errs
    for i in range(2):
        for a, b in zip(got[i], ref[i]):
            assert torch.equal(a, b)


def test_more_rows_than_one_grid_dimension_holds():
    """70,000 rows: the launches that put rows in a grid dimension of at most 65,535 go in
    chunks (staged probabilities, the empty slice's zero fill).  The staged call equals the
    fused call and the step equals the separate calls, bit for bit; the one-read step agrees
    on argmax and max; the argmax matches the oracle."""
    L, V, s, e, d = 70000, 64, 8, 56, 16
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s, d)) * 0.02).astype(np.float32))
    x_t, w_t = dev(x), dev(tab)
    say("70000 rows")
    mx, lse, ent, am = api.row_stats(x_t)
    fused = api.soft_embed(x_t, lse, s, e, w_t, 3.0, fused=True)
    staged = api.soft_embed(x_t, lse, s, e, w_t, 3.0, staged=True)
    step = api.soft_embed_step(x_t, s, e, w_t, 3.0)
    one = api.soft_embed_step(x_t, s, e, w_t, 3.0, onepass=True)
    empty = api.soft_embed_step(x_t, 16, 16, w_t, 3.0)
    torch.cuda.synchronize()
    assert torch.equal(staged, fused)
    for a, b in zip(step, (fused, mx, lse, ent, am)):
        assert torch.equal(a, b)
    assert torch.equal(one[1], mx) and torch.equal(one[4], am)
    assert rel_fro(one[0].cpu().numpy(), fused.cpu().numpy()) <= 5e-3
    assert torch.count_nonzero(empty[0]) == 0
    np.testing.assert_array_equal(am.cpu().numpy(), oracle.row_stats(x)["argmax"])
