"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test names what it pins.  The oracle is never compared with itself: the
expected values come from closed forms, special cases, independent library
routines (scipy, torch CPU casts), brute force written here in pure Python, or
numbers printed on the pages (tests/golden/page_figures.json).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from diffusion_self_conditioning_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")
RNG = np.random.default_rng(12345)


def _bf16_table(rows, d, rng=RNG):
    return wl.fp32_to_bf16_bits(rng.standard_normal((rows, d), dtype=np.float32) * np.float32(0.02))


def _table_values(bits):
    return wl.bf16_bits_to_fp32(bits).astype(np.float64)


# --- one-hot p: the expected embedding of a point mass is that token's row ----------
@pytest.mark.parametrize("k,s,e", [(0, 0, 512), (511, 0, 512), (130, 128, 256), (300, 128, 256),
                                   (5, 8, 512)])
def test_one_hot_returns_gamma_times_row(k, s, e):
    """Page 1, 'Where the shapes stop agreeing': e_i = sum_v p_iv W_v.  With p = e_k the sum is
    W_k; with gamma (page 1, 'The fix') it is gamma W_k; outside the slice it is 0."""
    V, d, gamma = 512, 24, np.float32(53.065998)
    x = wl.one_hot_logits(3, V, [k, k, k])
    table = _bf16_table(V, d)
    shard = table[s:]
    out = oracle.soft_embed(x, s, e, shard, gamma)
    want = np.zeros(d) if not (s <= k < e) else float(gamma) * _table_values(table[k])
    np.testing.assert_allclose(out, np.broadcast_to(want, out.shape), rtol=1e-12, atol=1e-80)  # e^-200 is not 0 in fp64
    st = oracle.row_stats(x)
    assert (st["argmax"] == k).all()
    assert np.all(np.abs(st["entropy"]) < 1e-60)          # H = 0 for a point mass
    np.testing.assert_allclose(st["lse"], 0.0, atol=1e-60)  # lse = 0 + log(1 + (V-1)e^-200)
    assert (st["max"] == 0.0).all()


def test_one_hot_fp32_table():
    V, d = 64, 5
    w = RNG.standard_normal((V, d)).astype(np.float32)
    x = wl.one_hot_logits(1, V, [17])
    out = oracle.soft_embed(x, 0, V, w, 16.0)
    np.testing.assert_allclose(out[0], 16.0 * w[17].astype(np.float64), rtol=1e-13)


# --- uniform p: gamma times the column mean; H = ln V; argmax = first index ---------
@pytest.mark.parametrize("V", [1, 7, 4096, 65536])
def test_uniform_distribution(V):
    """Uniform logits give p = 1/V: entropy ln V, lse = c + ln V, the tie goes to index 0,
    and the soft embedding is gamma times the mean of the table's rows."""
    d, c, gamma = 16, 0.5, np.float32(16.0)
    x = wl.uniform_logits(2, V, c)
    table = _bf16_table(V, d)
    st = oracle.row_stats(x)
    np.testing.assert_allclose(st["entropy"], math.log(V), rtol=1e-10, atol=1e-15)  # V-term sequential sum
    np.testing.assert_allclose(st["lse"], c + math.log(V), rtol=1e-13)
    assert (st["argmax"] == 0).all()
    out = oracle.soft_embed(x, 0, V, table, gamma)
    mean = _table_values(table).mean(axis=0)
    np.testing.assert_allclose(out, np.broadcast_to(float(gamma) * mean, out.shape),
                               rtol=1e-11, atol=1e-14)


def test_uniform_entropy_values_for_the_workload_widths():
    """ln 4096 and ln 262144 (the two vocabulary widths used here)."""
    for V, h in [(4096, 8.317766166719343), (262144, 12.476649250079015)]:
        st = oracle.row_stats(wl.uniform_logits(1, V, -3.25))
        assert abs(st["entropy"][0] - h) < 1e-10


def test_uniform_slice_is_partial_sum_over_slice():
    V, d, s, e = 256, 8, 64, 96
    table = _bf16_table(V, d)
    out = oracle.soft_embed(wl.uniform_logits(1, V), s, e, table[s:], 2.0)
    want = 2.0 * _table_values(table[s:e]).sum(axis=0) / V
    np.testing.assert_allclose(out[0], want, rtol=1e-12)


# --- partition identity (page 1, 'The fix') -----------------------------------------
@pytest.mark.parametrize("bounds", [[0, 1024], [0, 512, 1024], [0, 256, 512, 768, 1024],
                                    [0, 128, 256, 384, 512, 640, 768, 896, 1024],
                                    [0, 8, 600, 1000, 1024], [0, 1016, 1024]])
def test_partition_sum_equals_full_product(bounds):
    """P W = sum_r P[:, s_r:e_r] W^(r) for a disjoint, exhaustive vocab partition."""
    V, d = 1024, 40
    x = RNG.standard_normal((5, V), dtype=np.float32) * np.float32(3.0)
    table = _bf16_table(V, d)
    full = oracle.soft_embed(x, 0, V, table, 1.7)
    parts = sum(oracle.soft_embed(x, a, b, table[a:], 1.7) for a, b in zip(bounds[:-1], bounds[1:]))
    np.testing.assert_allclose(parts, full, rtol=1e-12, atol=1e-15)


def test_empty_slice_is_zero():
    x = RNG.standard_normal((2, 64), dtype=np.float32)
    out = oracle.soft_embed(x, 32, 32, _bf16_table(64, 4)[32:], 3.0)
    assert (out == 0).all()


# --- independent library routines --------------------------------------------------
def test_against_scipy_softmax_logsumexp_entropy():
    w = wl.get("tiny")
    x = wl.make_logits(w)
    _, tf32 = wl.make_table(w)
    st = oracle.row_stats(x)
    xd = x.astype(np.float64)
    p = scipy.special.softmax(xd, axis=1)
    np.testing.assert_allclose(st["lse"], scipy.special.logsumexp(xd, axis=1), rtol=1e-13)
    np.testing.assert_allclose(st["entropy"], scipy.stats.entropy(p, axis=1), rtol=1e-9, atol=1e-13)
    np.testing.assert_array_equal(st["argmax"], np.argmax(x, axis=1))
    np.testing.assert_array_equal(st["max"], x.max(axis=1).astype(np.float64))
    out = oracle.soft_embed(x, 0, w.vocab, tf32, w.gamma)
    ref = float(np.float32(w.gamma)) * (p @ tf32.astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-13)


def test_identity_table_returns_the_distribution():
    """With W = I (d = V) the soft embedding is gamma * p itself: p >= 0, sum p = 1."""
    V = 96
    x = RNG.standard_normal((4, V), dtype=np.float32) * np.float32(2.0)
    eye = np.eye(V, dtype=np.float32)
    p = oracle.soft_embed(x, 0, V, eye, 1.0)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(p, scipy.special.softmax(x.astype(np.float64), axis=1), rtol=1e-13)
    # a slice of the identity returns the matching columns of p
    q = oracle.soft_embed(x, 32, 64, eye[32:, 32:64].copy(), 1.0)
    np.testing.assert_allclose(q, p[:, 32:64], rtol=1e-14)


# --- brute force on tiny inputs, pure Python ---------------------------------------
def _brute(xrow, table, s, e, gamma, d=0):
    m = max(xrow)
    z = math.fsum(math.exp(v - m) for v in xrow)
    lse = m + math.log(z)
    p = [math.exp(v - lse) for v in xrow]
    h = -math.fsum(q * math.log(q) for q in p if q > 0)
    am = xrow.index(m)
    out = [gamma * math.fsum(p[v] * table[v - s][j] for v in range(s, e)) for j in range(d)]
    return m, am, lse, h, out


def test_brute_force_exhaustive_small():
    rng = np.random.default_rng(7)
    for L in (1, 2, 3):
        for V in range(1, 9):
            for d in range(1, 5):
                x = rng.integers(-4, 5, size=(L, V)).astype(np.float32)
                table = rng.integers(-3, 4, size=(V, d)).astype(np.float32) / np.float32(4)
                for s in range(0, V + 1, 2):
                    for e in range(s, V + 1, 3):
                        out = oracle.soft_embed(x, s, e, table[s:] if s < V else table[:0], 1.5)
                        for i in range(L):
                            _, _, _, _, bo = _brute([float(t) for t in x[i]],
                                                    [[float(t) for t in r] for r in table[s:]],
                                                    s, e, 1.5, d)
                            np.testing.assert_allclose(out[i], bo, rtol=1e-13, atol=1e-15)
                st = oracle.row_stats(x)
                for i in range(L):
                    m, am, lse, h, _ = _brute([float(t) for t in x[i]], [], 0, 0, 1.0)
                    assert st["max"][i] == m and st["argmax"][i] == am
                    assert abs(st["lse"][i] - lse) < 1e-13 and abs(st["entropy"][i] - h) < 1e-13


def test_brute_force_continuous_workload_distribution():
    """Element values on data drawn like the workloads' (logits N(0, 9) with a planted
    maximum 8 above the rest, table N(0, 0.02^2) rounded to bf16, gamma = fp32(sqrt(2816))):
    the oracle's statistics and embedding against the pure-Python evaluation from the
    definitions, on a slice in the middle of the row and on the whole row."""
    rng = np.random.default_rng(31)
    gamma = float(np.float32(math.sqrt(2816.0)))
    for L, V, d in ((2, 37, 5), (3, 130, 4)):
        x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
        for i in range(L):
            k = int(rng.integers(V))
            x[i, k] = np.float32(np.max(np.delete(x[i], k)) + 8)
        bits = _bf16_table(V, d, rng)
        table = _table_values(bits)
        st = oracle.row_stats(x)
        for s, e in ((0, V), (V // 3, V - 5)):
            out = oracle.soft_embed(x, s, e, bits[s:], gamma)
            for i in range(L):
                m, am, lse, h, bo = _brute([float(t) for t in x[i]],
                                           [[float(t) for t in r] for r in table[s:]], s, e, gamma, d)
                np.testing.assert_allclose(out[i], bo, rtol=1e-12, atol=1e-15)
                assert st["max"][i] == m and st["argmax"][i] == am
                assert abs(st["lse"][i] - lse) < 1e-12 and abs(st["entropy"][i] - h) < 1e-12


# --- invariants --------------------------------------------------------------------
def test_invariants_bounds_shift_linearity_permutation():
    V, d = 777, 12
    x = RNG.standard_normal((6, V), dtype=np.float32) * np.float32(3.0)
    table = _bf16_table(V, d)
    st = oracle.row_stats(x)
    assert np.all(st["entropy"] >= 0) and np.all(st["entropy"] <= math.log(V))
    assert np.all(st["max"] <= st["lse"]) and np.all(st["lse"] <= st["max"] + math.log(V))
    assert np.all(x[np.arange(6), st["argmax"]] == st["max"])
    base = oracle.soft_embed(x, 0, V, table, 1.0)
    # linear in gamma
    np.testing.assert_allclose(oracle.soft_embed(x, 0, V, table, 4.0), 4.0 * base, rtol=1e-14)
    # linear in W (fp32 tables: W1 + W2)
    w1 = RNG.standard_normal((V, d)).astype(np.float32)
    w2 = RNG.standard_normal((V, d)).astype(np.float32)
    a = oracle.soft_embed(x, 0, V, w1, 1.0) + oracle.soft_embed(x, 0, V, w2, 1.0)
    np.testing.assert_allclose(oracle.soft_embed(x, 0, V, w1 + w2, 1.0), a, rtol=1e-5, atol=1e-9)
    # invariant to a constant shift of the logits (the max shift of log-sum-exp)
    xq = np.round(x * 64) / np.float32(64)          # 6 fraction bits: x + 1024 is exact in fp32
    bq = oracle.soft_embed(xq, 0, V, table, 1.0)
    sh = oracle.soft_embed(xq + np.float32(1024.0), 0, V, table, 1.0)
    np.testing.assert_allclose(sh, bq, rtol=1e-12, atol=1e-15)
    st2 = oracle.row_stats(np.full((1, V), np.float32(900.0)))
    assert abs(st2["entropy"][0] - math.log(V)) < 1e-10 and math.isfinite(st2["lse"][0])
    # consistent vocabulary permutation leaves the embedding unchanged
    perm = RNG.permutation(V)
    np.testing.assert_allclose(oracle.soft_embed(x[:, perm], 0, V, table[perm], 1.0), base,
                               rtol=1e-12, atol=1e-15)


def test_argmax_first_index_on_ties():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-0.0, 0.0, -1.0, 0.0]], np.float32)
    st = oracle.row_stats(x)
    assert list(st["argmax"]) == [1, 0, 0]


def test_nonfinite_logits_rejected():
    x = np.zeros((1, 8), np.float32)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.row_stats(x)


# --- bf16 rounding used by the diagnostic mode -------------------------------------
def test_round_bf16_matches_torch_cpu_cast():
    import torch
    v = np.concatenate([RNG.random(2000) * 2.0 ** RNG.integers(-140, 3, 2000),
                        [1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 2 ** -130, 0.0]])
    v32 = v.astype(np.float32)
    want = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(v32.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_diagnostic_bf16_mode_is_close_to_exact():
    w = wl.get("tiny")
    x = wl.make_logits(w.diffuse())[:4]
    bits, _ = wl.make_table(w)
    a = oracle.soft_embed(x, 0, w.vocab, bits, w.gamma)
    b = oracle.soft_embed(x, 0, w.vocab, bits, w.gamma, round_p_bf16=True)
    rel = np.linalg.norm(a - b) / np.linalg.norm(a)
    assert 1e-4 < rel < 5e-3        # bf16 rounding of p is visible but small


# --- workload generator facts the tolerances rely on -------------------------------
def test_planted_max_is_unique_with_margin():
    w = wl.get("tiny")
    x = wl.make_logits(w)
    ks = wl.planted_index(w)
    st = oracle.row_stats(x)
    np.testing.assert_array_equal(st["argmax"], ks)
    srt = np.sort(x, axis=1)
    assert np.all(srt[:, -1] - srt[:, -2] >= 8.0 - 1e-5)
    assert np.all(st["entropy"] < 0.6)


def test_near_converged_statistics():
    """+20 planted over N(0,1) at V = 262,144: p_max = e^20 / (e^20 + sum e^x) with
    E[e^x] = e^(1/2); hence p_max ~ 0.99911 and H ~ 0.0178 nats."""
    w = wl.get("conv")
    x = wl.make_logits(w.with_rows(4))
    st = oracle.row_stats(x)
    zrest = (w.vocab - 1) * math.exp(0.5)
    pmax = math.exp(20) / (math.exp(20) + zrest)
    np.testing.assert_allclose(np.exp(st["max"] - st["lse"]), pmax, rtol=2e-5)
    assert np.all(np.abs(st["entropy"] - 0.0178) < 0.002)


def test_table_padding_rows_are_zero():
    w = wl.get("rank")
    small = wl.Workload("pad", 9, 1, 48, 8, 16, 32, 64, 1.0, 1.0, "none", False)
    bits, _ = wl.make_table(small)
    assert (bits[48:] == 0).all() and (bits[:48] != 0).any()
    assert w.table_rows - w.vocab == 256


# --- figures printed on page 1 -------------------------------------------------------
def test_page_figures():
    g = json.load(open(GOLDEN))
    V, d, L = g["vocab"]["value"], g["hidden"]["value"], g["canvas_len"]["value"]
    assert V * d * 2 == g["embedding_bytes_bf16"]["value"]
    assert round(V * d * 2 / 2 ** 30, 2) == g["embedding_gib_rounded"]["value"]
    full, rank = wl.get("full"), wl.get("rank")
    assert (full.vocab, full.d, full.rows) == (V, d, L)
    assert round(full.flops() / 1e9) == g["gflop_full_per_rank_step"]["value"]
    assert round(rank.flops() / 1e9, 1) == g["gflop_sharded_t4"]["value"]
    assert rank.k == g["shard_rows_t4"]["value"] == V // 4
    mib = L * d * 2 / 2 ** 20
    assert round(mib, 2) == g["reduced_tensor_mib"]["value"]
    assert round(2 * (4 - 1) / 4 * mib, 2) == g["ring_mib_per_rank_t4"]["value"]
    assert V // (2 * L) == g["crossover_kn"]["value"]


def test_gamma_is_fp32_sqrt_d():
    assert wl.get("full").gamma == float(np.float32(math.sqrt(2816)))
    assert Fraction(wl.get("tiny").gamma) == 16


# --- the range-wise form used to check the one-read calls --------------------------
def _bf16_py(x: float) -> float:
    """Nearest bf16 value (8 significant bits, ties to even) of a positive normal double,
    written with Python's round-half-even on the exact scaled significand."""
    if x == 0.0:
        return 0.0
    m, e = math.frexp(x)                 # x = m 2^e, m in [0.5, 1)
    return math.ldexp(round(m * 256.0), e - 8)


def _brute_ranges(xrow, table, bounds, gamma, d, rnd):
    m = max(xrow)
    lse = m + math.log(math.fsum(math.exp(v - m) for v in xrow))
    s = bounds[0]
    out = [0.0] * d
    for a, b in zip(bounds, bounds[1:]):
        mr = max(xrow[a:b])
        qs = [math.exp(xrow[v] - mr) for v in range(a, b)]
        if rnd:
            qs = [_bf16_py(q) for q in qs]
        f = math.exp(mr - lse)
        for j in range(d):
            out[j] += f * math.fsum(q * table[a + t - s][j] for t, q in enumerate(qs))
    return [gamma * o for o in out]


def test_ranges_brute_force_small():
    """Each range's probabilities against its own maximum, rescaled by e^(m_r - lse): the
    oracle's range-wise form against a pure-Python evaluation, with and without bf16
    rounding of e^(l - m_r)."""
    rng = np.random.default_rng(21)
    for L in (1, 3):
        for V in (5, 9, 16):
            d = 3
            x = (rng.standard_normal((L, V)) * 2).astype(np.float32)
            table = rng.integers(-3, 4, size=(V, d)).astype(np.float32) / np.float32(4)
            for bounds in ([0, V], [0, 2, V], [1, 3, V - 1], [2, 3, 4, V]):
                s, e = bounds[0], bounds[-1]
                for rnd in (False, True):
                    out = oracle.soft_embed_ranges(x, bounds, table[s:], 1.5, round_q_bf16=rnd)
                    for i in range(L):
                        bo = _brute_ranges([float(t) for t in x[i]],
                                           [[float(t) for t in r] for r in table[s:]],
                                           bounds, 1.5, d, rnd)
                        np.testing.assert_allclose(out[i], bo, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("bounds", [[0, 4096], [0, 128, 2048, 4096], [256, 1024, 1152, 3072]])
def test_ranges_without_rounding_are_the_partition_identity(bounds):
    """Page 1, 'The fix': the product over a slice is the sum of the products over any
    partition of it; rescaling each piece's softmax numerators changes nothing exactly."""
    w = wl.get("tiny")
    x = wl.make_logits(w.diffuse())[:5]
    bits, _ = wl.make_table(w)
    s, e = bounds[0], bounds[-1]
    got = oracle.soft_embed_ranges(x, bounds, bits[s:], w.gamma)
    want = oracle.soft_embed(x, s, e, bits[s:], w.gamma)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_ranges_one_hot_and_uniform():
    """A point mass in range r gives q = 1 there (exact in bf16) and gamma W_k; uniform logits
    give q = 1 everywhere and gamma times the column mean, with or without rounding."""
    V, d, gamma = 1024, 16, np.float32(53.065998)
    table = _bf16_table(V, d)
    bounds = [0, 256, 512, 896, 1024]
    x = wl.one_hot_logits(2, V, [300, 1000])
    for rnd in (False, True):
        out = oracle.soft_embed_ranges(x, bounds, table, gamma, round_q_bf16=rnd)
        for i, k in enumerate([300, 1000]):
            np.testing.assert_allclose(out[i], float(gamma) * _table_values(table[k]),
                                       rtol=1e-13, atol=1e-80)
        u = oracle.soft_embed_ranges(wl.uniform_logits(1, V, 0.25), bounds, table, gamma,
                                     round_q_bf16=rnd)
        np.testing.assert_allclose(u[0], float(gamma) * _table_values(table).mean(axis=0),
                                   rtol=1e-12, atol=1e-15)
