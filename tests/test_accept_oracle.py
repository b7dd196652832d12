"""Pins of the acceptance / convergence oracle (CPU only).

The rule (agentlenshq overview of DiffusionGemma in vLLM, section on the sampling
loop and entropy-bound denoising): accept tokens from the most to the least
confident until the cumulative entropy exceeds a fixed budget; converged when the
argmax has been stable for several steps and the mean entropy is below a
threshold, or at the step limit.  Expected values below are worked by hand from
that sentence (and the readings stated in oracle/accept.py), or come from an
independent formulation (numpy lexsort + integer cumsum).
"""
import itertools

import numpy as np
import pytest

from oracle.accept import FIX, accept_converge, fixed


def run(ent, budget, accepted=None, am=None, prev=None, stable=0, steps=0, k=2, tau=1.0,
        limit=100, canvas_len=None):
    ent = np.asarray(ent, dtype=np.float32)
    n = ent.size
    L = canvas_len or n
    nc = n // L
    return accept_converge(
        ent, np.zeros(n, np.int32) if am is None else am, L, budget, k, tau, limit,
        np.zeros(n, np.uint8) if accepted is None else accepted,
        np.full(n, -1, np.int32) if prev is None else prev,
        np.full(nc, stable, np.int32), np.full(nc, steps, np.int32))


def test_worked_example_budget_prefix():
    # order by entropy: pos 1 (0.125), pos 2 (0.25), pos 0 (0.5), pos 3 (2.0)
    # cumulative 0.125, 0.375, 0.875 -> budget 0.5 keeps the first two
    r = run([0.5, 0.125, 0.25, 2.0], 0.5)
    assert r["newly"].tolist() == [0, 1, 1, 0]
    assert r["accepted"].tolist() == [0, 1, 1, 0]


def test_budget_is_inclusive():
    # 0.125 + 0.25 + 0.5 = 0.875 exactly (dyadic values): a budget of 0.875 keeps three
    r = run([0.5, 0.125, 0.25, 2.0], 0.875)
    assert r["newly"].tolist() == [1, 1, 1, 0]


def test_zero_budget_still_accepts_the_most_confident():
    r = run([0.5, 0.125, 0.25, 2.0], 0.0)
    assert r["newly"].tolist() == [0, 1, 0, 0]


def test_huge_budget_accepts_every_candidate():
    r = run([0.5, 0.125, 0.25, 2.0], 1e9)
    assert r["newly"].tolist() == [1, 1, 1, 1]


def test_ties_go_to_the_lower_position():
    r = run([0.25, 0.25, 0.25], 0.6)          # two of three fit
    assert r["newly"].tolist() == [1, 1, 0]
    r = run([0.0, -0.0, 0.0], 0.0)            # -0 and +0 are equal entropies
    assert r["newly"].tolist() == [1, 1, 1]


def test_already_accepted_positions_are_not_candidates():
    acc = np.array([0, 1, 0, 0], np.uint8)
    r = run([0.5, 0.125, 0.25, 2.0], 0.8, accepted=acc)
    # candidates 2 (0.25), 0 (0.5), 3 (2.0): cumulative 0.25, 0.75 -> two taken
    assert r["newly"].tolist() == [1, 0, 1, 0]
    assert r["accepted"].tolist() == [1, 1, 1, 0]
    r = run([0.1, 0.2], 5.0, accepted=np.ones(2, np.uint8))
    assert r["newly"].tolist() == [0, 0]


def test_canvases_are_independent():
    ent = [0.5, 0.125, 0.25, 2.0] * 3
    r = run(ent, 0.5, canvas_len=4)
    assert r["newly"].tolist() == [0, 1, 1, 0] * 3


def test_stability_counter_and_convergence():
    am = np.array([3, 7, 7, 1], np.int32)
    ent = [2.0 ** -7, 2.0 ** -6, 2.0 ** -7, 2.0 ** -6]     # dyadic: mean exactly 0.01171875
    # first step: prev = -1 differs -> counter 0, not converged
    r = run(ent, 0.0, am=am, k=2, tau=0.02)
    assert r["stable_count"].tolist() == [0] and r["converged"].tolist() == [0]
    assert r["prev_argmax"].tolist() == am.tolist() and r["step_count"].tolist() == [1]
    # same argmax twice in a row -> counter 1, then 2 -> converged (mean < 0.02)
    r = run(ent, 0.0, am=am, prev=am, stable=0, steps=1, k=2, tau=0.02)
    assert r["stable_count"].tolist() == [1] and r["converged"].tolist() == [0]
    r = run(ent, 0.0, am=am, prev=am, stable=1, steps=2, k=2, tau=0.02)
    assert r["stable_count"].tolist() == [2] and r["converged"].tolist() == [1]
    # stable but entropy too high: not converged
    r = run(ent, 0.0, am=am, prev=am, stable=5, steps=2, k=2, tau=0.01171875)
    assert r["converged"].tolist() == [0]          # mean == tau is not below it
    # one changed position resets the counter
    p = am.copy(); p[2] = 0
    r = run(ent, 0.0, am=am, prev=p, stable=5, steps=2, k=2, tau=1.0)
    assert r["stable_count"].tolist() == [0] and r["converged"].tolist() == [0]
    # step limit
    r = run(ent, 0.0, am=am, prev=p, stable=0, steps=9, k=2, tau=0.0, limit=10)
    assert r["step_count"].tolist() == [10] and r["converged"].tolist() == [1]


def test_fixed_point_is_exact_scaling():
    assert fixed(np.float32(0.5)) == 2 ** 31
    assert fixed(np.float32(2.0 ** -33)) == 0         # half of 2^-32 rounds to even
    assert fixed(np.float32(3 * 2.0 ** -33)) == 2     # 1.5 units rounds to even (2)
    assert fixed(np.float32(-0.0)) == 0


def independent_accept(ent, acc, budget):
    """numpy formulation: lexsort candidates, exact integer cumsum, first exceed."""
    idx = np.flatnonzero(acc == 0)
    if idx.size == 0:
        return set()
    order = idx[np.lexsort((idx, ent[idx].astype(np.float64)))]
    q = np.array([round(float(h) * FIX) for h in ent[order]], dtype=object)
    cum = np.cumsum(q)
    over = [j for j in range(len(order)) if float(cum[j]) > budget * FIX]
    k = over[0] if over else len(order)
    return set(order[:max(k, 1)].tolist())


@pytest.mark.parametrize("seed", range(20))
def test_against_independent_formulation(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 40))
    ent = rng.choice(np.float32([0.0, 0.05, 0.25, 1.0, 3.5]), L) if seed % 2 else \
        rng.exponential(0.5, L).astype(np.float32)
    acc = (rng.random(L) < 0.3).astype(np.uint8)
    budget = float(rng.choice([0.0, 0.1, 1.0, 3.0, 50.0]))
    r = run(ent, budget, accepted=acc)
    got = set(np.flatnonzero(r["newly"]).tolist())
    assert got == independent_accept(ent, acc, budget)


def test_brute_force_small_canvases():
    """For non-negative entropies the accepted set is the largest 'lightest-first' set:
    among all subsets closed under the (entropy, position) order, the longest whose
    total fits the budget (at least one element)."""
    vals = np.float32([0.0, 0.125, 0.25, 0.5])
    for L in range(1, 5):
        for ent in itertools.product(vals, repeat=L):
            ent = np.array(ent, np.float32)
            key = sorted(range(L), key=lambda i: (float(ent[i]), i))
            for budget in (0.0, 0.125, 0.4, 0.75, 2.0):
                best = [key[0]]
                for k in range(1, L + 1):
                    if sum(float(ent[i]) for i in key[:k]) <= budget:
                        best = key[:k]
                r = run(ent, budget)
                assert set(np.flatnonzero(r["newly"]).tolist()) == set(best)
