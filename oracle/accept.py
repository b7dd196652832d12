"""Oracle of the sampler's entropy-bound acceptance and convergence test -- TEST
INFRASTRUCTURE (only tests/, the smoke check and the benchmark's CPU leg use it).

The rule (agentlenshq overview of DiffusionGemma in vLLM, section on the sampling
loop and entropy-bound denoising): tokens are accepted from the most confident to
the least confident until the cumulative entropy exceeds a fixed budget; a canvas
has converged when its argmax prediction has been stable for several steps and
its mean per-token entropy is below a threshold, or when a step limit is reached.

Readings where the page is silent (the same ones the C header states):
  * confidence order = entropy ascending, ties by lower position; only positions
    not yet accepted are candidates;
  * entropies count as exact fixed-point integers round_half_even(H * 2^32), so
    every sum is exact; "exceeds the budget" compares the running sum with
    budget * 2^32 in double precision;
  * a step accepts at least one candidate while any is left;
  * "stable for several steps": the whole canvas's argmax equals the previous
    step's, counted in consecutive steps;  "mean per-token entropy" is over all
    positions of the canvas.
Plain Python loops over each canvas; no blocking, no parallel scan.
"""
from __future__ import annotations

import numpy as np

FIX = 2.0 ** 32


def fixed(h) -> int:
    """Entropy (a float32 value) as an exact multiple of 2^-32 nats, ties to even."""
    return round(float(h) * FIX)


def accept_converge(entropy, argmax, canvas_len, budget, stable_steps, tau, step_limit,
                    accepted, prev_argmax, stable_count, step_count):
    """One sampler step for every canvas.

    Returns a dict of new arrays: newly (uint8), accepted (uint8), prev_argmax (int32),
    stable_count (int32), step_count (int32), converged (uint8).  Inputs are not modified.
    """
    ent = np.asarray(entropy, dtype=np.float32).ravel()
    am = np.asarray(argmax, dtype=np.int32).ravel()
    n = ent.size
    if n % canvas_len:
        raise ValueError("row count is not a multiple of canvas_len")
    n_canvas = n // canvas_len
    acc = np.array(accepted, dtype=np.uint8).ravel().copy()
    prev = np.array(prev_argmax, dtype=np.int32).ravel().copy()
    stable = np.array(stable_count, dtype=np.int32).ravel().copy()
    steps = np.array(step_count, dtype=np.int32).ravel().copy()
    newly = np.zeros(n, dtype=np.uint8)
    conv = np.zeros(n_canvas, dtype=np.uint8)
    limit = float(budget) * FIX
    for c in range(n_canvas):
        lo = c * canvas_len
        pos = range(lo, lo + canvas_len)
        # acceptance: candidates from most to least confident
        cand = sorted((i for i in pos if acc[i] == 0), key=lambda i: (float(ent[i]), i))
        total = 0
        taken = []
        for i in cand:
            total += fixed(ent[i])
            if float(total) > limit and taken:
                break
            taken.append(i)
            if float(total) > limit:       # the one forced pick already exceeds the budget
                break
        for i in taken:
            newly[i] = 1
            acc[i] = 1
        # convergence
        same = all(am[i] == prev[i] for i in pos)
        stable[c] = stable[c] + 1 if same else 0
        for i in pos:
            prev[i] = am[i]
        steps[c] += 1
        calm = float(sum(fixed(ent[i]) for i in pos)) < float(tau) * canvas_len * FIX
        conv[c] = 1 if (stable[c] >= stable_steps and calm) or steps[c] >= step_limit else 0
    return {"newly": newly, "accepted": acc, "prev_argmax": prev, "stable_count": stable,
            "step_count": steps, "converged": conv}
