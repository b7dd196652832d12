"""GPU parity of se_accept_converge against the oracle (bit-exact: every output is an
integer or flag decided from the same fp32 entropies in the same exact arithmetic).

The rule: agentlenshq overview of DiffusionGemma in vLLM, section on the sampling loop
and entropy-bound denoising.  Cases: several canvases over several consecutive
steps (state carried on both sides), ragged and maximal canvas lengths, ties,
signed zeros and tiny negative entropies, all-accepted canvases, and the entropies
and argmax that se_row_stats computes from seeded logits.
"""
import numpy as np
import pytest
import torch

from oracle.accept import accept_converge as ref_accept

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def gpu_api():
    from diffusion_self_conditioning_amd import _binding as B
    return B


class Pair:
    """The same sampler state on the GPU and in the oracle."""

    def __init__(self, n_canvas, L, accepted=None):
        n = n_canvas * L
        self.L = L
        acc = np.zeros(n, np.uint8) if accepted is None else accepted.astype(np.uint8)
        self.ref = {"accepted": acc.copy(), "prev_argmax": np.full(n, -1, np.int32),
                    "stable_count": np.zeros(n_canvas, np.int32),
                    "step_count": np.zeros(n_canvas, np.int32)}
        self.g = {k: torch.from_numpy(v.copy()).to(DEV) for k, v in self.ref.items()}
        self.g["newly"] = torch.full((n,), 7, dtype=torch.uint8, device=DEV)
        self.g["converged"] = torch.full((n_canvas,), 7, dtype=torch.uint8, device=DEV)

    def step(self, ent, am, budget, k, tau, limit):
        B = gpu_api()
        te = torch.from_numpy(np.ascontiguousarray(ent, np.float32)).to(DEV)
        ta = torch.from_numpy(np.ascontiguousarray(am, np.int32)).to(DEV)
        g = self.g
        B.se_accept_converge(te, ta, self.L, budget, k, tau, limit, g["accepted"],
                             g["prev_argmax"], g["stable_count"], g["step_count"], g["newly"],
                             g["converged"])
        torch.cuda.synchronize()
        r = ref_accept(ent, am, self.L, budget, k, tau, limit, self.ref["accepted"],
                       self.ref["prev_argmax"], self.ref["stable_count"], self.ref["step_count"])
        for key in ("accepted", "prev_argmax", "stable_count", "step_count"):
            self.ref[key] = r[key]
            assert np.array_equal(g[key].cpu().numpy(), r[key]), key
        assert np.array_equal(g["newly"].cpu().numpy(), r["newly"]), "newly"
        assert np.array_equal(g["converged"].cpu().numpy(), r["converged"]), "converged"
        return r


@pytest.mark.parametrize("n_canvas,L", [(8, 256), (1, 1), (3, 17), (2, 1024), (5, 255)])
def test_multi_step_parity(n_canvas, L):
    rng = np.random.default_rng(1000 * n_canvas + L)
    st = Pair(n_canvas, L)
    am = rng.integers(0, 50, n_canvas * L).astype(np.int32)
    for step in range(6):
        ent = rng.exponential(1.0, n_canvas * L).astype(np.float32)
        # argmax settles: a shrinking share of positions still changes
        change = rng.random(n_canvas * L) < (0.5 if step < 3 else 0.0)
        am = np.where(change, rng.integers(0, 50, n_canvas * L), am).astype(np.int32)
        budget = [0.0, 0.5, 3.0, 40.0, 1e9, 2.0][step]
        st.step(ent, am, budget, k=2, tau=1.2, limit=5)


def test_ties_signed_zeros_and_tiny_negatives():
    rng = np.random.default_rng(7)
    L = 256
    vals = np.float32([0.0, -0.0, -1e-8, 1e-30, 0.25, 0.25, 2.0])
    st = Pair(4, L)
    for budget in (0.0, 0.25, 1.0, 8.0):
        ent = rng.choice(vals, 4 * L).astype(np.float32)
        am = np.zeros(4 * L, np.int32)
        st.step(ent, am, budget, k=1, tau=0.5, limit=100)


def test_all_accepted_canvas_and_partial_state():
    rng = np.random.default_rng(9)
    L = 64
    acc = np.zeros(3 * L, np.uint8)
    acc[:L] = 1                                    # canvas 0 fully accepted
    acc[L:2 * L] = rng.random(L) < 0.5             # canvas 1 half accepted
    st = Pair(3, L, accepted=acc)
    ent = rng.exponential(0.3, 3 * L).astype(np.float32)
    r = st.step(ent, np.arange(3 * L, dtype=np.int32), 1.0, k=3, tau=0.1, limit=50)
    assert r["newly"][:L].sum() == 0


def test_on_row_stats_of_seeded_logits():
    """Entropies and argmax from se_row_stats on two seeded canvases of 256 positions."""
    from diffusion_self_conditioning_amd import api
    from diffusion_self_conditioning_amd import workloads as wl
    w = wl.get("tiny").with_rows(512)
    x = torch.from_numpy(wl.make_logits(w)).to(DEV)
    _, _, ent, am = api.row_stats(x)
    torch.cuda.synchronize()
    st = Pair(2, 256)
    e, a = ent.cpu().numpy(), am.cpu().numpy()
    st.step(e, a, 2.0, k=1, tau=0.5, limit=10)
    st.step(e, a, 2.0, k=1, tau=0.5, limit=10)     # same argmax: stable, low entropy


def test_repeatable():
    rng = np.random.default_rng(3)
    B = gpu_api()
    L, n = 256, 4 * 256
    ent = torch.from_numpy(rng.exponential(1.0, n).astype(np.float32)).to(DEV)
    am = torch.zeros(n, dtype=torch.int32, device=DEV)
    outs = []
    for _ in range(2):
        acc = torch.zeros(n, dtype=torch.uint8, device=DEV)
        prev = torch.full((n,), -1, dtype=torch.int32, device=DEV)
        sc = torch.zeros(4, dtype=torch.int32, device=DEV)
        stc = torch.zeros(4, dtype=torch.int32, device=DEV)
        nw = torch.empty(n, dtype=torch.uint8, device=DEV)
        cv = torch.empty(4, dtype=torch.uint8, device=DEV)
        B.se_accept_converge(ent, am, L, 3.0, 2, 1.0, 10, acc, prev, sc, stc, nw, cv)
        outs.append(nw.cpu())
    assert torch.equal(outs[0], outs[1])
