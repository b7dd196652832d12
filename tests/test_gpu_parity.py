"""GPU parity of libsoftembed against the fp64 oracle (MI355X).

All calls go through the C ABI (ctypes binding).  Tolerances:
  argmax, row max        bit-exact
  log-sum-exp            |d| <= 2e-6 * max(1, |lse|)
  entropy                |d| <= 1e-4 nats
  soft embedding (gate)  ||gpu - ref||_F / ||ref||_F <= 5e-3, ref = exact fp64 p
  soft embedding (diag)  vs the oracle that rounds p to bf16 first: relative Frobenius
                         <= 1e-4 and, element by element, |d_ij| <= 1e-4 * gamma *
                         sum_v p_iv |W_vj| (what fp32 accumulation of bf16 products allows)
"""
import math
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
DIAG = 1e-4


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_logits(x, extra=0, fill=1e30):
    """fp32 logits on the GPU with a row pitch rounded up to 8 floats (+ extra); the padding
    columns hold a huge value that would wreck any result that read them."""
    L, V = x.shape
    ld = ((V + 7) // 8) * 8 + extra
    if ld == V:
        return dev(x)
    buf = np.full((L, ld), np.float32(fill), np.float32)
    buf[:, :V] = x
    return dev(buf)[:, :V]


def rel_fro(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


def abs_bits(bits):
    return (bits & np.uint16(0x7FFF)).astype(np.uint16)


def gpu_stats(x_np, extra=0):
    t_view = dev_logits(x_np, extra)
    mx, lse, ent, am = api.row_stats(t_view)
    torch.cuda.synchronize()
    return t_view, dict(max=mx.cpu().numpy(), lse=lse.cpu().numpy(), entropy=ent.cpu().numpy(),
                        argmax=am.cpu().numpy())


def check_stats(g, r, rows=None):
    idx = slice(None) if rows is None else rows
    np.testing.assert_array_equal(g["argmax"][idx], r["argmax"])
    np.testing.assert_array_equal(g["max"][idx].astype(np.float64), r["max"])
    lse_tol = 2e-6 * np.maximum(1.0, np.abs(r["lse"]))
    assert np.all(np.abs(g["lse"][idx] - r["lse"]) <= lse_tol), \
        np.max(np.abs(g["lse"][idx] - r["lse"]) / lse_tol)
    assert np.max(np.abs(g["entropy"][idx] - r["entropy"])) <= 1e-4


def gpu_soft_embed(x_t, lse_t, s, e, w_t, gamma, fused, w_rows=None, out=None):
    n, d = x_t.shape[0], w_t.shape[1]
    if out is None:
        out = torch.full((n, d), float("nan"), device=DEV, dtype=torch.float32)
    ws = api.workspace(n, s, e, d, DEV)
    if fused:
        B.se_soft_embed_fused(x_t, lse_t, s, e, w_t, gamma, out, ws, w_rows=w_rows)
    else:
        V = x_t.shape[1]
        p = torch.zeros((n, ((V + 7) // 8) * 8), device=DEV, dtype=torch.bfloat16)[:, :V]
        B.se_probs_bf16(x_t, lse_t, s, e, p)
        B.se_soft_embed(p, s, e, w_t, gamma, out, ws, w_rows=w_rows)
    torch.cuda.synchronize()
    return out


def check_embed(got, x_np, s, e, shard_bits, gamma, shard_f32=None, rows=None):
    """Gate against the exact oracle (fp32 table when there is one) and the bf16 diagnostic."""
    xr = x_np if rows is None else x_np[rows]
    g = got if rows is None else got[rows]
    exact = oracle.soft_embed(xr, s, e, shard_f32 if shard_f32 is not None else shard_bits, gamma)
    diag = oracle.soft_embed(xr, s, e, shard_bits, gamma, round_p_bf16=True)
    scale = oracle.soft_embed(xr, s, e, abs_bits(shard_bits), gamma)
    assert np.all(np.isfinite(g))
    r_gate, r_diag = rel_fro(g, exact), rel_fro(g, diag)
    say(f"rel_fro gate={r_gate:.3e} diag={r_diag:.3e}")
    assert r_gate <= GATE, r_gate
    assert r_diag <= DIAG, r_diag
    bad = np.abs(g - diag) > DIAG * np.abs(scale) + 1e-30
    assert not bad.any(), (np.argwhere(bad)[:5], np.max(np.abs(g - diag) / (np.abs(scale) + 1e-30)))
    return r_gate


# ----------------------------------------------------------------------------- row stats
ROW_CASES = {
    "tiny": lambda: wl.make_logits(wl.get("tiny")),
    "tiny-diffuse": lambda: wl.make_logits(wl.get("tiny"), plant="none"),
    "ragged-V": lambda: np.random.default_rng(3).standard_normal((37, 4099), dtype=np.float32) * 3,
    "one-hot": lambda: wl.one_hot_logits(5, 1000, [0, 999, 17, 512, 3]),
    "uniform-4096": lambda: wl.uniform_logits(3, 4096, 0.25),
    "uniform-262144": lambda: wl.uniform_logits(2, 262144, -1.5),
    "V1": lambda: np.array([[3.5], [-2.0]], np.float32),
    "V3": lambda: np.array([[1.0, 7.0, 7.0], [0.0, 0.0, 0.0]], np.float32),
    "ties": lambda: np.tile(np.array([[1.0, 5.0, 2.0, 5.0, 5.0, 0.0, 0.0, 5.0]], np.float32), (2, 512)),
    "large-values": lambda: (np.random.default_rng(4).standard_normal((8, 5000)) * 30 + 500).astype(np.float32),
    "one-hot-underflow": lambda: wl.one_hot_logits(2, 70000, [69999, 5], hot=100.0, cold=-100.0),
}


@pytest.mark.parametrize("case", sorted(ROW_CASES))
@pytest.mark.parametrize("pad", [0, 12])
def test_row_stats_parity(case, pad):
    x = ROW_CASES[case]()
    say("row_stats", case, x.shape, "pad", pad)
    _, g = gpu_stats(x, pad)
    check_stats(g, oracle.row_stats(x))


def test_row_stats_closed_forms():
    say("row_stats closed forms")
    _, g = gpu_stats(wl.uniform_logits(2, 262144, 0.0))
    assert np.all(np.abs(g["entropy"] - math.log(262144)) <= 1e-4)
    assert np.all(g["argmax"] == 0)
    _, g = gpu_stats(wl.one_hot_logits(3, 4096, [7, 0, 4095]))
    assert list(g["argmax"]) == [7, 0, 4095]
    assert np.all(np.abs(g["entropy"]) <= 1e-4) and np.all(g["lse"] == 0.0)


# ------------------------------------------------------------------------- soft embedding
def _ragged_case(plant):
    rng = np.random.default_rng(11)
    L, V, d, s, e = 300, 20011, 520, 1024, 17003
    x = rng.standard_normal((L, V), dtype=np.float32) * np.float32(3.0)
    if plant:
        ks = rng.integers(s, e, size=L)
        x[np.arange(L), ks] = x.max(axis=1) + np.float32(8.0)
    table = wl.fp32_to_bf16_bits(rng.standard_normal((V, d), dtype=np.float32) * np.float32(0.02))
    return x, s, e, table[s:], None, 7.25


def _tiny_case(plant):
    w = wl.get("tiny")
    x = wl.make_logits(w, plant=None if plant else "none")
    bits, f32 = wl.make_table(w)
    return x, 0, w.vocab, bits, f32, w.gamma


def _one_hot_case(_):
    rng = np.random.default_rng(5)
    V, d = 3000, 264
    ks = [0, 7, 1500, 2999, 100, 2047]
    x = wl.one_hot_logits(len(ks), V, ks)
    table = wl.fp32_to_bf16_bits(rng.standard_normal((V, d), dtype=np.float32) * np.float32(0.02))
    return x, 0, V, table, None, 53.065998


def _uniform_case(_):
    rng = np.random.default_rng(6)
    V, d = 8192, 256
    table = wl.fp32_to_bf16_bits(rng.standard_normal((V, d), dtype=np.float32) * np.float32(0.02))
    return wl.uniform_logits(33, V, 1.0), 0, V, table, None, 16.0


EMBED_CASES = {
    "tiny": lambda: _tiny_case(True),
    "tiny-diffuse": lambda: _tiny_case(False),
    "ragged": lambda: _ragged_case(True),
    "ragged-diffuse": lambda: _ragged_case(False),
    "one-hot": lambda: _one_hot_case(None),
    "uniform": lambda: _uniform_case(None),
}


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
@pytest.mark.parametrize("case", sorted(EMBED_CASES))
def test_soft_embed_parity(case, fused):
    x, s, e, shard, shard_f32, gamma = EMBED_CASES[case]()
    say("soft_embed", case, "fused" if fused else "unfused", x.shape, (s, e), shard.shape)
    x_t = dev_logits(x)
    _, lse, _, _ = api.row_stats(x_t)
    got = gpu_soft_embed(x_t, lse, s, e, dev(shard), gamma, fused).cpu().numpy()
    check_embed(got, x, s, e, shard, gamma, shard_f32)


def test_closed_forms_on_gpu():
    """one-hot rows return gamma * W[k]; uniform rows return gamma * column mean."""
    x, s, e, shard, _, gamma = _one_hot_case(None)
    say("closed forms one-hot")
    x_t = dev_logits(x)
    _, lse, _, _ = api.row_stats(x_t)
    got = gpu_soft_embed(x_t, lse, s, e, dev(shard), gamma, True).cpu().numpy()
    rows = wl.bf16_bits_to_fp32(shard[[0, 7, 1500, 2999, 100, 2047]]).astype(np.float64)
    np.testing.assert_allclose(got, np.float32(gamma) * rows, rtol=2e-6, atol=1e-7)
    x, s, e, shard, _, gamma = _uniform_case(None)
    say("closed forms uniform")
    x_t = dev_logits(x)
    _, lse, _, _ = api.row_stats(x_t)
    got = gpu_soft_embed(x_t, lse, s, e, dev(shard), gamma, True).cpu().numpy()
    mean = wl.bf16_bits_to_fp32(shard).astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(got, np.broadcast_to(gamma * mean, got.shape), rtol=1e-4, atol=1e-6)


def test_fused_equals_unfused_bitwise_and_repeatable():
    x, s, e, shard, _, gamma = _ragged_case(False)
    say("bitwise fused/unfused/repeat")
    x_t, w_t = dev_logits(x), dev(shard)
    _, lse, _, _ = api.row_stats(x_t)
    a = gpu_soft_embed(x_t, lse, s, e, w_t, gamma, True)
    b = gpu_soft_embed(x_t, lse, s, e, w_t, gamma, True)
    c = gpu_soft_embed(x_t, lse, s, e, w_t, gamma, False)
    assert torch.equal(a, b)
    assert torch.equal(a, c)


@pytest.mark.parametrize("bounds", [[0, 20008], [0, 10000, 20008], [0, 4096, 8192, 12288, 20008],
                                    [0, 8, 2504, 5000, 7504, 10000, 12504, 15000, 20008]])
def test_partition_sum_matches_full_call(bounds):
    rng = np.random.default_rng(21)
    L, V, d = 70, 20008, 264
    x = rng.standard_normal((L, V), dtype=np.float32) * np.float32(3.0)
    table = wl.fp32_to_bf16_bits(rng.standard_normal((V, d), dtype=np.float32) * np.float32(0.02))
    say("partition", bounds)
    x_t, tab = dev_logits(x), dev(table)
    _, lse, _, _ = api.row_stats(x_t)
    full = gpu_soft_embed(x_t, lse, 0, V, tab, 1.0, True).cpu().numpy().astype(np.float64)
    parts = sum(gpu_soft_embed(x_t, lse, a, b, tab[a:b], 1.0, True).cpu().numpy().astype(np.float64)
                for a, b in zip(bounds[:-1], bounds[1:]))
    assert rel_fro(parts, full) <= 1e-5


def test_padding_never_read_and_guard_bands():
    """The last rank's shard carries padding rows: fill them with NaN.  Write the output into a
    larger buffer: values outside [0, L) x [0, d) must stay untouched."""
    rng = np.random.default_rng(8)
    L, V, d, s = 40, 4096, 136, 3072
    pad_rows = 64
    x = rng.standard_normal((L, V), dtype=np.float32) * np.float32(3.0)
    table = wl.fp32_to_bf16_bits(rng.standard_normal((V, d), dtype=np.float32) * np.float32(0.02))
    shard = np.concatenate([table[s:], np.full((pad_rows, d), 0x7FC0, np.uint16)])
    say("padding poison + guard bands")
    x_t = dev_logits(x)
    _, lse, _, _ = api.row_stats(x_t)
    for fused in (True, False):
        big = torch.full((L + 3, d + 12), 12345.0, device=DEV, dtype=torch.float32)
        out = big[1:L + 1, 4:4 + d]
        gpu_soft_embed(x_t, lse, s, V, dev(shard), 2.5, fused, out=out)
        bn = big.cpu().numpy()
        assert np.all(bn[0] == 12345.0) and np.all(bn[L + 1:] == 12345.0)
        assert np.all(bn[:, :4] == 12345.0) and np.all(bn[:, 4 + d:] == 12345.0)
        check_embed(bn[1:L + 1, 4:4 + d], x, s, V, shard, 2.5)


def test_degenerate_shapes():
    rng = np.random.default_rng(9)
    say("degenerate shapes")
    # empty slice -> zeros
    x = rng.standard_normal((5, 64), dtype=np.float32)
    x_t = dev_logits(x)
    _, lse, _, _ = api.row_stats(x_t)
    tab = dev(wl.fp32_to_bf16_bits(rng.standard_normal((64, 16), dtype=np.float32)))
    out = gpu_soft_embed(x_t, lse, 32, 32, tab[32:], 3.0, True)
    assert torch.count_nonzero(out).item() == 0
    # zero rows: no-op, output untouched
    empty = torch.empty((0, 64), device=DEV)
    o = torch.empty((0, 16), device=DEV)
    B.se_soft_embed_fused(empty, torch.empty(0, device=DEV), 0, 64, tab, 1.0, o)
    # vocabulary of one, single row, narrow hidden size
    for L, V, d, s, e in [(1, 1, 8, 0, 1), (1, 9, 8, 8, 9), (3, 64, 8, 0, 64), (17, 136, 16, 8, 129)]:
        x = rng.standard_normal((L, V), dtype=np.float32)
        table = wl.fp32_to_bf16_bits(rng.standard_normal((V, d), dtype=np.float32) * np.float32(0.5))
        x_t = dev_logits(x)
        _, lse, _, _ = api.row_stats(x_t)
        for fused in (True, False):
            got = gpu_soft_embed(x_t, lse, s, e, dev(table[s:]), 1.5, fused).cpu().numpy()
            check_embed(got, x, s, e, table[s:], 1.5)


def test_errors_leave_outputs_untouched():
    say("error path on GPU buffers")
    x = dev(np.zeros((4, 256), np.float32))
    lse = torch.zeros(4, device=DEV)
    tab = torch.zeros((64, 16), device=DEV, dtype=torch.int16)
    out = torch.full((4, 16), 7.0, device=DEV)
    with pytest.raises(B.SoftEmbedError) as ei:
        B.se_soft_embed_fused(x, lse, 0, 256, tab, 1.0, out)          # 256-long slice, 64-row shard
    assert ei.value.status == B.SE_ERR_SLICE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# ---------------------------------------------------------- full sizes (sampled outputs)
FULL = ["rank", "full", "conv", "batch"]


@pytest.fixture(scope="module")
def tables():
    cache = {}

    def get(name):
        w = wl.get(name)
        key = (w.seed, w.table_rows)
        if key not in cache:
            cache.clear()
            bits, _ = wl.make_table(w)
            cache[key] = (bits, dev(bits))
        return cache[key]
    return get


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name, tables):
    w = wl.get(name)
    say("full-size", name, "generating inputs")
    bits, tab_t = tables(name)
    x = wl.make_logits(w)
    rng = np.random.default_rng(100 + w.seed)
    srows = np.unique(np.concatenate([[0, w.rows - 1], rng.integers(0, w.rows, 2)]))
    stat_rows = np.unique(np.concatenate([srows, rng.integers(0, w.rows, 28)]))
    say("full-size", name, "gpu calls")
    x_t = dev_logits(x)
    mx, lse, ent, am = api.row_stats(x_t)
    shard_t = tab_t[w.vocab_start:w.vocab_end]
    out = gpu_soft_embed(x_t, lse, w.vocab_start, w.vocab_end, shard_t, w.gamma, True,
                         w_rows=w.k).cpu().numpy()
    g = dict(max=mx.cpu().numpy(), lse=lse.cpu().numpy(), entropy=ent.cpu().numpy(),
             argmax=am.cpu().numpy())
    say("full-size", name, "oracle on sampled rows", list(srows))
    check_stats(g, oracle.row_stats(x[stat_rows]), rows=stat_rows)
    np.testing.assert_array_equal(g["argmax"], wl.planted_index(w))     # planted argmax, all rows
    check_embed(out, x, w.vocab_start, w.vocab_end, bits[w.vocab_start:w.vocab_end], w.gamma,
                rows=srows)
    if name == "conv":
        assert np.all(np.abs(g["entropy"] - 0.0178) < 0.003)


def test_full_size_rank_diffuse_and_partition(tables):
    """Diffuse companion of the one-rank workload (no planted max), and the four-rank partition
    of the full vocabulary summed on the host against one full-vocabulary call."""
    w = wl.get("rank")
    bits, tab_t = tables("rank")
    x = wl.make_logits(w, plant="none")
    say("full-size rank diffuse")
    x_t = dev_logits(x)
    _, lse, _, _ = api.row_stats(x_t)
    out = gpu_soft_embed(x_t, lse, w.vocab_start, w.vocab_end, tab_t[w.vocab_start:w.vocab_end],
                         w.gamma, True).cpu().numpy()
    check_embed(out, x, w.vocab_start, w.vocab_end, bits[w.vocab_start:w.vocab_end], w.gamma,
                rows=np.array([0, 77, 255]))
    say("full-size 4-rank partition")
    V = w.vocab
    full = gpu_soft_embed(x_t, lse, 0, V, tab_t[:V], w.gamma, True).cpu().numpy().astype(np.float64)
    q = V // 4
    parts = sum(gpu_soft_embed(x_t, lse, r * q, (r + 1) * q, tab_t[r * q:(r + 1) * q], w.gamma,
                               True).cpu().numpy().astype(np.float64) for r in range(4))
    assert rel_fro(parts, full) <= 1e-5
    # last rank with its padding rows poisoned: never read
    pad = tab_t[3 * q:].clone().view(torch.int16)
    pad[q:] = 0x7FC0                                  # bf16 NaN
    last = gpu_soft_embed(x_t, lse, 3 * q, V, pad, w.gamma, True, w_rows=pad.shape[0])
    assert torch.isfinite(last).all()
