"""The on-device sum of per-rank partials (calvarado04.com/tag/vllm, "The fix":
E^sc = gamma * sum_r S^(r), result in the embedding dtype).

CPU: the oracle's pins -- a single part is the identity, dyadic parts add exactly,
the fixed order r = 0 .. T-1 is visible in fp32 (1e8 + 1 - 1e8 = 0), bf16 rounds to
nearest even as torch's CPU cast does, and the fp32 sum lies within the classical bound
(T - 1) u sum |x_r| of the exact sum (math.fsum), whatever the order.  GPU (marked): bit-exact against the oracle for random parts, and the
partition identity end to end: four rank slices of the fused call, summed on the GPU,
match one full-slice call.
"""
import numpy as np
import pytest

from oracle.reduce import reduce_partials


def test_single_part_is_identity():
    x = np.random.default_rng(0).standard_normal((3, 8)).astype(np.float32)
    s, _ = reduce_partials(x[None])
    assert np.array_equal(s, x)


def test_dyadic_parts_add_exactly():
    parts = np.array([[[0.5]], [[0.25]], [[0.125]]], np.float32)
    s, b = reduce_partials(parts)
    assert s[0, 0] == np.float32(0.875)
    assert b[0, 0] == 0x3F60                   # 0.875 = 1.75 * 2^-1 in bf16


def test_order_is_fixed():
    parts = np.array([[[1e8]], [[1.0]], [[-1e8]]], np.float32)
    s, _ = reduce_partials(parts)
    assert s[0, 0] == 0.0                       # (1e8 + 1) rounds to 1e8 in fp32
    s2, _ = reduce_partials(parts[[0, 2, 1]])
    assert s2[0, 0] == 1.0


def test_bf16_ties_to_even():
    one_half_ulp = np.float32(1.0 + 2.0 ** -8)   # halfway between bf16 1.0 and 1.0078125
    three_half = np.float32(1.0 + 3 * 2.0 ** -8)  # halfway between 1.0078125 and 1.015625
    _, b = reduce_partials(np.array([[[one_half_ulp, three_half]]], np.float32))
    assert b[0].tolist() == [0x3F80, 0x3F82]


def _exact_sum(parts):
    """The exact sum over axis 0 of fp32 values, element by element (math.fsum is exact up to
    its final rounding to double, far below fp32's)."""
    import math
    t = parts.shape[0]
    flat = parts.reshape(t, -1).astype(np.float64)
    return np.array([math.fsum(flat[:, j]) for j in range(flat.shape[1])]).reshape(parts.shape[1:])


def _within_fp32_sum_bound(got, parts):
    """Any order of T - 1 fp32 additions stays within (T - 1) u sum |x_r| of the exact sum
    (u = 2^-24; the classical bound for recursive summation)."""
    t = parts.shape[0]
    bound = (t - 1) * 2.0 ** -24 * np.abs(parts.astype(np.float64)).sum(axis=0) * (1 + 1e-6)
    return np.all(np.abs(got.astype(np.float64) - _exact_sum(parts)) <= bound)


def test_sum_is_the_exact_sum_within_the_fp32_bound():
    rng = np.random.default_rng(5)
    for t in (1, 2, 4, 8, 23):
        parts = (rng.standard_normal((t, 7, 33)) * 10.0 ** rng.integers(-4, 5, (t, 7, 33))).astype(np.float32)
        s, _ = reduce_partials(parts)
        assert _within_fp32_sum_bound(s, parts)
        if t == 1:
            assert np.array_equal(s, parts[0])


def test_bf16_output_is_torch_cast_of_the_sum():
    import torch
    rng = np.random.default_rng(6)
    parts = (rng.standard_normal((4, 9, 65)) * 3).astype(np.float32)
    s, b = reduce_partials(parts)
    want = torch.from_numpy(s).to(torch.bfloat16).view(torch.uint16).numpy().astype(np.uint16)
    assert np.array_equal(b, want)


@pytest.mark.gpu
@pytest.mark.parametrize("t,n,d,ld", [(1, 4, 4, 4), (2, 17, 8, 12), (4, 256, 2816, 2816),
                                      (8, 3, 64, 64)])
def test_gpu_bit_exact(t, n, d, ld):
    import torch
    from diffusion_self_conditioning_amd import _binding as B
    rng = np.random.default_rng(t * 100 + n)
    parts = (rng.standard_normal((t, n, ld)) * 10.0 ** rng.integers(-3, 4, (t, n, ld))).astype(np.float32)
    dev = torch.device("cuda:0")
    tp = torch.from_numpy(parts).to(dev)
    out = torch.full((n, d + 4), 7.0, device=dev)[:, :d]
    ob = torch.zeros((n, d + 4), dtype=torch.bfloat16, device=dev)[:, :d]
    B.se_reduce_partials(tp[:, :, :d] if ld == d else tp, out=out, out_bf16=ob)
    torch.cuda.synchronize()
    want, wbits = reduce_partials(parts[:, :, :d])
    assert _within_fp32_sum_bound(out.cpu().numpy(), parts[:, :, :d])
    assert np.array_equal(out.cpu().numpy(), want)
    assert np.array_equal(ob.cpu().view(torch.uint16).numpy().astype(np.uint16), wbits)


@pytest.mark.gpu
def test_gpu_partition_end_to_end():
    import torch
    import oracle
    from diffusion_self_conditioning_amd import _binding as B
    from diffusion_self_conditioning_amd import api
    from diffusion_self_conditioning_amd import workloads as wl
    w = wl.get("tiny")
    dev = torch.device("cuda:0")
    x_np = wl.make_logits(w)
    bits, f32 = wl.make_table(w)
    x = torch.from_numpy(x_np).to(dev)
    table = torch.from_numpy(bits).to(dev)
    _, lse, _, _ = api.row_stats(x)
    T, V = 4, w.vocab
    parts = torch.empty((T, w.rows, w.d), device=dev)
    for r in range(T):
        s, e = r * V // T, (r + 1) * V // T
        ws = api.workspace(w.rows, s, e, w.d, dev)
        B.se_soft_embed_fused(x, lse, s, e, table[s:e], w.gamma, parts[r], ws)
    full = api.soft_embed(x, lse, 0, V, table, w.gamma, fused=True)
    out = torch.empty((w.rows, w.d), device=dev)
    ob = torch.empty((w.rows, w.d), dtype=torch.bfloat16, device=dev)
    B.se_reduce_partials(parts, out=out, out_bf16=ob)
    torch.cuda.synchronize()
    got, ref_full = out.double().cpu().numpy(), full.double().cpu().numpy()
    assert np.linalg.norm(got - ref_full) / np.linalg.norm(ref_full) <= 1e-5
    want = oracle.soft_embed(x_np, 0, V, f32, w.gamma)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= 5e-3
    _, wbits = reduce_partials(parts.cpu().numpy())
    assert np.array_equal(ob.cpu().view(torch.uint16).numpy().astype(np.uint16), wbits)
