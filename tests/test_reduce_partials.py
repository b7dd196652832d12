"""The on-device sum of per-rank partials (calvarado04.com/tag/vllm, "The fix":
E^sc = gamma * sum_r S^(r), result in the embedding dtype).

CPU: the oracle's pins -- a single part is the identity, dyadic parts add exactly,
the fixed order r = 0 .. T-1 is visible in fp32 (1e8 + 1 - 1e8 = 0), bf16 rounds to
nearest even.  GPU (marked): bit-exact against the oracle for random parts, and the
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
