"""GPU parity of the e4m3 table path: se_quantize_table_fp8, se_soft_embed_fp8,
se_soft_embed_fp8_fused, se_soft_embed_step_fp8 and se_soft_embed_step_onepass_fp8
(MI355X), all through the C ABI.

Bars:
  quantizer                codes and scales bit-exact with oracle.fp8.quantize_table
  contraction vs oracle    relative Frobenius <= 5e-3 against the fp64 soft embedding of
                           the oracle's dequantized table (the gate of the bf16 path)
  contraction vs bf16 path bit-exact: the e4m3 kernels on the oracle's codes equal the
                           bf16 kernels on the oracle's dequantized bf16 table (code x
                           power-of-two scale is exact in bf16; same accumulation order)
  decode                   a one-hot probability row returns code value x scale exactly,
                           for every finite code
  one-read e4m3 step       bit-exact with the bf16 one-read step on the dequantized table
                           (the sweep stores each probability times its row's power-of-two
                           scale and the contraction reads the codes as they are), and the
                           oracle gate
The table inputs of the GPU contraction are the oracle's codes, never the GPU
quantizer's, so no expected value depends on the HIP path.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
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


def padded(a, ld, fill):
    """2-D device tensor view [rows, cols] of a buffer with row pitch ld, padding = fill."""
    rows, cols = a.shape
    buf = np.full((rows, ld), fill, dtype=a.dtype)
    buf[:, :cols] = a
    return dev(buf)[:, :cols]


def gpu_quantize(bits, ld_w=None, ld_q=None):
    rows, d = bits.shape
    w_t = padded(bits, ld_w or d, np.uint16(0x7FC0))
    c_t = padded(np.zeros((rows, d), np.uint8), ld_q or d, np.uint8(0xA5))
    s_t = torch.full((rows,), float("nan"), device=DEV)
    B.se_quantize_table_fp8(w_t, c_t, s_t)
    torch.cuda.synchronize()
    return c_t, s_t


def check_quantizer(bits, ld_w=None, ld_q=None):
    c_t, s_t = gpu_quantize(bits, ld_w, ld_q)
    codes, scale = fp8.quantize_table(bits)
    got_c, got_s = c_t.cpu().numpy(), s_t.cpu().numpy()
    bad = np.argwhere(got_c != codes)
    assert bad.size == 0, [(tuple(i), hex(got_c[tuple(i)]), hex(codes[tuple(i)]),
                            hex(bits[tuple(i)])) for i in bad[:8]]
    np.testing.assert_array_equal(got_s, scale)
    if ld_q:   # the pitch padding of the codes buffer is untouched
        full = c_t.as_strided((c_t.shape[0], ld_q), (ld_q, 1)).cpu().numpy()
        assert np.all(full[:, bits.shape[1]:] == 0xA5)


def crafted_table(d=64):
    """Rows that exercise every rounding case of the quantizer."""
    mags = fp8._MAGS
    mids = (mags[1:] + mags[:-1]) / 2                 # exact ties, 5 significant bits at most
    base = np.concatenate([[448.0], mids, -mids[::3], mags[::5]])
    rows = []
    rows.append(np.zeros(d))                          # all zero
    rows.append(-np.zeros(d))                         # negative zeros
    r = np.zeros(d); r[7] = 1.0; rows.append(r)       # a single one
    for j in (-20, -8, 0, 5, 100):                    # ties at several scales
        for o in range(0, len(base), d):
            chunk = base[o:o + d]
            rr = np.zeros(d); rr[:len(chunk)] = chunk; rr[0] = 448.0
            rows.append(rr * 2.0 ** j)
    rows.append(np.linspace(-3e38, 3e38, d))          # near the bf16 maximum
    rows.append(np.full(d, 1.5 * 2.0 ** -130))        # bf16 subnormals: k clamps at -126
    rows.append(np.linspace(-1e-30, 1e-30, d))
    rng = np.random.default_rng(21)
    rows.extend(rng.standard_normal((20, d)) * 0.02)
    t = np.array(rows, dtype=np.float32)
    return (t.view(np.uint32) >> 16).astype(np.uint16)   # all values above are bf16-exact


def test_quantizer_tiny_table():
    w = wl.get("tiny")
    bits, _ = wl.make_table(w)
    say("quantize tiny", bits.shape)
    check_quantizer(bits)


@pytest.mark.parametrize("d,ld_w,ld_q", [(64, None, None), (64, 72, 80), (16, 24, 32), (48, None, 64)])
def test_quantizer_crafted_rows(d, ld_w, ld_q):
    bits = crafted_table(d)
    say("quantize crafted", bits.shape, ld_w, ld_q)
    check_quantizer(bits, ld_w, ld_q)


def test_decode_every_code_one_hot():
    """Row i of P is one-hot at vocab i (exactly 1.0 in bf16): out[i] = code x scale."""
    K, d = 256, 16
    codes = ((np.arange(K)[:, None] + 16 * np.arange(d)[None, :]) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00               # NaN codes are not table values
    scale = np.float32(2.0) ** (np.arange(K) % 41 - 20).astype(np.float32)
    want = fp8.dequantize(codes, scale)
    c_t, s_t = dev(codes), dev(scale)
    probs = np.zeros((K, K), np.uint16)
    probs[np.arange(K), np.arange(K)] = 0x3F80
    out = torch.full((K, d), float("nan"), device=DEV)
    ws = api.workspace(K, 0, K, d, DEV)
    say("decode unfused")
    B.se_soft_embed_fp8(dev(probs), 0, K, c_t, s_t, 1.0, out, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().astype(np.float64), want)
    say("decode fused")
    x = wl.one_hot_logits(K, K, np.arange(K), hot=0.0, cold=-200.0)
    x_t = dev(x)
    _, lse, _, _ = api.row_stats(x_t)
    out2 = torch.full((K, d), float("nan"), device=DEV)
    B.se_soft_embed_fp8_fused(x_t, lse, 0, K, c_t, s_t, 1.0, out2, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out2.cpu().numpy().astype(np.float64), want)


def _pair(x, s, e, codes, scale, gamma, pad_rows=0, d_view=None):
    """(fp8 fused, fp8 unfused, bf16 fused, bf16 unfused) outputs on the same inputs; the
    e4m3 shard gets pad_rows rows of NaN codes / NaN scales after the slice."""
    K, d = codes.shape[0], codes.shape[1]
    cpad = np.concatenate([codes, np.full((pad_rows, d), 0x7F, np.uint8)])
    spad = np.concatenate([scale, np.full(pad_rows, np.nan, np.float32)])
    dq = fp8.dequantize_bf16_bits(codes, scale)
    c_t, s_t, dq_t = dev(cpad), dev(spad), dev(dq)
    x_t = dev(x)
    L = x.shape[0]
    _, lse, _, _ = api.row_stats(x_t)
    ws = api.workspace(L, s, e, d, DEV)
    outs = []
    for fn in ("fp8_fused", "fp8", "bf16_fused", "bf16"):
        o = torch.full((L, d), float("nan"), device=DEV)
        if fn == "fp8_fused":
            B.se_soft_embed_fp8_fused(x_t, lse, s, e, c_t, s_t, gamma, o, ws)
        elif fn == "bf16_fused":
            B.se_soft_embed_fused(x_t, lse, s, e, dq_t, gamma, o, ws)
        else:
            V = x.shape[1]
            p = torch.zeros((L, ((V + 7) // 8) * 8), device=DEV, dtype=torch.bfloat16)[:, :V]
            B.se_probs_bf16(x_t, lse, s, e, p)
            if fn == "fp8":
                B.se_soft_embed_fp8(p, s, e, c_t, s_t, gamma, o, ws)
            else:
                B.se_soft_embed(p, s, e, dq_t, gamma, o, ws)
        torch.cuda.synchronize()
        outs.append(o)
    return outs, dq


CASES = {
    # name: (L, V, s, e, d, seed)
    "tiny": (16, 4096, 0, 4096, 256, 1),
    "ragged": (17, 20008, 8, 20008, 48, 2),
    "slice-1": (5, 1000, 16, 17, 16, 3),
    "slice-63": (33, 1000, 64, 127, 2816, 4),
    "slice-4097": (255, 8200, 8, 4105, 272, 5),
    "two-tiles-rows": (300, 2048, 0, 2048, 512, 6),
    # whole 256-row tiles (staged probabilities take the ping-pong contraction): a tail of
    # one position, two row tiles with a 72-position tail, a tail alone, a held slice
    "whole-tile-tail": (256, 8200, 8, 4105, 272, 7),
    "two-whole-tiles": (512, 5000, 40, 240, 256, 8),
    "whole-tile-k63": (256, 1004, 64, 127, 2816, 9),
    "whole-tile-held-slice": (256, 65536, 16384, 49152, 512, 10),
    "whole-tile-d16": (256, 5000, 0, 4097, 16, 11),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_fp8_contraction_parity(case):
    L, V, s, e, d, seed = CASES[case]
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    tab = (rng.standard_normal((e - s, d)) * 0.02).astype(np.float32)
    bits = (tab.view(np.uint32) >> 16).astype(np.uint16)
    codes, scale = fp8.quantize_table(bits)
    say("fp8 contraction", case, (L, V, s, e, d))
    (f8f, f8u, bff, bfu), dq = _pair(x, s, e, codes, scale, 7.5, pad_rows=24)
    assert torch.equal(f8f, bff), "fp8 fused != bf16 fused on the dequantized table"
    assert torch.equal(f8u, bfu), "fp8 != bf16 on the dequantized table"
    assert torch.equal(f8f, f8u), "fp8 fused != fp8 unfused"
    ref = oracle.soft_embed(x, s, e, fp8.dequantize(codes, scale).astype(np.float32), 7.5)
    r = rel_fro(f8f.cpu().numpy(), ref)
    say("rel_fro", f"{r:.3e}")
    assert r <= GATE


def test_fp8_quantization_error_against_the_bf16_table():
    """Not a parity bar: the size of the e4m3 table's effect on the soft embedding."""
    L, V, d = 64, 8192, 256
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    bits = ((rng.standard_normal((V, d)) * 0.02).astype(np.float32).view(np.uint32) >> 16
            ).astype(np.uint16)
    codes, scale = fp8.quantize_table(bits)
    (f8f, _, _, _), _ = _pair(x, 0, V, codes, scale, 16.0)
    ref_bf16 = oracle.soft_embed(x, 0, V, bits, 16.0)
    r = rel_fro(f8f.cpu().numpy(), ref_bf16)
    say("e4m3 vs bf16 table rel_fro", f"{r:.3e}")
    assert r < 0.05


def test_fp8_rank_full_size():
    """One tensor-parallel rank at its real shape (L=256, slice [65536, 131072) of the
    262,400-row table, d=2816): the quantizer over the whole shard bit-exact with the
    oracle, the e4m3 fused call bit-exact with the bf16 fused call on the dequantized
    table, and sampled rows against the fp64 oracle."""
    w = wl.get("rank")
    say("fp8 rank: generating table")
    bits, _ = wl.make_table(w)
    shard = np.ascontiguousarray(bits[w.vocab_start:w.vocab_end])
    del bits
    say("fp8 rank: gpu quantize")
    c_t, s_t = gpu_quantize(shard)
    say("fp8 rank: oracle quantize")
    codes, scale = fp8.quantize_table(shard)
    assert np.array_equal(c_t.cpu().numpy(), codes)
    np.testing.assert_array_equal(s_t.cpu().numpy(), scale)
    del c_t, s_t
    x = wl.make_logits(w)
    say("fp8 rank: gpu calls")
    (f8f, f8u, bff, bfu), dq = _pair(x, w.vocab_start, w.vocab_end, codes, scale, w.gamma)
    assert torch.equal(f8f, bff)
    assert torch.equal(f8u, bfu)
    rows = np.array([0, 100, 255])
    say("fp8 rank: oracle rows", list(rows))
    ref = oracle.soft_embed(x[rows], w.vocab_start, w.vocab_end, dq, w.gamma)
    r = rel_fro(f8f.cpu().numpy()[rows], ref)
    say("rel_fro", f"{r:.3e}")
    assert r <= GATE


@pytest.mark.parametrize("case", sorted(CASES))
def test_fp8_step_equals_row_stats_then_fp8_fused(case):
    """se_soft_embed_step_fp8: statistics bitwise se_row_stats', embedding bitwise
    se_soft_embed_fp8_fused's on the oracle's codes (NaN codes and scales past the slice,
    never read), and within the gate of the fp64 oracle on the dequantized table."""
    L, V, s, e, d, seed = CASES[case]
    rng = np.random.default_rng(seed + 50)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    tab = (rng.standard_normal((e - s, d)) * 0.02).astype(np.float32)
    bits = (tab.view(np.uint32) >> 16).astype(np.uint16)
    codes, scale = fp8.quantize_table(bits)
    c_t = dev(np.concatenate([codes, np.full((24, d), 0x7F, np.uint8)]))
    s_t = dev(np.concatenate([scale, np.full(24, np.nan, np.float32)]))
    x_t = dev(x)
    say("fp8 step", case, (L, V, s, e, d))
    out, mx, lse, ent, am = api.soft_embed_step_fp8(x_t, s, e, c_t, s_t, 7.5)
    mx2, lse2, ent2, am2 = api.row_stats(x_t)
    ref = torch.full((L, d), float("nan"), device=DEV)
    B.se_soft_embed_fp8_fused(x_t, lse2, s, e, c_t, s_t, 7.5, ref, api.workspace(L, s, e, d, DEV))
    torch.cuda.synchronize()
    for a, b in ((mx, mx2), (lse, lse2), (ent, ent2), (am, am2), (out, ref)):
        assert torch.equal(a, b)
    r = rel_fro(out.cpu().numpy(),
                oracle.soft_embed(x, s, e, fp8.dequantize(codes, scale).astype(np.float32), 7.5))
    say("rel_fro", f"{r:.3e}")
    assert r <= GATE


def test_fp8_step_empty_slice():
    x_t = dev(np.random.default_rng(3).standard_normal((4, 64)).astype(np.float32))
    out, mx, lse, ent, am = api.soft_embed_step_fp8(
        x_t, 16, 16, dev(np.zeros((8, 16), np.uint8)), dev(np.ones(8, np.float32)), 1.0)
    mx2, lse2, ent2, am2 = api.row_stats(x_t)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    for a, b in ((mx, mx2), (lse, lse2), (ent, ent2), (am, am2)):
        assert torch.equal(a, b)


def test_fp8_step_rank_full_size():
    """The one-rank shape: the e4m3 step equals se_row_stats + se_soft_embed_fp8_fused bit for
    bit, and its argmax is the planted index."""
    w = wl.get("rank")
    bits, _ = wl.make_table(w)
    shard = np.ascontiguousarray(bits[w.vocab_start:w.vocab_end])
    del bits
    say("fp8 step rank: gpu quantize")
    c_t, s_t = gpu_quantize(shard)
    x = wl.make_logits(w)
    x_t = dev(x)
    say("fp8 step rank: gpu calls")
    out, mx, lse, ent, am = api.soft_embed_step_fp8(x_t, w.vocab_start, w.vocab_end, c_t, s_t,
                                                    w.gamma)
    mx2, lse2, ent2, am2 = api.row_stats(x_t)
    ref = torch.empty_like(out)
    B.se_soft_embed_fp8_fused(x_t, lse2, w.vocab_start, w.vocab_end, c_t, s_t, w.gamma, ref,
                              api.workspace(w.rows, w.vocab_start, w.vocab_end, w.d, DEV))
    torch.cuda.synchronize()
    for a, b in ((mx, mx2), (lse, lse2), (ent, ent2), (am, am2), (out, ref)):
        assert torch.equal(a, b)
    np.testing.assert_array_equal(am.cpu().numpy(), wl.planted_index(w))


# ---- se_soft_embed_step_onepass_fp8: the row scales carried by the staged probabilities --

def dev_logits(x):
    """x in a buffer whose row pitch is a multiple of 4, padded with huge values past V."""
    L, V = x.shape
    ld = ((V + 3) // 4) * 4
    buf = np.full((L, ld), np.float32(1e30), np.float32)
    buf[:, :V] = x
    return dev(buf)[:, :V]


ONEPASS_CASES = {
    # name: (L, V, s, e, d, seed)
    "tiny": (16, 4096, 0, 4096, 256, 31),
    "ragged": (17, 20008, 8, 20008, 48, 32),
    "slice-1": (5, 1000, 16, 17, 16, 33),
    "slice-63": (33, 1003, 64, 127, 2816, 34),        # V not a multiple of 4
    "slice-in-middle": (64, 50000, 12344, 37001, 128, 35),
    "two-row-tiles": (300, 2048, 1024, 2048, 512, 36),
    "whole-tile-tail": (256, 30003, 1000, 13337, 272, 37),
    "merge-in-contraction": (13, 20008, 8, 20008, 48, 38),
    "merge-row-tiles": (511, 100011, 8, 100008, 528, 39),
    "long-splits": (17, 150011, 8, 150003, 2816, 40),
    "long-splits-two-tiles": (300, 160011, 8, 160011, 2816, 41),
    "short-splits": (256, 3500, 8, 3011, 2816, 42),
    "d16": (256, 5000, 0, 4097, 16, 43),
}


def fp8_inputs(L, V, s, e, d, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    if e == s:                                    # an empty slice reads no table rows
        return x, np.zeros((8, d), np.uint8), np.ones(8, np.float32)
    bits = wl.fp32_to_bf16_bits((rng.standard_normal((e - s, d)) * 0.02).astype(np.float32))
    codes, scale = fp8.quantize_table(bits)
    return x, codes, scale


@pytest.mark.parametrize("case", sorted(ONEPASS_CASES))
def test_fp8_onepass_step_equals_bf16_onepass_on_the_dequantized_table(case):
    """se_soft_embed_step_onepass_fp8 on the oracle's codes (codes and scales past the slice:
    NaN, never read): statistics and embedding bit for bit se_soft_embed_step_onepass's on
    the oracle's dequantized table (a power-of-two scale moves exactly from the table row to
    the probability), and within the gate of the fp64 oracle on the dequantized table."""
    L, V, s, e, d, seed = ONEPASS_CASES[case]
    x, codes, scale = fp8_inputs(L, V, s, e, d, seed)
    dq = fp8.dequantize_bf16_bits(codes, scale)
    c_t = dev(np.concatenate([codes, np.full((24, d), 0x7F, np.uint8)]))
    s_t = dev(np.concatenate([scale, np.full(24, np.nan, np.float32)]))
    dq_t = dev(np.concatenate([dq, np.full((24, d), 0x7FC0, np.uint16)]))
    x_t = dev_logits(x)
    say("fp8 one-read step", case, (L, V, s, e, d))
    got = api.soft_embed_step_fp8(x_t, s, e, c_t, s_t, 7.5, onepass=True)
    ref = api.soft_embed_step(x_t, s, e, dq_t, 7.5, onepass=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "max", "lse", "entropy", "argmax"), got, ref):
        assert torch.equal(a, b), name
    r = rel_fro(got[0].cpu().numpy(),
                oracle.soft_embed(x, s, e, fp8.dequantize(codes, scale).astype(np.float32), 7.5))
    say("rel_fro", f"{r:.3e}")
    assert r <= GATE


def test_fp8_onepass_step_repeats():
    L, V, s, e, d = 64, 50000, 8, 40008, 256
    x, codes, scale = fp8_inputs(L, V, s, e, d, 44)
    c_t, s_t, x_t = dev(codes), dev(scale), dev_logits(x)
    say("fp8 one-read step: repeat")
    a = api.soft_embed_step_fp8(x_t, s, e, c_t, s_t, 2.0, onepass=True)
    b = api.soft_embed_step_fp8(x_t, s, e, c_t, s_t, 2.0, onepass=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("shape", [(8, 512, 16, 16, 16), (4096, 110000, 0, 110000, 1024)],
                         ids=["empty-slice", "long-split-ranges"])
def test_fp8_onepass_step_falls_back_to_the_two_pass_step(shape):
    """An empty slice, or split ranges longer than 24,576 positions (4096 rows x 4 n-tiles,
    4 splits of 27,520 positions): the call is se_soft_embed_step_fp8 in the same
    workspace, bit for bit."""
    L, V, s, e, d = shape
    x, codes, scale = fp8_inputs(L, V, s, e, d, 45)
    c_t, s_t, x_t = dev(codes), dev(scale), dev(x)
    ws = api.step_onepass_workspace(L, V, s, e, d, DEV)
    say("fp8 one-read step fallback", shape)
    a = api.soft_embed_step_fp8(x_t, s, e, c_t, s_t, 1.5, onepass=True, ws=ws)
    b = api.soft_embed_step_fp8(x_t, s, e, c_t, s_t, 1.5)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_fp8_onepass_step_rejects_an_unaligned_scale_array():
    L, V, s, e, d = 8, 4096, 0, 4096, 64
    x, codes, scale = fp8_inputs(L, V, s, e, d, 46)
    s_t = dev(np.concatenate([[0.0], scale]).astype(np.float32))[1:]     # 4 bytes past 16
    with pytest.raises(B.SoftEmbedError) as err:
        api.soft_embed_step_fp8(dev_logits(x), s, e, dev(codes), s_t, 1.0, onepass=True)
    assert err.value.status == B.SE_ERR_ALIGN


def test_fp8_onepass_step_rank_full_size():
    """The one-rank shape (L=256, slice [65536, 131072), d=2816) on the oracle's codes: bit
    for bit se_soft_embed_step_onepass on the oracle's dequantized shard, the planted argmax,
    and sampled rows against the fp64 oracle."""
    w = wl.get("rank")
    bits, _ = wl.make_table(w)
    shard = np.ascontiguousarray(bits[w.vocab_start:w.vocab_end])
    del bits
    say("fp8 one-read rank: oracle quantize")
    codes, scale = fp8.quantize_table(shard)
    del shard
    dq = fp8.dequantize_bf16_bits(codes, scale)
    x = wl.make_logits(w)
    x_t = dev(x)
    say("fp8 one-read rank: gpu calls")
    got = api.soft_embed_step_fp8(x_t, w.vocab_start, w.vocab_end, dev(codes), dev(scale),
                                  w.gamma, onepass=True)
    ref = api.soft_embed_step(x_t, w.vocab_start, w.vocab_end, dev(dq), w.gamma, onepass=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "max", "lse", "entropy", "argmax"), got, ref):
        assert torch.equal(a, b), name
    np.testing.assert_array_equal(got[4].cpu().numpy(), wl.planted_index(w))
    rows = np.array([0, 77, 255])
    say("fp8 one-read rank: oracle rows", list(rows))
    r = rel_fro(got[0].cpu().numpy()[rows],
                oracle.soft_embed(x[rows], w.vocab_start, w.vocab_end, dq, w.gamma))
    say("rel_fro", f"{r:.3e}")
    assert r <= GATE


@pytest.mark.parametrize("case", ["ragged", "two-whole-tiles", "whole-tile-held-slice",
                                  "slice-4097"])
def test_fp8_step_scale_alignment_forms_agree(case):
    """se_soft_embed_step_fp8 with a 16-byte aligned scale array (the statistics pass carries
    the scales, codes read in place) and with one 4 bytes past such an address (the codes
    turned into bf16 rows): the same outputs bit for bit."""
    L, V, s, e, d, seed = CASES[case]
    rng = np.random.default_rng(seed + 70)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    x[np.arange(L), rng.integers(0, V, L)] += 8.0
    bits = wl.fp32_to_bf16_bits((rng.standard_normal((e - s, d)) * 0.02).astype(np.float32))
    codes, scale = fp8.quantize_table(bits)
    c_t, x_t = dev(codes), dev(x)
    s_al = dev(scale)
    s_un = dev(np.concatenate([[np.float32(0)], scale]).astype(np.float32))[1:]
    assert s_al.data_ptr() % 16 == 0 and s_un.data_ptr() % 16 == 4
    say("fp8 step scale forms", case, (L, V, s, e, d))
    a = api.soft_embed_step_fp8(x_t, s, e, c_t, s_al, 7.5)
    b = api.soft_embed_step_fp8(x_t, s, e, c_t, s_un, 7.5)
    torch.cuda.synchronize()
    for name, u, v in zip(("out", "max", "lse", "entropy", "argmax"), a, b):
        assert torch.equal(u, v), name


def random_shapes(n, seed):
    """Seeded shapes within the calls' layout rules (vocab_start a multiple of 8, d a
    multiple of 16): rows 1..600 (one to three row tiles), vocabularies up to 60,000,
    slices from one position to the whole row, d 16..1024."""
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        L = int(r.integers(1, 601))
        V = int(r.integers(64, 60001))
        s = 8 * int(r.integers(0, V // 8))
        e = int(r.integers(s + 1, V + 1))
        d = 16 * int(r.integers(1, 65))
        out.append((L, V, s, e, d))
    return out


@pytest.mark.parametrize("shape", random_shapes(16, 2026), ids=lambda sh: "x".join(map(str, sh)))
def test_fp8_steps_on_random_shapes(shape):
    """On seeded random shapes: the one-read e4m3 step bit for bit the bf16 one-read step on
    the oracle's dequantized table; the two-pass e4m3 step with 16-byte aligned scales (codes
    read in place) bit for bit its form with unaligned scales (codes converted); both within
    the gate of the fp64 oracle."""
    L, V, s, e, d = shape
    seed = L * 7919 + V * 31 + s + e + d
    x, codes, scale = fp8_inputs(L, V, s, e, d, seed)
    dq = fp8.dequantize_bf16_bits(codes, scale)
    c_t, dq_t, x_t = dev(codes), dev(dq), dev_logits(x)
    s_al = dev(scale)
    s_un = dev(np.concatenate([[np.float32(0)], scale]).astype(np.float32))[1:]
    say("fp8 random shape", shape)
    one = api.soft_embed_step_fp8(x_t, s, e, c_t, s_al, 3.0, onepass=True)
    one_bf = api.soft_embed_step(x_t, s, e, dq_t, 3.0, onepass=True)
    two = api.soft_embed_step_fp8(x_t, s, e, c_t, s_al, 3.0)
    two_cv = api.soft_embed_step_fp8(x_t, s, e, c_t, s_un, 3.0)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "max", "lse", "entropy", "argmax"), one, one_bf):
        assert torch.equal(a, b), ("one-read", name)
    for name, a, b in zip(("out", "max", "lse", "entropy", "argmax"), two, two_cv):
        assert torch.equal(a, b), ("two-pass", name)
    ref = oracle.soft_embed(x, s, e, fp8.dequantize(codes, scale).astype(np.float32), 3.0)
    for o in (one[0], two[0]):
        r = rel_fro(o.cpu().numpy(), ref)
        assert r <= GATE, r
