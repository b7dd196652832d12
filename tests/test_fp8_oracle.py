"""Pins of the e4m3 table oracle (CPU only).

The format is OCP 8-bit floating point, E4M3 variant (the FP8 weights of the
agentlenshq overview of DiffusionGemma in vLLM, section on performance and
quantization).  Pins: hand-worked values from the format's definition (bias 7,
subnormals, largest finite 448, ties to even), an independent library routine
(torch's float8_e4m3fn casts on the CPU) over every code and over many values
including every exact tie, the power-of-two scale rule worked by hand and by brute
force, and invariants of the quantized table (error within half a unit in the last
place, exact bf16 dequantization, the row maximum lands in the top binade).
"""
import numpy as np
import pytest
import torch

from oracle import fp8
from oracle.fp8 import (decode_e4m3, dequantize, dequantize_bf16_bits, encode_e4m3,
                        quantize_table, row_exponent)


def test_hand_worked_codes():
    # sign | exponent (bias 7) | mantissa
    assert decode_e4m3(0x38) == 1.0                  # 0 0111 000
    assert decode_e4m3(0x7E) == 448.0                # 0 1111 110 = 1.75 * 2^8
    assert np.isnan(decode_e4m3(0x7F)) and np.isnan(decode_e4m3(0xFF))
    assert decode_e4m3(0x08) == 2.0 ** -6            # smallest normal
    assert decode_e4m3(0x01) == 2.0 ** -9            # smallest subnormal
    assert decode_e4m3(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert decode_e4m3(0xC0) == -2.0
    assert decode_e4m3(0x44) == 3.0                  # 1.5 * 2^1
    assert decode_e4m3(0x80) == 0.0 and np.signbit(decode_e4m3(0x80))


@pytest.mark.parametrize("x,code", [
    (1.0, 0x38), (448.0, 0x7E), (-2.0, 0xC0), (3.0, 0x44),
    (2.0 ** -9, 0x01),
    (2.0 ** -10, 0x00),            # half the smallest subnormal: tie, to the even code 0
    (0.75 * 2.0 ** -9, 0x01),      # nearer to 2^-9 than to 0
    (1.5 * 2.0 ** -9, 0x02),       # tie between codes 1 and 2: even
    (7.5 * 2.0 ** -9, 0x08),       # tie across the subnormal / normal boundary: even
    (1.0625, 0x38),                # tie between 1.0 (0x38) and 1.125 (0x39): even
    (1.1875, 0x3A),                # tie between 1.125 (0x39) and 1.25 (0x3A): even
    (432.0, 0x7E),                 # tie between 416 (0x7D) and 448 (0x7E): even
    (-0.0, 0x80), (-1e-6, 0x80), (0.0, 0x00),
])
def test_hand_worked_rounding(x, code):
    assert int(encode_e4m3(x)) == code


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_encode_matches_torch_including_every_tie():
    mags = fp8._MAGS
    mids = (mags[1:] + mags[:-1]) / 2              # every exact tie (fp32-representable)
    rng = np.random.default_rng(11)
    x = np.concatenate([mags, mids, -mags, -mids, rng.uniform(-448, 448, 50000),
                        rng.normal(0, 0.01, 50000), mids[:20] * 1e-3, -mids[:20] * 1e-3,
                        [0.0, -0.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3(x.astype(np.float64)), ref)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        encode_e4m3(449.0)
    with pytest.raises(ValueError):
        encode_e4m3(np.nan)


@pytest.mark.parametrize("a,k", [
    (448.0, 0), (450.0, 1), (224.0, -1), (225.0, 0), (0.02, -14), (1.0, -8), (3.5, -7),
    (3.0e38, 120), (1e-40, -126), (0.0, 0),
])
def test_scale_rule_worked(a, k):
    # 0.02: 448 * 2^-15 = 0.0137 < 0.02 <= 448 * 2^-14 = 0.0273
    assert row_exponent(a) == k


def test_scale_rule_brute_force():
    rng = np.random.default_rng(5)
    for a in np.concatenate([rng.lognormal(0, 8, 300), [2.0 ** j for j in range(-100, 100, 7)],
                             [448.0 * 2.0 ** j for j in range(-20, 20, 3)]]):
        ks = [k for k in range(-126, 140) if a <= 448.0 * 2.0 ** k]
        assert row_exponent(a) == ks[0]


def random_table(rows, d, seed, std=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, d)) * std).astype(np.float32)
    return (w.view(np.uint32) >> 16).astype(np.uint16)       # truncation is fine for a fixture


def test_quantized_table_invariants():
    bits = random_table(64, 96, 1)
    bits[3] = 0                                              # zero row
    bits[4] = 0x8000                                         # negative zeros
    bits[5, :] = 0; bits[5, 7] = 0x3F80                      # a single 1.0
    codes, scale = quantize_table(bits)
    w = fp8.bf16_bits_to_f64(bits)
    deq = dequantize(codes, scale)
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    assert np.all(codes[4] == 0x80)
    assert scale[5] == 2.0 ** -8 and codes[5, 7] == 0x78     # 256 = 1.0 * 2^8: 0 1111 000
    for r in range(64):
        s = float(scale[r])
        assert s == 2.0 ** round(np.log2(s))                 # a power of two
        if np.any(w[r] != 0):
            # the row maximum lands in the top binade: 224 < max / s <= 448
            assert 224.0 < np.max(np.abs(w[r])) / s <= 448.0
        # each value within half a unit in the last place of its e4m3 neighbourhood
        q = w[r] / s
        e = np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6)))
        half_ulp = 2.0 ** (e - 3) / 2
        assert np.all(np.abs(deq[r] / s - q) <= half_ulp)
    assert not np.any((codes & 0x7F) == 0x7F)                # never NaN
    # dequantized values are exact bf16 values
    dq_bits = dequantize_bf16_bits(codes, scale)
    assert np.array_equal(fp8.bf16_bits_to_f64(dq_bits), deq)


def test_quantization_commutes_with_power_of_two_row_scaling():
    bits = random_table(8, 64, 2)
    w = fp8.bf16_bits_to_f64(bits)
    w2 = (w * 2.0 ** 5).astype(np.float32)
    bits2 = (w2.view(np.uint32) >> 16).astype(np.uint16)
    c1, s1 = quantize_table(bits)
    c2, s2 = quantize_table(bits2)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2, s1 * np.float32(32.0))


def test_moving_a_row_scale_onto_the_probability_is_exact():
    """The reading behind the one-read e4m3 step: for a power of two 2^k (the row scales,
    k in [-126, 0] here) and a probability p in (0, 1], bf16(p 2^k) = bf16(p) 2^k whenever
    p 2^k stays in bf16's normal range, so each product p 2^k code equals bf16(p) times the
    dequantized entry code 2^k exactly.  Checked with torch's CPU bfloat16 cast (round to
    nearest even) on random and boundary probabilities."""
    rng = np.random.default_rng(5)
    p = np.concatenate([rng.random(20000), np.exp(-rng.random(20000) * 80.0),
                        [1.0, 0.5, 2.0 ** -20, 1 - 2.0 ** -24, 1.00390625 / 2]]).astype(np.float32)
    for k in (-126, -100, -40, -14, -12, -7, -1, 0):
        s = np.float32(2.0 ** k)
        scaled = torch.from_numpy(p * s).to(torch.bfloat16).to(torch.float64).numpy()
        moved = torch.from_numpy(p).to(torch.bfloat16).to(torch.float64).numpy() * float(s)
        normal = p.astype(np.float64) * float(s) >= 2.0 ** -126
        assert normal.sum() > 0
        np.testing.assert_array_equal(scaled[normal], moved[normal])
        # and the code products agree exactly in fp64 (bf16 x e4m3 values are exact there)
        code_vals = decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))
        c = code_vals[rng.integers(0, len(code_vals), normal.sum())]
        np.testing.assert_array_equal(scaled[normal] * c, moved[normal] * c)
