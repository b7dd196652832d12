"""Oracle of the e4m3 (OCP FP8) embedding table -- TEST INFRASTRUCTURE (only tests/,
the smoke check and the benchmark's CPU leg use it).

The pages serve the model with FP8 weights (agentlenshq overview of DiffusionGemma
in vLLM, section on performance and quantization: the quantized checkpoints hold
FP8 weights with fully dynamic activations) and give no scaling scheme.  Reading
taken here (the library's header states the same):
  * element format: OCP 8-bit floating point, E4M3 variant -- sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
    (m / 8) 2^-6; S.1111.111 is NaN; no infinities; largest finite value 448;
  * one power-of-two scale per vocabulary row: 2^k with k the smallest integer
    (at least -126) such that the row's largest magnitude is <= 448 2^k, k = 0
    for an all-zero row;
  * code = the e4m3 value nearest to w 2^-k, ties to the even code (mantissa LSB
    0), a zero result keeps the sign of w;
  * the dequantized table is code value times 2^k, exact in fp64 (and in bf16).
The soft embedding over an e4m3 table is the ordinary soft embedding over the
dequantized table (oracle.soft_embed).  Plain numpy: a decode table of the 127
non-negative finite values and a sorted search for the nearest one.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
K_MIN = -126


def decode_e4m3(codes) -> np.ndarray:
    """Values (fp64) of e4m3 codes; NaN for S.1111.111."""
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


_MAGS = decode_e4m3(np.arange(127))          # codes 0x00 .. 0x7E, increasing values


def encode_e4m3(x) -> np.ndarray:
    """Nearest e4m3 code of each value (|x| <= 448), ties to the even code."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("values must be finite and within +-448")
    a = np.abs(x)
    hi = np.minimum(np.searchsorted(_MAGS, a, side="left"), 126)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def row_exponent(absmax: float) -> int:
    """Smallest integer k >= -126 with absmax <= 448 * 2^k (0 for a zero row)."""
    a = float(absmax)
    if a == 0.0:
        return 0
    k = math.ceil(math.log2(a / E4M3_MAX))
    while a > E4M3_MAX * 2.0 ** k:
        k += 1
    while a <= E4M3_MAX * 2.0 ** (k - 1):
        k -= 1
    return max(k, K_MIN)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def quantize_table(w_bits: np.ndarray, chunk: int = 2048):
    """(codes uint8 [rows, d], scale float32 [rows]) of a bf16 table given as bits.
    Rows are processed in blocks only to bound memory; each row is independent."""
    w_bits = np.asarray(w_bits)
    if w_bits.ndim != 2:
        raise ValueError("table must be 2-D")
    rows = w_bits.shape[0]
    codes = np.empty(w_bits.shape, dtype=np.uint8)
    scale = np.empty(rows, dtype=np.float32)
    for r0 in range(0, rows, chunk):
        w = bf16_bits_to_f64(w_bits[r0:r0 + chunk])
        absmax = np.max(np.abs(w), axis=1) if w.shape[1] else np.zeros(w.shape[0])
        k = np.array([row_exponent(a) for a in absmax], dtype=np.float64)
        scale[r0:r0 + chunk] = (2.0 ** k).astype(np.float32)
        codes[r0:r0 + chunk] = encode_e4m3(w * (2.0 ** -k)[:, None])
    return codes, scale


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp64 table: code value times the row's scale."""
    return decode_e4m3(codes) * np.asarray(scale, dtype=np.float64)[:, None]


def dequantize_bf16_bits(codes: np.ndarray, scale: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """The dequantized table as bf16 bit patterns (every value is exactly a bf16)."""
    out = np.empty(codes.shape, dtype=np.uint16)
    for r0 in range(0, codes.shape[0], chunk):
        f = dequantize(codes[r0:r0 + chunk], scale[r0:r0 + chunk]).astype(np.float32)
        u = f.view(np.uint32)
        if np.any(u & 0xFFFF):
            raise ValueError("dequantized value not representable in bf16")
        out[r0:r0 + chunk] = (u >> 16).astype(np.uint16)
    return out
