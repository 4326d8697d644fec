"""OCP 8-bit floating point, E4M3 ("e4m3fn") codec, written from the OCP FP8 spec.

TEST INFRASTRUCTURE ONLY: this file belongs to the CPU oracle.  Only tests/,
the smoke check and the benchmark's CPU-baseline leg may import it.

Format (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits.  Exponent field 0 is subnormal
(value = m * 2^-9).  There are no infinities; S.1111.111 is NaN, so the
largest finite magnitude is 2^8 * 1.75 = 448.

The fp8 weights and the group-128 fp32 scales follow the "FP8 e4m3" test weights
and group-128 scaling of [colibri issue_budget.md, header notes on
issue_grouped_quant.md and glm_fp8_emit.py].
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
GROUP = 128


def _decode_bits(c: np.ndarray) -> np.ndarray:
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man.astype(np.float64) * 2.0 ** -9
    nrm = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    val = sign * np.where(exp == 0, sub, nrm)
    return np.where((exp == 15) & (man == 7), np.nan, val)


# The 256 code points decoded once from the bit fields above.
_TABLE = _decode_bits(np.arange(256, dtype=np.int64))


def decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for S.1111.111)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def _round_half_even(a: np.ndarray) -> np.ndarray:
    f = np.floor(a)
    d = a - f
    up = (d > 0.5) | ((d == 0.5) & (np.mod(f, 2.0) == 1.0))
    return f + up


def encode_rne(v) -> np.ndarray:
    """Finite values with |v| <= 448 -> nearest e4m3 code, ties to even mantissa.

    The caller clamps to +-448 first (the quantiser does).  Every step below is
    exact in float64: the inputs are float32 values and all divisions are by
    powers of two.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("encode_rne expects finite values within +-448")
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0x00)
    code = np.zeros(v.shape, dtype=np.int64)
    # Subnormal range (a < 2^-6): step 2^-9, mantissa m in 0..8 (m = 8 is the smallest normal).
    small = a < 2.0 ** -6
    code = np.where(small, _round_half_even(a / 2.0 ** -9).astype(np.int64), code)
    # Normal range: a in [2^e, 2^(e+1)), step 2^(e-3).
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(small, 1.0, a)))
    # log2 of an exact power of two is exact; guard the floor against representation edges.
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    m = _round_half_even(a / np.exp2(e - 3))          # 8..16
    carry = m >= 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    nrm = ((e + 7).astype(np.int64) << 3) | (m.astype(np.int64) - 8)
    code = np.where(small, code, nrm)
    return (code | sign).astype(np.uint8)


def quantise_group128(v: np.ndarray):
    """Dynamic per-row, per-128-group e4m3 quantisation, decided in float32.

    For each row and each group of 128 consecutive elements along the last axis:
      amax = max |v|;  s = fp32(amax / 448)  (s = 1 when amax = 0);
      q = RNE_e4m3(clamp(fp32(v / s), -448, 448)).
    Returns (codes uint8 [..., C], scales float32 [..., C/128]); v ~= decode(q) * s.
    """
    v32 = np.asarray(v, dtype=np.float32)
    *lead, C = v32.shape
    if C % GROUP:
        raise ValueError("last dimension must be a multiple of 128")
    g = v32.reshape(*lead, C // GROUP, GROUP)
    amax = np.abs(g).max(axis=-1)
    s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0))
    r = (g / s[..., None]).astype(np.float32)
    r = np.clip(r, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    q = encode_rne(r).reshape(*lead, C)
    return q, s.astype(np.float32)


def dequantise_group128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """codes [..., C] and scales [..., C/128] -> float64 values decode(q) * s."""
    *lead, C = q.shape
    d = decode(q).reshape(*lead, C // GROUP, GROUP)
    return (d * np.asarray(s, dtype=np.float64)[..., None]).reshape(*lead, C)
