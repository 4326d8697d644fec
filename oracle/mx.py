"""OCP microscaling (MX) formats used by the 4-bit expert weights: MXFP4 weights
(E2M1 elements) and MXFP8 activations (E4M3 elements), each block of 32
consecutive contraction elements sharing one E8M0 scale.  Written from the OCP
Microscaling Formats (MX) v1.0 specification.

TEST INFRASTRUCTURE ONLY: this file belongs to the CPU oracle.  Only tests/,
the smoke check and the benchmark's CPU-baseline leg may import it.

Why this format: the 4-bit group-scaled weights the pages point to for the
decode-bound layers (NVFP4 and FP8 x FP4 in [DeepGEMM fork PR #5] and
[DeepGEMM PR #381], the W4A8 / int4 group-128 notes in [colibri
issue_budget.md]) are realised here in the block-scaled FP4 format that the
MI355X matrix cores multiply natively.

Formats:
  * E8M0 scale code e (8 bits, no sign, no mantissa): 2^(e - 127); 255 is NaN.
  * E2M1 element (4 bits): sign, 2 exponent bits with bias 1, 1 mantissa bit;
    exponent field 0 is subnormal (m * 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2, 3,
    4, 6; no infinities or NaN.
  * E4M3 elements: see oracle.e4m3.
  * Storage: MXFP4 codes two per byte along the contraction, element 2i in the
    low nibble; scales one byte per 32 elements, [rows, K/32].

Reading taken where the pages are silent (listed in the design notes): the
activations entering a contraction against MXFP4 weights are quantised per row
and 32-element block to MXFP8 with the MX scale rule, shared exponent =
floor(log2(amax)) - 8 (8 = the E4M3 exponent of its largest normal), elements
rounded to nearest even and clamped to +-448; a block of zeros gets scale code
127 (2^0).  The element code is decided in float32, as the kernel decides it.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

BLOCK = 32
E2M1_MAX = 6.0
E4M3_EMAX = 8          # exponent of the largest normal E4M3 value (448 = 1.75 * 2^8)


# ----------------------------------------------------------------------------- codecs

def e8m0_decode(codes) -> np.ndarray:
    """uint8 scale codes -> 2^(e - 127) as float64 (NaN for 255)."""
    e = np.asarray(codes, dtype=np.int64)
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))


def _e2m1_bits(c: np.ndarray) -> np.ndarray:
    sign = np.where(c & 0x8, -1.0, 1.0)
    exp = (c >> 1) & 0x3
    man = c & 0x1
    sub = man * 0.5
    nrm = (1.0 + man * 0.5) * np.exp2(exp.astype(np.float64) - 1.0)
    return sign * np.where(exp == 0, sub, nrm)


_E2M1 = _e2m1_bits(np.arange(16, dtype=np.int64))


def e2m1_decode(codes) -> np.ndarray:
    """4-bit codes (0..15) -> float64 values."""
    return _E2M1[np.asarray(codes, dtype=np.int64) & 0xF]


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes (element 2i from the low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 weights [rows, K/2] bytes with E8M0 scales [rows, K/32] -> float64 [rows, K]."""
    vals = e2m1_decode(unpack_fp4(packed))
    s = e8m0_decode(scales)
    return vals * np.repeat(s, BLOCK, axis=-1)


# ----------------------------------------------------------------------------- activation quantiser

def quantise_mxfp8(v) -> tuple:
    """Rows of float32 activations [rows, K] -> (e4m3 codes uint8 [rows, K], E8M0
    scale codes uint8 [rows, K/32]).

    Per 32-element block: amax = max |v|; shared exponent s = floor(log2(amax)) - 8
    (clamped to [-127, 127]); scale code s + 127; element = round-to-nearest-even
    e4m3 of v / 2^s, clamped to +-448.  amax = 0 gives s = 0 and zero codes.  v / 2^s
    is exact in float32 (a power-of-two division of float32 values far from the
    subnormal range of float32), so the element code depends only on float32 data.
    """
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    if K % BLOCK:
        raise ValueError("the contraction must be a multiple of 32")
    blocks = v.reshape(rows, K // BLOCK, BLOCK).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    # floor(log2(amax)) exactly: frexp gives amax = m * 2^e with m in [0.5, 1).
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    s = np.where(amax > 0, e.astype(np.int64) - 1 - E4M3_EMAX, 0)
    s = np.clip(s, -127, 127)
    scaled = blocks * np.exp2(-s.astype(np.float64))[..., None]
    scaled = np.clip(scaled, -e4m3.E4M3_MAX, e4m3.E4M3_MAX)
    codes = e4m3.encode_rne(scaled.reshape(rows, K))
    return codes.astype(np.uint8), (s + 127).astype(np.uint8)


def dequant_mxfp8(codes, scales) -> np.ndarray:
    """(e4m3 codes [rows, K], E8M0 scales [rows, K/32]) -> float64 [rows, K]."""
    return e4m3.decode(codes) * np.repeat(e8m0_decode(scales), BLOCK, axis=-1)
