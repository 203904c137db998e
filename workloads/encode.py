"""Storage encodings of the attention inputs.

bfloat16: the upper 16 bits of an IEEE binary32 value, rounded to nearest with
ties to even.

e4m3 ("fp8 e4m3fn" of the OCP 8-bit floating point specification): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
subnormals m * 2^-9; the all-ones exponent field is a normal binade except for
mantissa 111, which is NaN; there is no infinity; the largest finite magnitude
is 1.75 * 2^8 = 448.  The encoder below rounds to nearest, ties to the even
code, and saturates magnitudes above 448 to 448.

The per-token scale of the MLA prefill workload is one fp32 value per
(token, head) row: scale = amax(|row|) / 448, computed in fp32 from the fp32
originals, and the codes are e4m3(row / scale).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- bfloat16

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bfloat16 bit patterns (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)  # keep a quiet NaN
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> fp32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- e4m3

def _e4m3_positive_grid() -> np.ndarray:
    """Values of codes 0x00..0x7E (every non-negative finite e4m3 value), ascending."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


_E4M3_GRID = _e4m3_positive_grid()
E4M3_MAX = 448.0


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Real values -> e4m3fn codes: round to nearest, ties to even code, saturate at 448."""
    a64 = np.abs(np.asarray(x, dtype=np.float64))
    neg = np.signbit(np.asarray(x, dtype=np.float64))
    nan = np.isnan(a64)
    a = np.where(nan, 0.0, np.minimum(a64, E4M3_MAX))
    hi = np.searchsorted(_E4M3_GRID, a, side="left")          # grid[hi] >= a
    hi = np.clip(hi, 0, len(_E4M3_GRID) - 1)
    lo = np.clip(hi - 1, 0, len(_E4M3_GRID) - 1)
    d_hi = _E4M3_GRID[hi] - a
    d_lo = a - _E4M3_GRID[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    return code


def quantize_rows_e4m3(x32: np.ndarray):
    """Per-row e4m3 quantisation along the last axis.

    Returns (codes uint8 of x's shape, scale fp32 of x.shape[:-1]) with
    scale = amax/448 in fp32 (1.0 for an all-zero row) and codes = e4m3(x/scale),
    the division done in fp32.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    scaled = (x32 / scale[..., None]).astype(np.float32)
    return e4m3_encode(scaled), scale
