"""Decoding of the stored input bits into exact fp64 values (oracle side).

bfloat16 bits b decode to the binary32 value whose upper half is b and whose
lower half is zero.  e4m3 codes decode through a 256-entry table built from the
OCP 8-bit floating point definition of E4M3: value = (-1)^s * 2^(e-7) * (1 + m/8)
for exponent field e in 1..15, (-1)^s * 2^-6 * (m/8) for e = 0, and NaN for the
codes S.1111.111 (there is no infinity).  The MLA prefill page
("MLASmemStorage") gives the Q, K_nope and V shared-memory buffers a qkv dtype
of their own and the rope buffers another; the fp8 nope operands use this
format.
"""
import math

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _build_e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = math.nan
        elif e == 0:
            t[code] = s * math.ldexp(m / 8.0, -6)
        else:
            t[code] = s * math.ldexp(1.0 + m / 8.0, e - 7)
    return t


E4M3_TABLE = _build_e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
