"""Per-token e4m3 quantisation, oracle side.  TEST INFRASTRUCTURE ONLY (see the package
header): only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline use it.

What it computes.  The per-token-scale MLA prefill of the "MLASmemStorage" page (sm100
MLA prefill with per-token scales: `q_scale_smem` holds one fp32 scale per Q-tile row,
`k_scale_smem` one per K-tile row) consumes e4m3 nope operands with one fp32 scale per
(token, head) row.  The step that produces them, for every row x of fp32 values:

    amax  = max_j |x_j|                           (exact)
    scale = fl32(amax / 448)                       (fp32 division; 1.0 when amax == 0)
    q_j   = fl32(x_j / scale)                      (fp32 division)
    code_j = e4m3fn(q_j)                           (nearest code, ties to even, saturating at 448)

448 is the largest finite e4m3fn magnitude (OCP 8-bit floating point, E4M3: exponent bias
7, 3 mantissa bits, subnormals m * 2^-9, no infinity, S.1111.111 = NaN).  Rows must be
finite.  The encoder below works on the exact value of q (an fp32 number is exact in fp64):
it splits |q| into a binade and rounds the scaled mantissa with round-half-even, instead of
searching a table.

parity pins: tests/test_oracle_quantize.py (torch float8_e4m3fn casts, every code point
and every midpoint between neighbouring codes, an exact-rational brute force, the scale
and saturation properties, planted mistakes).
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_round(q: np.ndarray) -> np.ndarray:
    """Finite real values -> e4m3fn codes (uint8), round to nearest even, saturate at 448."""
    q = np.asarray(q, dtype=np.float64)
    if not np.isfinite(q).all():
        raise ValueError("e4m3_round: non-finite input")
    a = np.minimum(np.abs(q), E4M3_MAX)
    sign = np.where(np.signbit(q), 0x80, 0x00).astype(np.int64)
    # binade exponent e with 2^e <= a < 2^(e+1); values below 2^-6 use the subnormal step 2^-9
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    # guard log2 rounding at binade edges: enforce 2^e <= a < 2^(e+1)
    e = np.where(np.ldexp(1.0, e) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= a, e + 1, e)
    normal = a >= 2.0 ** -6
    # normal: a = 2^e * (1 + k/8), k = rne(8 * (a / 2^e - 1)); carry into the next binade
    k_n = np.rint(8.0 * (np.ldexp(a, -e) - 1.0)).astype(np.int64)
    e_n = e + (k_n == 8)
    k_n = np.where(k_n == 8, 0, k_n)
    code_n = ((e_n + 7) << 3) | k_n
    # subnormal: a = k * 2^-9, k = rne(a * 2^9) in 0..8 (k = 8 is the smallest normal, code 0x08)
    k_s = np.rint(np.ldexp(a, 9)).astype(np.int64)
    code = np.where(normal, code_n, k_s)
    code = np.minimum(code, 0x7E)  # 448 is code 0x7E; the rounding above never passes it after the clamp
    return (code | sign).astype(np.uint8)


def row_scale(amax: np.ndarray) -> np.ndarray:
    """fp32 scale of rows with fp32 absolute maximum amax: fl32(amax / 448), 1.0 for a zero row."""
    amax = np.asarray(amax, dtype=np.float32)
    return np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0)).astype(np.float32)


def quantize_rows(x32: np.ndarray):
    """Quantise every row (last axis) of fp32 x: returns (codes uint8 like x, scale fp32 x.shape[:-1])."""
    import oracle.quantize as me  # look the readings up at call time (the mutation tests replace them)
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = me.row_scale(amax)
    q = (x32 / scale[..., None]).astype(np.float32)
    return me.e4m3_round(q), scale
