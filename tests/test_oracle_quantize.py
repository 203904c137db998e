"""Pins of the oracle's per-token e4m3 quantiser (CPU only).

The encoder is checked against torch's float8_e4m3fn casts (an independent
implementation of the OCP E4M3 format), against every code point and every midpoint
between neighbouring codes of the format definition, and against an exact-rational
brute force that scans all codes.  The row quantiser is checked for the properties its
definition fixes (the row maximum lands on +-448, zero rows, the error bound) and
against the input generator's own, separately written, quantiser.  Planted mistakes in
the oracle must fail these pins.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.quantize as oq
from oracle import E4M3_TABLE
from workloads import quantize_rows_e4m3


def _torch_codes(q):
    return torch.from_numpy(np.asarray(q, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_matches_torch():
    rng = np.random.default_rng(7)
    parts = [rng.standard_normal(100_000) * s for s in (1.0, 30.0, 2.0 ** -7, 2.0 ** -10)]
    q = np.clip(np.concatenate(parts), -448, 448).astype(np.float32)
    q = np.concatenate([q, np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, -(2.0 ** -9), 2.0 ** -10])])
    assert (oq.e4m3_round(q) == _torch_codes(q)).all()


def test_code_points_and_midpoints():
    pos = E4M3_TABLE[:0x7F]                       # codes 0x00..0x7E, ascending, finite
    codes = np.arange(0x7F, dtype=np.uint8)
    assert (oq.e4m3_round(pos) == codes).all()
    assert (oq.e4m3_round(-pos[1:]) == (codes[1:] | 0x80)).all()
    mid = (pos[:-1] + pos[1:]) / 2                # exact in fp64; ties go to the even code
    even = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert (oq.e4m3_round(mid) == even).all()
    # just above / below a midpoint goes to the nearer code
    assert (oq.e4m3_round(np.nextafter(mid, np.inf)) == codes[1:]).all()
    assert (oq.e4m3_round(np.nextafter(mid, -np.inf)) == codes[:-1]).all()


def _brute(v: float) -> int:
    """Nearest e4m3 code by exact rational comparison against every finite code of the
    value's sign (ties: the even code)."""
    x = Fraction(v)
    sign = 0x80 if np.signbit(v) else 0x00
    best = None
    for c in range(0x7F):  # magnitudes of codes 0x00..0x7E
        e, m = c >> 3, c & 7
        val = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        key = (abs(val - abs(x)), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1] | sign


def test_encoder_brute_force():
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.uniform(-448, 448, 300), rng.uniform(-0.02, 0.02, 300), [0.0, -0.0, 448.0, 447.9]])
    vals = vals.astype(np.float32)
    got = oq.e4m3_round(vals)
    for v, g in zip(vals, got):
        assert g == _brute(float(v)), (float(v), hex(g))


def test_saturation():
    assert (oq.e4m3_round(np.float32([460.0, 464.0, 1e6, -1e6])) == np.uint8([0x7E, 0x7E, 0x7E, 0xFE])).all()


def test_rows_scale_and_max():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)).astype(np.float32) * np.float32(rng.uniform(1e-3, 1e3, (64, 1)))
    codes, scale = oq.quantize_rows(x)
    amax = np.abs(x).max(axis=1)
    assert scale.dtype == np.float32 and (scale == (amax / np.float32(448)).astype(np.float32)).all()
    imax = np.abs(x).argmax(axis=1)
    top = codes[np.arange(64), imax]
    assert ((top & 0x7F) == 0x7E).all()
    assert (((top & 0x80) != 0) == (x[np.arange(64), imax] < 0)).all()
    # every code is the nearest one to x/scale: error at most half the local code spacing
    q = (x / scale[:, None]).astype(np.float64)
    deq = E4M3_TABLE[codes]
    a = np.abs(q)
    e = np.maximum(np.floor(np.log2(np.maximum(a, 2.0 ** -6))), -6)
    assert (np.abs(deq - q) <= np.ldexp(1.0, (e - 3).astype(int)) / 2 + 1e-12).all()


def test_zero_row():
    codes, scale = oq.quantize_rows(np.zeros((2, 16), np.float32))
    assert (scale == 1.0).all() and (codes == 0).all()


def test_matches_generator_quantiser():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((256, 128)).astype(np.float32)
    c1, s1 = oq.quantize_rows(x)
    c2, s2 = quantize_rows_e4m3(x)
    assert (s1 == s2).all() and (c1 == c2).all()


def _all_pins():
    out = []
    for fn in (test_encoder_matches_torch, test_code_points_and_midpoints, test_encoder_brute_force,
               test_saturation, test_rows_scale_and_max, test_zero_row):
        try:
            fn()
            out.append(False)
        except (AssertionError, ValueError):
            out.append(True)
    return out


def _round_toward_zero(q):
    q = np.asarray(q, np.float64)
    a = np.minimum(np.abs(q), 448.0)
    grid = E4M3_TABLE[:0x7F]
    idx = np.searchsorted(grid, a, side="right") - 1
    return (idx | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)


def _ties_away(q):
    q = np.asarray(q, np.float64)
    out = oq.__dict__["_orig_round"](q)
    grid = E4M3_TABLE[:0x7F]
    a = np.minimum(np.abs(q), 448.0)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    tie = (grid[hi] - a) == (a - grid[lo])
    return np.where(tie & (hi != lo), (hi | np.where(np.signbit(q), 0x80, 0)), out).astype(np.uint8)


MUTANTS = {
    "scale_fnuz_240": ("row_scale", lambda amax: np.where(np.asarray(amax) > 0, (np.asarray(amax, np.float32) / np.float32(240)).astype(np.float32), np.float32(1)).astype(np.float32)),
    "scale_inverted": ("row_scale", lambda amax: np.where(np.asarray(amax) > 0, (np.float32(448) / np.maximum(np.asarray(amax, np.float32), np.float32(1e-30))).astype(np.float32), np.float32(1)).astype(np.float32)),
    "round_toward_zero": ("e4m3_round", _round_toward_zero),
    "ties_away_from_zero": ("e4m3_round", _ties_away),
    "no_sign": ("e4m3_round", lambda q: (oq.__dict__["_orig_round"](np.abs(np.asarray(q, np.float64))))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_quantiser_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(oq.__dict__, "_orig_round", oq.e4m3_round)
    monkeypatch.setattr(oq, attr, fn)
    assert any(_all_pins()), name
