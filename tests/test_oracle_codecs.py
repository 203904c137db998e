"""Pins of the input encodings and of the oracle's decoders (CPU only).

The oracle's e4m3 table is checked against the OCP OFP8 specification's printed
code points (tests/golden/e4m3_spec_points.txt) and against torch's
float8_e4m3fn, an independent implementation of the same format.  The
generator's encoders (bf16 round-to-nearest-even, e4m3 round-to-nearest-even
with saturation, per-row amax/448 scaling) are checked against torch casts.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import E4M3_TABLE, bf16_to_f64, e4m3_to_f64
from workloads import bf16_bits, e4m3_encode, quantize_rows_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spec_points.txt")


def _spec_points():
    pts = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                pts.append((int(c, 16), float(v)))
    return pts


def test_e4m3_table_spec_points():
    pts = _spec_points()
    assert len(pts) >= 10
    for code, val in pts:
        got = E4M3_TABLE[code]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3_table_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(E4M3_TABLE) == nan).all()
    assert (E4M3_TABLE[~nan] == ref[~nan]).all()
    # the grid is monotone over the positive codes and symmetric in sign
    pos = E4M3_TABLE[:0x7F]
    assert (np.diff(pos) > 0).all()
    assert (E4M3_TABLE[0x80:0xFF] == -pos).all()


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, size=100_000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()


def test_bf16_encode_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact ties: fp32 values whose low 16 bits are 0x8000
    ties = (rng.integers(0, 2 ** 15, size=4096).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]      # NaN payloads are not rounding cases
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, 65504.0, 3.4e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bf16_bits(x) == ref).all()


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1_000_000).astype(np.float32) * np.float32(60.0)
    x = x[np.abs(x) < 464.0]
    # every midpoint between neighbouring codes, and the codes themselves
    pos = E4M3_TABLE[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, pos.astype(np.float32), -pos.astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3_encode(x)
    # +-0 may differ only in sign bit for -0.0 inputs; compare decoded values where both zero
    same = (got == ref) | ((E4M3_TABLE[got] == 0) & (E4M3_TABLE[ref] == 0))
    assert same.all()


def test_e4m3_encode_saturates():
    got = e4m3_encode(np.array([448.0, 470.0, 1e6, -1e6, np.nan], np.float32))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7F]


def test_quantize_rows_amax_maps_to_448():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 8, 128)).astype(np.float32)
    codes, scale = quantize_rows_e4m3(x)
    assert scale.dtype == np.float32 and scale.shape == (64, 8)
    amax = np.abs(x).max(-1)
    assert (scale == (amax / np.float32(448.0)).astype(np.float32)).all()
    deq = e4m3_to_f64(codes) * scale[..., None].astype(np.float64)
    # the amax element of every row is encoded as +-448 exactly
    idx = np.abs(x).argmax(-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0]
    assert ((top & 0x7F) == 0x7E).all()
    # relative error of e4m3 RNE is at most 2^-4 for normals, absolute 2^-10 * scale below
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[..., None])
    assert (err <= bound + 1e-12).all()
    # all-zero row
    c0, s0 = quantize_rows_e4m3(np.zeros((1, 16), np.float32))
    assert s0[0] == 1.0 and (c0 == 0).all()
