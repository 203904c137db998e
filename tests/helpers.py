"""Shared helpers of the GPU tests: moving generator output to the device, decoding it for
the oracle, and the parity bars.

Parity bars (max-abs error, relative L2 error over the compared tensor):
  bf16 paths: 1e-2 and 5e-3; e4m3 paths (MLA prefill nope or V, e4m3 decode caches): 3e-2 and
  1e-2 (against the oracle on the dequantised inputs).  fp32 path: 1e-4 and 1e-5, derived from the arithmetic: fp32 products
  and sums over <= 4096 terms of O(1) values, exp2 to about 1 ulp, give errors of order 1e-6.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

BF16_TOL = (1e-2, 5e-3)
FP8_TOL = (3e-2, 1e-2)
# Decode over e4m3 caches is an fp8 path: it is held to the fp8 bar against the oracle on the
# dequantised cache.  The bf16 bar cannot hold there: a row with one visible key returns
# bf16(v_scale) * code rounded to bf16 (P carries the value scale), two roundings of up to
# 2^-9 relative each, i.e. up to 2^-8 |V|, past 1e-2 once |V| exceeds ~2.5.
E4M3_CACHE_TOL = FP8_TOL
F32_TOL = (1e-4, 1e-5)
# LSE (no bar is stated for it; derived from the arithmetic): the kernels sum the row's P after
# rounding each value to bf16 (the P that multiplies V), so the row sum l carries a relative
# error up to the bf16 unit roundoff 2^-8 when one key dominates, i.e. |d ln l| <= ln(1 + 2^-8)
# = 3.9e-3, plus fp32 rounding of the scaled logits (< 5e-4 for |logit| < 10^3).
LSE_TOL = 4.5e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_bf16_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return host_bf16_f64(t)
    return t.detach().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, tol, what: str):
    ma, rl = errors(got, ref)
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{what}: non-finite output"
    say(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e} (bars {tol[0]:.0e}, {tol[1]:.0e})")
    assert ma <= tol[0] and rl <= tol[1], f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e} exceed {tol}"


def assert_lse_close(got, ref, what: str, tol: float = LSE_TOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf_r = np.isneginf(ref)
    assert (np.isneginf(got) == inf_r).all(), f"{what}: -inf pattern differs"
    if (~inf_r).any():
        err = float(np.abs(got[~inf_r] - ref[~inf_r]).max())
        say(f"  {what}: lse max_abs={err:.3e}")
        assert err <= tol, f"{what}: lse error {err}"
