"""GPU parity of mla_prefill_fwd (e4m3 nope with per-token scales + bf16 rope) against the oracle
run on the dequantised inputs."""
import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as fa
import oracle
from tests.helpers import (BF16_TOL, FP8_TOL, assert_close, assert_lse_close, dev, dev_bf16, host_f64, say)
from workloads import make_mla_prefill, workload

pytestmark = pytest.mark.gpu

MLA = "mla_prefill_fp8_causal_b1_h128_s8192"


def _inputs(w):
    d = make_mla_prefill(w)
    t = {k: (dev_bf16(d[k]) if d[k].dtype == np.uint16 else dev(d[k])) for k in
         ("q_nope", "k_nope", "q_scale", "k_scale", "q_rope", "k_rope", "v")}
    return d, t


def _oracle_inputs(d):
    return dict(q_nope=oracle.e4m3_to_f64(d["q_nope"]), k_nope=oracle.e4m3_to_f64(d["k_nope"]),
                q_rope=oracle.bf16_to_f64(d["q_rope"]), k_rope=oracle.bf16_to_f64(d["k_rope"]),
                v=oracle.bf16_to_f64(d["v"]), q_scale=d["q_scale"].astype(np.float64),
                k_scale=d["k_scale"].astype(np.float64))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,H,Hr", [(200, 4, 1), (333, 2, 2), (64, 3, 1)])
def test_mla_prefill_fp8_small(causal, S, H, Hr):
    w = workload(MLA, Sq=S, Skv=S, Hq=H, Hkv=H, Hr=Hr, causal=causal)
    say(f"case mla prefill fp8 S={S} H={H} Hr={Hr} causal={causal}")
    d, t = _inputs(w)
    o, lse = fa.mla_prefill(t["q_nope"], t["q_rope"], t["k_nope"], t["k_rope"], t["v"], t["q_scale"], t["k_scale"],
                            causal=causal, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    x = _oracle_inputs(d)
    ro, rl = oracle.mla_prefill(x["q_nope"], x["q_rope"], x["k_nope"], x["k_rope"], x["v"], x["q_scale"],
                                x["k_scale"], w.scale, causal)
    assert_close(host_f64(o), ro, FP8_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


def test_mla_prefill_bf16_nope_without_scales():
    w = workload(MLA, Sq=150, Skv=150, Hq=2, Hkv=2)
    rng = np.random.default_rng(11)
    shp = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).cuda().to(torch.bfloat16)
    qn, kn, qr, kr, v = shp(1, 150, 2, 128), shp(1, 150, 2, 128), shp(1, 150, 2, 64), shp(1, 150, 1, 64), shp(1, 150, 2, 128)
    o = fa.mla_prefill(qn, qr, kn, kr, v, None, None, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    ones = np.ones((1, 150, 2))
    ro, _ = oracle.mla_prefill(host_f64(qn), host_f64(qr), host_f64(kn), host_f64(kr), host_f64(v), ones, ones,
                               w.scale, True)
    assert_close(host_f64(o), ro, BF16_TOL, "O")


def test_mla_prefill_full_workload_sampled():
    """The full MLA prefill workload (B1 H128 S8192, e4m3 nope + scales); sampled rows of a few heads."""
    w = workload(MLA)
    say(f"case {w.name} (sampled rows)")
    d, t = _inputs(w)
    o, lse = fa.mla_prefill(t["q_nope"], t["q_rope"], t["k_nope"], t["k_rope"], t["v"], t["q_scale"], t["k_scale"],
                            causal=True, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095, 8191], rng.integers(0, 8192, 10)]))
    got, ref, gl, rlse = [], [], [], []
    for h in (0, 77, 127):
        sl = lambda a: a[:, :, h:h + 1]
        ro, rl = oracle.mla_prefill_rows(
            oracle.e4m3_to_f64(sl(d["q_nope"])), oracle.bf16_to_f64(sl(d["q_rope"])),
            oracle.e4m3_to_f64(sl(d["k_nope"])), oracle.bf16_to_f64(d["k_rope"]), oracle.bf16_to_f64(sl(d["v"])),
            sl(d["q_scale"]).astype(np.float64), sl(d["k_scale"]).astype(np.float64), w.scale, True, 0, 0, rows)
        got.append(host_f64(o[0, rows, h])); ref.append(ro)
        gl.append(lse[0, h, rows].cpu().numpy()); rlse.append(rl)
    assert_close(np.stack(got), np.stack(ref), FP8_TOL, "O sampled")
    assert_lse_close(np.stack(gl), np.stack(rlse), "LSE sampled")
