"""GPU parity of mla_prefill_fwd (e4m3 nope with per-token scales + bf16 rope; bf16 or e4m3 V)
against the oracle run on the dequantised inputs."""
import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as fa
import oracle
from tests.helpers import (BF16_TOL, FP8_TOL, assert_close, assert_lse_close, dev, dev_bf16, host_f64, say)
from workloads import make_mla_prefill, quantize_rows_e4m3, workload

pytestmark = pytest.mark.gpu

MLA = "mla_prefill_fp8_causal_b1_h128_s8192"


MLA8V = "mla_prefill_fp8v_causal_b1_h128_s8192"


def _inputs(w):
    d = make_mla_prefill(w)
    names = ("q_nope", "k_nope", "q_scale", "k_scale", "q_rope", "k_rope", "v") + (("v_scale",) if "v_scale" in d else ())
    t = {k: (dev_bf16(d[k]) if d[k].dtype == np.uint16 else dev(d[k])) for k in names}
    return d, t


def _v_f64(d):
    """V as the oracle sees it: bf16 values, or e4m3 codes times their row scales."""
    if "v_scale" in d:
        return oracle.e4m3_to_f64(d["v"]) * d["v_scale"][..., None].astype(np.float64)
    return oracle.bf16_to_f64(d["v"])


def _oracle_inputs(d):
    return dict(q_nope=oracle.e4m3_to_f64(d["q_nope"]), k_nope=oracle.e4m3_to_f64(d["k_nope"]),
                q_rope=oracle.bf16_to_f64(d["q_rope"]), k_rope=oracle.bf16_to_f64(d["k_rope"]),
                v=_v_f64(d), q_scale=d["q_scale"].astype(np.float64), k_scale=d["k_scale"].astype(np.float64))


def _call(t, w, causal):
    return fa.mla_prefill(t["q_nope"], t["q_rope"], t["k_nope"], t["k_rope"], t["v"], t["q_scale"], t["k_scale"],
                          causal=causal, scale=w.scale, return_lse=True, v_scale=t.get("v_scale"))


@pytest.mark.parametrize("name", [MLA, MLA8V])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,H,Hr", [(200, 4, 1), (333, 2, 2), (64, 3, 1)])
def test_mla_prefill_fp8_small(name, causal, S, H, Hr):
    w = workload(name, Sq=S, Skv=S, Hq=H, Hkv=H, Hr=Hr, causal=causal)
    say(f"case {name} S={S} H={H} Hr={Hr} causal={causal}")
    d, t = _inputs(w)
    o, lse = _call(t, w, causal)
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


@pytest.mark.parametrize("causal", [True, False])
def test_mla_prefill_bf16_nope_with_scales_and_e4m3_v(causal):
    """bf16 nope operands with per-token q/k scales, one k_rope head per query head, and an
    e4m3 V with one fp32 scale per (token, head) row."""
    S, H = 170, 2
    rng = np.random.default_rng(12)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    bf = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    qn, kn, qr, kr = bf(f(1, S, H, 128)), bf(f(1, S, H, 128)), bf(f(1, S, H, 64)), bf(f(1, S, H, 64))
    qs = rng.uniform(0.5, 2.0, (1, S, H)).astype(np.float32)
    ks = rng.uniform(0.5, 2.0, (1, S, H)).astype(np.float32)
    codes, vs = quantize_rows_e4m3(f(1, S, H, 128))
    scale = 192 ** -0.5
    say(f"case mla prefill bf16 nope + scales, e4m3 V, S={S} H={H} Hr={H} causal={causal}")
    o, lse = fa.mla_prefill(qn, qr, kn, kr, dev(codes), dev(qs), dev(ks), causal=causal, scale=scale,
                            return_lse=True, v_scale=dev(vs))
    torch.cuda.synchronize()
    vd = oracle.e4m3_to_f64(codes) * vs[..., None].astype(np.float64)
    ro, rl = oracle.mla_prefill(host_f64(qn), host_f64(qr), host_f64(kn), host_f64(kr), vd, qs, ks, scale, causal)
    assert_close(host_f64(o), ro, FP8_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


@pytest.mark.parametrize("name", [MLA, MLA8V])
def test_mla_prefill_full_workload_sampled(name):
    """The full MLA prefill workload (B1 H128 S8192, e4m3 nope + scales; bf16 or e4m3 V); sampled
    rows of a few heads."""
    w = workload(name)
    say(f"case {w.name} (sampled rows)")
    d, t = _inputs(w)
    o, lse = _call(t, w, True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095, 8191], rng.integers(0, 8192, 10)]))
    got, ref, gl, rlse = [], [], [], []
    for h in (0, 77, 127):
        sl = lambda a: a[:, :, h:h + 1]
        ro, rl = oracle.mla_prefill_rows(
            oracle.e4m3_to_f64(sl(d["q_nope"])), oracle.bf16_to_f64(sl(d["q_rope"])),
            oracle.e4m3_to_f64(sl(d["k_nope"])), oracle.bf16_to_f64(d["k_rope"]), sl(_v_f64(d)),
            sl(d["q_scale"]).astype(np.float64), sl(d["k_scale"]).astype(np.float64), w.scale, True, 0, 0, rows)
        got.append(host_f64(o[0, rows, h])); ref.append(ro)
        gl.append(lse[0, h, rows].cpu().numpy()); rlse.append(rl)
    assert_close(np.stack(got), np.stack(ref), FP8_TOL, "O sampled")
    assert_lse_close(np.stack(gl), np.stack(rlse), "LSE sampled")


def test_mla_prefill_fp8v_matches_bf16v_on_the_dequantised_values():
    """e4m3 V with scales against bf16 V holding the dequantised values (code * scale rounded to
    bf16): two GPU outputs, each rounded to bf16 on its own, so they may differ by a whole bf16
    ulp (1.6e-2 for |O| in [2, 4)); held to the e4m3 path's bar."""
    w = workload(MLA8V, Sq=300, Skv=300, Hq=3, Hkv=3)
    d, t = _inputs(w)
    o8, _ = _call(t, w, True)
    vb = torch.from_numpy((oracle.e4m3_to_f64(d["v"]) * d["v_scale"][..., None]).astype(np.float32)).cuda()
    tb = dict(t, v=vb.to(torch.bfloat16))
    tb.pop("v_scale")
    ob, _ = _call(tb, w, True)
    torch.cuda.synchronize()
    assert_close(host_f64(o8), host_f64(ob), FP8_TOL, "e4m3 V vs bf16 V")
