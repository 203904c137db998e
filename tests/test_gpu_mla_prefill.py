"""GPU parity of mla_prefill_fwd (e4m3 nope with per-token scales + bf16 rope; bf16 or e4m3 V)
against the oracle run on the dequantised inputs."""
import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as fa
import oracle
from tests.helpers import (BF16_TOL, FP8_TOL, assert_close, assert_lse_close, dev, dev_bf16, host_f64, say)
from workloads import e4m3_encode, make_mla_prefill, quantize_rows_e4m3, workload

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


# ------------------------------------------------------------------------------------------
# Batches of several sequences with Sq != Skv: the per-batch offsets of q_nope, q_rope,
# q_scale, k_nope, k_rope, k_scale, v and v_scale, and the bottom-right causal alignment.

def _mla_general(B, Sq, Skv, H, Hr, nope_fp8, with_scales, v_fp8, seed):
    """GPU tensors and the oracle's fp64 view of one MLA prefill problem."""
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    bf = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    qs = ks = None
    if nope_fp8 and with_scales:
        qc, qs = quantize_rows_e4m3(f(B, Sq, H, 128))
        kc, ks = quantize_rows_e4m3(f(B, Skv, H, 128))
    elif nope_fp8:
        # raw e4m3 codes of small values (no scales: q_scale = k_scale = 1)
        qc, kc = e4m3_encode(0.3 * f(B, Sq, H, 128)), e4m3_encode(0.3 * f(B, Skv, H, 128))
    if nope_fp8:
        qn_t, kn_t = dev(qc), dev(kc)
        qn, kn = oracle.e4m3_to_f64(qc), oracle.e4m3_to_f64(kc)
    else:
        qn_t, kn_t = bf(f(B, Sq, H, 128)), bf(f(B, Skv, H, 128))
        qn, kn = host_f64(qn_t), host_f64(kn_t)
        if with_scales:
            qs = rng.uniform(0.5, 2.0, (B, Sq, H)).astype(np.float32)
            ks = rng.uniform(0.5, 2.0, (B, Skv, H)).astype(np.float32)
    qr_t, kr_t = bf(f(B, Sq, H, 64)), bf(f(B, Skv, Hr, 64))
    vs = None
    if v_fp8:
        vc, vs = quantize_rows_e4m3(f(B, Skv, H, 128))
        v_t, v = dev(vc), oracle.e4m3_to_f64(vc) * vs[..., None].astype(np.float64)
    else:
        v_t = bf(f(B, Skv, H, 128))
        v = host_f64(v_t)
    t = dict(q_nope=qn_t, k_nope=kn_t, q_rope=qr_t, k_rope=kr_t, v=v_t,
             q_scale=None if qs is None else dev(qs), k_scale=None if ks is None else dev(ks),
             v_scale=None if vs is None else dev(vs))
    x = dict(q_nope=qn, k_nope=kn, q_rope=host_f64(qr_t), k_rope=host_f64(kr_t), v=v,
             q_scale=np.ones((B, Sq, H)) if qs is None else qs.astype(np.float64),
             k_scale=np.ones((B, Skv, H)) if ks is None else ks.astype(np.float64))
    return t, x


MLA_BATCHED = [
    # B, Sq, Skv, H, Hr, nope e4m3, scales, V e4m3, causal
    (2, 77, 333, 3, 1, True, True, False, True),      # Sq < Skv, shared rope head
    (3, 200, 90, 2, 2, True, True, False, True),      # Sq > Skv: leading rows see no key
    (2, 150, 260, 2, 2, True, True, True, False),     # e4m3 V, one rope head per head
    (3, 129, 65, 4, 1, True, True, True, True),       # e4m3 V, Sq > Skv
    (2, 100, 300, 2, 1, False, True, False, True),    # bf16 nope with scales
    (2, 190, 130, 3, 3, False, False, False, True),   # bf16 nope without scales, Sq > Skv
    (3, 64, 200, 2, 2, False, True, True, False),     # bf16 nope, e4m3 V, non-causal
    (2, 96, 257, 2, 1, True, False, False, True),     # e4m3 nope without scales
    (2, 300, 300, 2, 1, True, True, False, True),     # Sq = Skv across two sequences
    (2, 2080, 2200, 2, 1, True, True, False, True),   # long causal rows: 256-row blocks, ragged tail
    (1, 2300, 2100, 2, 2, True, True, True, True),    # the same with e4m3 V, Sq > Skv
]


@pytest.mark.parametrize("B,Sq,Skv,H,Hr,nope8,scales,v8,causal", MLA_BATCHED)
def test_mla_prefill_batched(B, Sq, Skv, H, Hr, nope8, scales, v8, causal):
    say(f"case mla prefill B={B} Sq={Sq} Skv={Skv} H={H} Hr={Hr} nope_e4m3={nope8} scales={scales} "
        f"v_e4m3={v8} causal={causal}")
    t, x = _mla_general(B, Sq, Skv, H, Hr, nope8, scales, v8, seed=100 + B * 7 + Sq)
    o, lse = fa.mla_prefill(t["q_nope"], t["q_rope"], t["k_nope"], t["k_rope"], t["v"], t["q_scale"],
                            t["k_scale"], causal=causal, scale=192 ** -0.5, return_lse=True, v_scale=t["v_scale"])
    torch.cuda.synchronize()
    ro, rl = oracle.mla_prefill(x["q_nope"], x["q_rope"], x["k_nope"], x["k_rope"], x["v"], x["q_scale"],
                                x["k_scale"], 192 ** -0.5, causal)
    tol = FP8_TOL if (nope8 or v8) else BF16_TOL
    assert_close(host_f64(o), ro, tol, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")
    # each sequence alone gives the same rows (the batch offsets select the right sequence)
    b = B - 1
    ob = fa.mla_prefill(*(t[n][b:b + 1].contiguous() for n in ("q_nope", "q_rope", "k_nope", "k_rope", "v")),
                        *(None if t[n] is None else t[n][b:b + 1].contiguous() for n in ("q_scale", "k_scale")),
                        causal=causal, scale=192 ** -0.5,
                        v_scale=None if t["v_scale"] is None else t["v_scale"][b:b + 1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(ob[0].view(torch.int16), o[b].view(torch.int16)), "last sequence alone differs"


def test_mla_prefill_bitwise_repeatable():
    """Two calls on the same inputs give the same bits: the 256-row path whose second causal block
    runs its keys in descending order and whose output rows go through LDS, and the 128-row
    path with e4m3 V."""
    for args in [(1, 2100, 2100, 2, 1, True, True, False), (2, 300, 333, 2, 2, True, True, True)]:
        B, Sq, Skv, H, Hr, nope8, scales, v8 = args
        say(f"case mla prefill repeatability B={B} Sq={Sq} Skv={Skv} H={H} v_e4m3={v8}")
        t, _ = _mla_general(B, Sq, Skv, H, Hr, nope8, scales, v8, seed=5 + Sq)
        outs = [fa.mla_prefill(t["q_nope"], t["q_rope"], t["k_nope"], t["k_rope"], t["v"], t["q_scale"], t["k_scale"],
                               causal=True, scale=192 ** -0.5, return_lse=True, v_scale=t["v_scale"]) for _ in range(2)]
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16)), "O differs between calls"
        assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32)), "LSE differs between calls"
