"""GPU parity of attn_decode_fwd and mla_decode_fwd (split-KV + combine) against the oracle."""
import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as fa
import oracle
from tests.helpers import BF16_TOL, E4M3_CACHE_TOL, assert_close, assert_lse_close, dev, dev_bf16, host_f64, say
from workloads import make_decode, make_mla_decode, workload
from workloads.encode import bf16_bits

pytestmark = pytest.mark.gpu

GQA = "gqa_decode_bf16_b64_hq32_hkv8_d128_l8192"
MLA = "mla_decode_bf16_b64_h128_dk576_dv512_l4096"


def _gqa(w, lens=None, batches=None):
    d = make_decode(w, batches=batches, lens=lens)
    return dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]), dev(d["kv_lens"])


def _check_gqa(w, lens):
    say(f"case gqa decode B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lmax={w.Skv} lens={list(lens)[:8]}")
    q, k, v, kl = _gqa(w, lens=lens)
    o, lse = fa.decode(q, k, v, kl, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(host_f64(q), host_f64(k), host_f64(v), np.asarray(lens), w.scale)
    assert_close(host_f64(o), ro, BF16_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (16, 1), (12, 4)])
def test_gqa_decode_small(Hq, Hkv):
    lens = [1, 31, 32, 33, 257, 1000, 0, 513]
    w = workload(GQA, B=len(lens), Hq=Hq, Hkv=Hkv, Skv=1000)
    _check_gqa(w, lens)


def test_decode_lengths_out_of_range_are_clamped():
    """kv_lens entries below 0 or above max_kv_len are clamped to [0, max_kv_len] in the kernels
    (the ABI's stated behaviour): the result equals the call with the clamped lengths."""
    raw = np.array([-5, 1000, 1700, 3, -1], np.int32)
    clamped = np.clip(raw, 0, 1000)
    w = workload(GQA, B=len(raw), Hq=8, Hkv=2, Skv=1000)
    q, k, v, _ = _gqa(w, lens=clamped)
    o, lse = fa.decode(q, k, v, dev(raw), scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(host_f64(q), host_f64(k), host_f64(v), clamped, w.scale)
    assert_close(host_f64(o), ro, BF16_TOL, "GQA O")
    assert_lse_close(lse.cpu().numpy(), rl, "GQA LSE")
    wm = workload(MLA, B=len(raw), Hq=16, Skv=1000)
    d = make_mla_decode(wm, lens=clamped)
    qm, kvm = dev_bf16(d["q"]), dev_bf16(d["kv"])
    om, lm = fa.mla_decode(qm, kvm, dev(raw), dv=512, scale=wm.scale, return_lse=True)
    torch.cuda.synchronize()
    rom, rlm = oracle.mla_decode(host_f64(qm), host_f64(kvm), clamped, 512, wm.scale)
    assert_close(host_f64(om), rom, BF16_TOL, "MLA O")
    assert_lse_close(lm.cpu().numpy(), rlm, "MLA LSE")


def test_gqa_decode_long_single_sequence():
    w = workload(GQA, B=1, Skv=20000)
    _check_gqa(w, [19999])


def test_gqa_decode_full_workload_sampled():
    """The full decode workload (B64, 32/8 heads, cache 8192, lengths U[1024, 8192]); sampled sequences."""
    w = workload(GQA)
    say(f"case {w.name} (sampled sequences)")
    q, k, v, kl = _gqa(w)
    o, lse = fa.decode(q, k, v, kl, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    lens = kl.cpu().numpy()
    picks = [int(np.argmin(lens)), int(np.argmax(lens)), 0, 63, 31]
    ro, rl = [], []
    for b in picks:
        L = int(lens[b])
        r, l = oracle.decode(host_f64(q[b:b + 1]), host_f64(k[b:b + 1, :L]), host_f64(v[b:b + 1, :L]),
                             np.array([L]), w.scale)
        ro.append(r[0]); rl.append(l[0])
    assert_close(host_f64(o[picks]), np.stack(ro), BF16_TOL, "O sampled")
    assert_lse_close(lse[picks].cpu().numpy(), np.stack(rl), "LSE sampled")


def test_gqa_decode_matches_single_row_prefill():
    """A decode row equals the last row of a bottom-right causal prefill over the same keys."""
    w = workload(GQA, B=2, Skv=700)
    q, k, v, kl = _gqa(w, lens=[700, 700])
    od = fa.decode(q, k, v, kl, scale=w.scale)
    op = fa.prefill(q[:, None].contiguous(), k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert_close(host_f64(od), host_f64(op[:, 0]), BF16_TOL, "decode vs prefill")


def test_gqa_decode_zero_query_gives_mean():
    lens = [5, 300]
    w = workload(GQA, B=2, Hq=8, Hkv=2, Skv=300)
    q, k, v, kl = _gqa(w, lens=lens)
    q.zero_()
    o = fa.decode(q, k, v, kl)
    torch.cuda.synchronize()
    vv = host_f64(v)
    ref = np.stack([np.repeat(vv[b, :lens[b]].mean(0), 4, axis=0) for b in range(2)])
    assert_close(host_f64(o), ref, BF16_TOL, "mean of V")


def _mla(w, lens=None):
    d = make_mla_decode(w, lens=lens)
    return dev_bf16(d["q"]), dev_bf16(d["kv"]), dev(d["kv_lens"])


@pytest.mark.parametrize("H", [128, 16, 32, 48, 64, 80, 96, 112])
def test_mla_decode_small(H):
    lens = [1, 33, 300, 0, 128]
    w = workload(MLA, B=len(lens), Hq=H, Skv=300)
    say(f"case mla decode H={H} lens={lens}")
    q, kv, kl = _mla(w, lens=lens)
    o, lse = fa.mla_decode(q, kv, kl, dv=512, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(host_f64(q), host_f64(kv), np.asarray(lens), 512, w.scale)
    assert_close(host_f64(o), ro, BF16_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


def test_mla_decode_full_workload_sampled():
    w = workload(MLA)
    say(f"case {w.name} (sampled sequences)")
    q, kv, kl = _mla(w)
    o, lse = fa.mla_decode(q, kv, kl, dv=512, scale=w.scale, return_lse=True)
    torch.cuda.synchronize()
    picks = [0, 37, 63]
    ro, rl = oracle.mla_decode(host_f64(q[picks]), host_f64(kv[picks]), np.full(3, 4096), 512, w.scale)
    assert_close(host_f64(o[picks]), ro, BF16_TOL, "O sampled")
    assert_lse_close(lse[picks].cpu().numpy(), rl, "LSE sampled")


def test_mla_decode_growing_scores():
    """Scores that climb steeply along each sequence: the 64 rope columns of every key are a
    ramp times one direction that all queries share (plus noise), so each split of 8 tiles
    sees its scores grow by hundreds of log2 units (the kernel passes over such a split again
    with a higher softmax reference).  V (the first 512 columns) stays small noise.  Checked
    against the oracle."""
    B, H, L = 64, 16, 1024
    rng = np.random.default_rng(11)
    u = rng.standard_normal(64)
    q = rng.standard_normal((B, H, 576))
    q[..., 512:] = u
    kv = 0.5 * rng.standard_normal((B, L, 576))
    kv[..., 512:] += (330.0 * np.arange(L) / L)[None, :, None] * u
    lens = np.full(B, L, np.int32)
    lens[1], lens[2] = 1000, 777
    qd, kvd = dev_bf16(bf16_bits(q.astype(np.float32))), dev_bf16(bf16_bits(kv.astype(np.float32)))
    scale = 576 ** -0.5
    say(f"case mla decode growing scores B={B} H={H} L={L}")
    o, lse = fa.mla_decode(qd, kvd, dev(lens), dv=512, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(host_f64(qd), host_f64(kvd), lens, 512, scale)
    assert_close(host_f64(o), ro, BF16_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


# ------------------------------------------------------------------------------------------
# e4m3 caches with per-token scales: the oracle runs on the dequantised caches (code * scale)

GQA8 = "gqa_decode_fp8_b64_hq32_hkv8_d128_l8192"


def _gqa8(w, lens=None):
    d = make_decode(w, lens=lens)
    t = (dev_bf16(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["kv_lens"]), dev(d["k_scale"]), dev(d["v_scale"]))
    kd = oracle.e4m3_to_f64(d["k"]) * d["k_scale"][..., None].astype(np.float64)
    vd = oracle.e4m3_to_f64(d["v"]) * d["v_scale"][..., None].astype(np.float64)
    return t, kd, vd


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (16, 1), (12, 4)])
def test_gqa_decode_fp8_small(Hq, Hkv):
    lens = [1, 31, 32, 33, 257, 1000, 0, 513]
    w = workload(GQA8, B=len(lens), Hq=Hq, Hkv=Hkv, Skv=1000)
    say(f"case gqa decode e4m3 Hq={Hq} Hkv={Hkv} lens={lens}")
    (q, k, v, kl, ks, vs), kd, vd = _gqa8(w, lens=lens)
    o, lse = fa.decode(q, k, v, kl, scale=w.scale, return_lse=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(host_f64(q), kd, vd, np.asarray(lens), w.scale)
    assert_close(host_f64(o), ro, E4M3_CACHE_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


@pytest.mark.parametrize("G", range(1, 17))
def test_gqa_decode_every_group_size(G):
    """Every compiled group size (query heads per kv head, 1..16) over two kv heads, with a
    bf16 and an e4m3 cache."""
    lens = [1, 33, 200, 0]
    _check_gqa(workload(GQA, B=len(lens), Hq=2 * G, Hkv=2, Skv=200), lens)
    w = workload(GQA8, B=len(lens), Hq=2 * G, Hkv=2, Skv=200)
    say(f"case gqa decode e4m3 Hq={w.Hq} Hkv={w.Hkv} lens={lens}")
    (q, k, v, kl, ks, vs), kd, vd = _gqa8(w, lens=lens)
    o, lse = fa.decode(q, k, v, kl, scale=w.scale, return_lse=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(host_f64(q), kd, vd, np.asarray(lens), w.scale)
    assert_close(host_f64(o), ro, E4M3_CACHE_TOL, "O e4m3")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE e4m3")


def test_gqa_decode_fp8_full_workload_sampled():
    w = workload(GQA8)
    say(f"case {w.name} (sampled sequences)")
    (q, k, v, kl, ks, vs), kd, vd = _gqa8(w)
    o, lse = fa.decode(q, k, v, kl, scale=w.scale, return_lse=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    lens = kl.cpu().numpy()
    picks = [int(np.argmin(lens)), int(np.argmax(lens)), 0, 63, 31]
    ro, rl = [], []
    for b in picks:
        L = int(lens[b])
        r, l = oracle.decode(host_f64(q[b:b + 1]), kd[b:b + 1, :L], vd[b:b + 1, :L], np.array([L]), w.scale)
        ro.append(r[0]); rl.append(l[0])
    assert_close(host_f64(o[picks]), np.stack(ro), E4M3_CACHE_TOL, "O sampled")
    assert_lse_close(lse[picks].cpu().numpy(), np.stack(rl), "LSE sampled")


def test_gqa_decode_fp8_matches_bf16_on_the_dequantised_cache():
    """The e4m3 path equals the bf16 path run on the dequantised cache (rounded to bf16)."""
    lens = [700, 129]
    w = workload(GQA8, B=2, Skv=700)
    (q, k, v, kl, ks, vs), kd, vd = _gqa8(w, lens=lens)
    o8 = fa.decode(q, k, v, kl, scale=w.scale, k_scale=ks, v_scale=vs)
    kb = torch.from_numpy(kd.astype(np.float32)).to(torch.bfloat16).cuda()
    vb = torch.from_numpy(vd.astype(np.float32)).to(torch.bfloat16).cuda()
    ob = fa.decode(q, kb, vb, kl, scale=w.scale)
    torch.cuda.synchronize()
    assert_close(host_f64(o8), host_f64(ob), BF16_TOL, "e4m3 vs bf16 path")


MLA8 = "mla_decode_fp8_b64_h128_dk576_dv512_l4096"


def _mla8(w, lens=None):
    d = make_mla_decode(w, lens=lens)
    t = (dev_bf16(d["q"]), dev(d["kv"]), dev(d["kv_lens"]), dev(d["kv_scale"]))
    return t, oracle.e4m3_to_f64(d["kv"]) * d["kv_scale"][..., None].astype(np.float64)


@pytest.mark.parametrize("H", [128, 16, 32, 48, 64, 80, 96, 112])
def test_mla_decode_fp8_small(H):
    lens = [1, 33, 300, 0, 128, 31, 32, 255]
    w = workload(MLA8, B=len(lens), Hq=H, Skv=300)
    say(f"case mla decode e4m3 H={H} lens={lens}")
    (q, kv, kl, ks), kvd = _mla8(w, lens=lens)
    o, lse = fa.mla_decode(q, kv, kl, dv=512, scale=w.scale, return_lse=True, kv_scale=ks)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(host_f64(q), kvd, np.asarray(lens), 512, w.scale)
    assert_close(host_f64(o), ro, E4M3_CACHE_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


def test_mla_decode_fp8_long_single_sequence():
    w = workload(MLA8, B=1, Skv=9000)
    say(f"case mla decode e4m3 B=1 len=8999")
    (q, kv, kl, ks), kvd = _mla8(w, lens=[8999])
    o, lse = fa.mla_decode(q, kv, kl, dv=512, scale=w.scale, return_lse=True, kv_scale=ks)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(host_f64(q), kvd, np.array([8999]), 512, w.scale)
    assert_close(host_f64(o), ro, E4M3_CACHE_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


def test_mla_decode_fp8_full_workload_sampled():
    w = workload(MLA8)
    say(f"case {w.name} (sampled sequences)")
    (q, kv, kl, ks), kvd = _mla8(w)
    o, lse = fa.mla_decode(q, kv, kl, dv=512, scale=w.scale, return_lse=True, kv_scale=ks)
    torch.cuda.synchronize()
    picks = [0, 37, 63]
    ro, rl = oracle.mla_decode(host_f64(q[picks]), kvd[picks], np.full(3, 4096), 512, w.scale)
    assert_close(host_f64(o[picks]), ro, E4M3_CACHE_TOL, "O sampled")
    assert_lse_close(lse[picks].cpu().numpy(), rl, "LSE sampled")


def test_mla_decode_fp8_matches_bf16_on_the_dequantised_cache():
    """The e4m3 path equals the bf16 path run on the dequantised cache (rounded to bf16)."""
    lens = [700, 97]
    w = workload(MLA8, B=2, Skv=700)
    (q, kv, kl, ks), kvd = _mla8(w, lens=lens)
    o8 = fa.mla_decode(q, kv, kl, dv=512, scale=w.scale, kv_scale=ks)
    kvb = torch.from_numpy(kvd.astype(np.float32)).to(torch.bfloat16).cuda()
    ob = fa.mla_decode(q, kvb, kl, dv=512, scale=w.scale)
    torch.cuda.synchronize()
    assert_close(host_f64(o8), host_f64(ob), BF16_TOL, "e4m3 vs bf16 path")


# ------------------------------------------------------------------------------------------
# Head dim 64 (bf16 and e4m3 caches)

@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (16, 1), (12, 4), (14, 2)])
def test_gqa_decode_d64(Hq, Hkv):
    lens = [1, 31, 32, 33, 257, 1000, 0, 513]
    w = workload(GQA, B=len(lens), Hq=Hq, Hkv=Hkv, Skv=1000, D=64, Dv=64, scale=64 ** -0.5)
    _check_gqa(w, lens)
    w8 = workload(GQA8, B=len(lens), Hq=Hq, Hkv=Hkv, Skv=1000, D=64, Dv=64, scale=64 ** -0.5)
    say(f"case gqa decode e4m3 D=64 Hq={Hq} Hkv={Hkv} lens={lens}")
    (q, k, v, kl, ks, vs), kd, vd = _gqa8(w8, lens=lens)
    o, lse = fa.decode(q, k, v, kl, scale=w8.scale, return_lse=True, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(host_f64(q), kd, vd, np.asarray(lens), w8.scale)
    assert_close(host_f64(o), ro, E4M3_CACHE_TOL, "O e4m3")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE e4m3")


def test_gqa_decode_d64_long_sequences():
    """Head dim 64 over a batch with long sequences (many 1024-key splits) and a single long one."""
    lens = [8192, 5000, 1024, 3333]
    _check_gqa(workload(GQA, B=4, Hq=32, Hkv=8, Skv=8192, D=64, Dv=64, scale=64 ** -0.5), lens)
    _check_gqa(workload(GQA, B=1, Hq=4, Hkv=1, Skv=12000, D=64, Dv=64, scale=64 ** -0.5), [11999])


# ------------------------------------------------------------------------------------------
# Invariants of the split-KV path: the result does not depend on how the keys are split, and
# a call repeated on the same inputs gives the same bits.

def _pad_cache(x: torch.Tensor, L: int) -> torch.Tensor:
    """The same cache rows in a cache of max length L (rows past the old end are zero)."""
    out = torch.zeros((x.shape[0], L) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    out[:, :x.shape[1]] = x
    return out


def test_gqa_decode_independent_of_the_split_plan():
    """The same sequences in caches of max length 1024, 4096 and 16384: the split planner cuts
    them into 32-, 128- and 512-key splits (one wave per (split, batch, kv head), at least
    2048 waves); every result matches the oracle and the others."""
    lens = [1000, 517, 33, 1, 999, 640, 256, 800]
    for dtype_name in (GQA, GQA8):
        w = workload(dtype_name, B=8, Hq=32, Hkv=8, Skv=1000)
        outs = []
        if dtype_name == GQA:
            q, k, v, kl = _gqa(w, lens=lens)
            kd, vd, extra = host_f64(k), host_f64(v), {}
        else:
            (q, k, v, kl, ks, vs), kd, vd = _gqa8(w, lens=lens)
        ro, rl = oracle.decode(host_f64(q), kd, vd, np.asarray(lens), w.scale)
        for L in (1024, 4096, 16384):
            say(f"case gqa decode split plan {dtype_name} Lmax={L} ({fa.decode_workspace_size(8, 32, 8, 128, L)} B)")
            if dtype_name == GQA:
                o, lse = fa.decode(q, _pad_cache(k, L), _pad_cache(v, L), kl, scale=w.scale, return_lse=True)
            else:
                o, lse = fa.decode(q, _pad_cache(k, L), _pad_cache(v, L), kl, scale=w.scale, return_lse=True,
                                   k_scale=_pad_cache(ks, L), v_scale=_pad_cache(vs, L))
            torch.cuda.synchronize()
            assert_close(host_f64(o), ro, BF16_TOL if dtype_name == GQA else E4M3_CACHE_TOL, f"O Lmax={L}")
            assert_lse_close(lse.cpu().numpy(), rl, f"LSE Lmax={L}")
            outs.append(host_f64(o))
        for o in outs[1:]:
            assert_close(o, outs[0], BF16_TOL, "against the 32-key splits")


def test_mla_decode_independent_of_the_split_plan():
    """MLA decode of the same sequences in latent caches of max length 1024, 8192 and 16384:
    32-, 128- and 256-key splits."""
    lens = [1000, 333, 1, 700]
    for name in (MLA, MLA8):
        w = workload(name, B=4, Hq=128, Skv=1000)
        if name == MLA:
            q, kv, kl = _mla(w, lens=lens)
            kvd, extra = host_f64(kv), {}
        else:
            (q, kv, kl, ks), kvd = _mla8(w, lens=lens)
        ro, rl = oracle.mla_decode(host_f64(q), kvd, np.asarray(lens), 512, w.scale)
        outs = []
        for L in (1024, 8192, 16384):
            say(f"case mla decode split plan {name} Lmax={L} ({fa.mla_decode_workspace_size(4, 128, 512, L)} B)")
            if name == MLA:
                o, lse = fa.mla_decode(q, _pad_cache(kv, L), kl, dv=512, scale=w.scale, return_lse=True)
            else:
                o, lse = fa.mla_decode(q, _pad_cache(kv, L), kl, dv=512, scale=w.scale, return_lse=True,
                                       kv_scale=_pad_cache(ks, L))
            torch.cuda.synchronize()
            assert_close(host_f64(o), ro, BF16_TOL if name == MLA else E4M3_CACHE_TOL, f"O Lmax={L}")
            assert_lse_close(lse.cpu().numpy(), rl, f"LSE Lmax={L}")
            outs.append(host_f64(o))
        for o in outs[1:]:
            assert_close(o, outs[0], BF16_TOL, "against the 32-key splits")


def test_decode_calls_are_bitwise_repeatable():
    """The same call twice gives identical bits (fixed merge order, no atomics), for GQA and MLA
    decode with bf16 and e4m3 caches."""
    lens = [1000, 517, 33, 1, 640]
    w = workload(GQA, B=5, Hq=32, Hkv=8, Skv=1000)
    q, k, v, kl = _gqa(w, lens=lens)
    runs = [fa.decode(q, k, v, kl, scale=w.scale, return_lse=True) for _ in range(3)]
    w8 = workload(GQA8, B=5, Hq=16, Hkv=2, Skv=1000, D=64, Dv=64, scale=64 ** -0.5)
    (q8, k8, v8, kl8, ks, vs), _, _ = _gqa8(w8, lens=lens)
    runs8 = [fa.decode(q8, k8, v8, kl8, scale=w8.scale, return_lse=True, k_scale=ks, v_scale=vs) for _ in range(3)]
    wm = workload(MLA, B=5, Hq=128, Skv=1000)
    qm, kvm, klm = _mla(wm, lens=lens)
    runsm = [fa.mla_decode(qm, kvm, klm, dv=512, scale=wm.scale, return_lse=True) for _ in range(3)]
    wm8 = workload(MLA8, B=5, Hq=64, Skv=1000)
    (qm8, kvm8, klm8, ksm), _ = _mla8(wm8, lens=lens)
    runsm8 = [fa.mla_decode(qm8, kvm8, klm8, dv=512, scale=wm8.scale, return_lse=True, kv_scale=ksm) for _ in range(3)]
    torch.cuda.synchronize()
    for name, rs in (("gqa bf16", runs), ("gqa e4m3 d64", runs8), ("mla bf16", runsm), ("mla e4m3", runsm8)):
        say(f"case repeatability {name}")
        for o, lse in rs[1:]:
            assert torch.equal(o.view(torch.int16), rs[0][0].view(torch.int16)), name
            assert torch.equal(lse.view(torch.int32), rs[0][1].view(torch.int32)), name


def test_decode_identical_value_rows_return_that_row():
    """If every visible V row is the same vector, the output is that vector whatever q and K are
    (the softmax weights sum to one): GQA (bf16, e4m3) and MLA decode."""
    lens = [700, 1, 64]
    w = workload(GQA, B=3, Hq=8, Hkv=2, Skv=700)
    q, k, v, kl = _gqa(w, lens=lens)
    row = v[0, 0, :, :].clone()                           # [Hkv, D]
    v[:] = row[None, None]
    o = fa.decode(q, k, v, kl, scale=w.scale)
    torch.cuda.synchronize()
    ref = np.repeat(host_f64(row)[None], 3, axis=0).repeat(4, axis=1)   # head h reads kv head h // 4
    assert_close(host_f64(o), ref, BF16_TOL, "GQA identical V rows")
    w8 = workload(GQA8, B=3, Hq=8, Hkv=2, Skv=700)
    (q8, k8, v8, kl8, ks, vs), _, _ = _gqa8(w8, lens=lens)
    v8[:] = v8[0, 0][None, None]
    vs[:] = vs[0, 0][None, None]
    o8 = fa.decode(q8, k8, v8, kl8, scale=w8.scale, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    rowd = oracle.e4m3_to_f64(v8[0, 0].cpu().numpy()) * vs[0, 0].cpu().numpy()[:, None].astype(np.float64)
    assert_close(host_f64(o8), np.repeat(rowd[None], 3, axis=0).repeat(4, axis=1), E4M3_CACHE_TOL,
                 "GQA e4m3 identical V rows")
    wm = workload(MLA, B=3, Hq=32, Skv=700)
    qm, kvm, klm = _mla(wm, lens=lens)
    # the first 512 columns (V) equal across rows; the rope columns (K only) stay random
    kvm[:, :, :512] = kvm[0, 0, :512][None, None]
    om = fa.mla_decode(qm, kvm, klm, dv=512, scale=wm.scale)
    torch.cuda.synchronize()
    refm = np.broadcast_to(host_f64(kvm[0, 0, :512]), (3, 32, 512))
    assert_close(host_f64(om), refm, BF16_TOL, "MLA identical V rows")
