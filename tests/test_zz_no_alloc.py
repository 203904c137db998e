"""attn_decode_fwd_static -- GQA decode with the split partials in the library's static per-GPU
buffer (no workspace, no allocation) -- against attn_decode_fwd on the same inputs, called
through the C ABI: two calls in a row, the second on a smaller problem, with a bf16 and an
e4m3 cache.  The kernels and split plan are those of attn_decode_fwd, so the outputs match it
bit for bit (and so lie within the bf16 bar of it)."""
import ctypes

import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as fa
from tests.helpers import BF16_TOL, assert_close, dev, dev_bf16, host_f64, say
from workloads import make_decode, workload

pytestmark = pytest.mark.gpu

GQA = "gqa_decode_bf16_b64_hq32_hkv8_d128_l8192"
GQA8 = "gqa_decode_fp8_b64_hq32_hkv8_d128_l8192"


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _static_call(q, k, v, kl, ks, vs, fp8, scale):
    B, Hq, D = q.shape
    Lmax, Hkv = k.shape[1], k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    st = fa.lib().attn_decode_fwd_static(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(kl), _p(ks), _p(vs),
                                         fa.ATTN_FP8_E4M3 if fp8 else fa.ATTN_BF16, B, Hq, Hkv, D, Lmax,
                                         scale, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fa.status_string(st)
    return o, lse


def _inputs(name, **kw):
    w = workload(name, **kw)
    d = make_decode(w)
    t = dict(q=dev_bf16(d["q"]), kl=dev(d["kv_lens"]))
    if w.dtype == "fp8":
        t.update(k=dev(d["k"]), v=dev(d["v"]), ks=dev(d["k_scale"]), vs=dev(d["v_scale"]))
    else:
        t.update(k=dev_bf16(d["k"]), v=dev_bf16(d["v"]), ks=None, vs=None)
    return w, t


@pytest.mark.parametrize("name", [GQA, GQA8])
def test_static_decode_matches_the_workspace_entry_point(name):
    cases = [dict(), dict(B=5, Skv=700, Hq=16, Hkv=2, len_lo=1, len_hi=700)]   # full workload, then smaller
    for kw in cases:
        w, t = _inputs(name, **kw)
        fp8 = w.dtype == "fp8"
        need = fa.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.Skv)
        say(f"case static decode {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lmax={w.Skv} partials={need} B")
        assert need <= fa.DECODE_STATIC_SCRATCH_BYTES
        o_s, lse_s = _static_call(t["q"], t["k"], t["v"], t["kl"], t["ks"], t["vs"], fp8, w.scale)
        o_w, lse_w = fa.decode(t["q"], t["k"], t["v"], t["kl"], scale=w.scale, return_lse=True,
                               k_scale=t["ks"], v_scale=t["vs"])
        torch.cuda.synchronize()
        assert_close(host_f64(o_s), host_f64(o_w), BF16_TOL, "static vs workspace O")
        assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16)), "outputs differ bitwise"
        assert torch.equal(lse_s.view(torch.int32), lse_w.view(torch.int32)), "LSEs differ bitwise"


def test_static_decode_binding_and_limit():
    """The binding's decode_static with caller-supplied out/lse allocates nothing and matches
    decode(); a request past the buffer raises before any launch."""
    w, t = _inputs(GQA, B=3, Skv=300, Hq=8, Hkv=2, len_lo=1, len_hi=300)
    out = torch.empty_like(t["q"])
    lse = torch.empty((3, 8), dtype=torch.float32, device="cuda")
    fa.decode_static(t["q"], t["k"], t["v"], t["kl"], scale=w.scale, out=out, lse=lse)
    ref = fa.decode(t["q"], t["k"], t["v"], t["kl"], scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    big = torch.zeros((64, 16384, 8, 128), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    kl = torch.full((64,), 16384, dtype=torch.int32, device="cuda")
    with pytest.raises(fa.AttnError) as e:
        fa.decode_static(q, big, big, kl)
    assert e.value.status == -8
    torch.cuda.synchronize()
