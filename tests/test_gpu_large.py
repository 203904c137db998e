"""GPU parity at tensor sizes past 2^31 elements (64-bit offsets in every kernel): prefill
with 2^31-element q and o, GQA and MLA decode with caches past 2^31 elements whose last batch
entry holds the long sequence.  Inputs are drawn on the device from a seeded generator; the
oracle checks the rows and batch entries at the far ends of the tensors."""
import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as fa
import oracle
from tests.helpers import BF16_TOL, assert_close, assert_lse_close, dev, host_f64, say

pytestmark = pytest.mark.gpu


def _randn(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)


def test_prefill_q_and_o_past_2_31_elements():
    B, Sq, Skv, H, D = 1, 524288, 64, 32, 128  # q, o: 2^31 elements each
    say(f"case large prefill Sq={Sq} Skv={Skv} H={H} D={D} (q, o: {B * Sq * H * D} elements)")
    q = _randn((B, Sq, H, D), 31)
    k = _randn((B, Skv, H, D), 32)
    v = _randn((B, Skv, H, D), 33)
    o, lse = fa.prefill(q, k, v, causal=False, scale=D ** -0.5, return_lse=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, Sq // 2, Sq - 2, Sq - 1])
    kh, vh = host_f64(k), host_f64(v)
    for h in (0, H - 1):
        qs = host_f64(q[:, rows, h:h + 1])
        ro, rl = oracle.prefill_rows(qs, kh[:, :, h:h + 1], vh[:, :, h:h + 1], D ** -0.5, False, 0, 0,
                                     np.arange(len(rows)))
        assert_close(host_f64(o[0, rows, h]), ro, BF16_TOL, f"O head {h}")
        assert_lse_close(lse[0, h, rows].cpu().numpy(), rl, f"LSE head {h}")
    del q, o, lse
    torch.cuda.empty_cache()


def test_gqa_decode_cache_past_2_31_elements():
    B, L, Hq, Hkv, D = 256, 65536, 2, 1, 128  # each cache: 2^31 elements
    say(f"case large GQA decode B={B} max_len={L} (cache: {B * L * Hkv * D} elements)")
    k = _randn((B, L, Hkv, D), 41)
    v = _randn((B, L, Hkv, D), 42)
    q = _randn((B, Hq, D), 43)
    lens = np.full(B, 3, np.int32)
    lens[B - 1], lens[B - 2], lens[0] = L, L - 17, 1
    o, lse = fa.decode(q, k, v, dev(lens), scale=D ** -0.5, return_lse=True)
    torch.cuda.synchronize()
    bs = [0, B - 2, B - 1]
    ro, rl = oracle.decode(host_f64(q[bs]), host_f64(k[bs]), host_f64(v[bs]), lens[bs], D ** -0.5)
    assert_close(host_f64(o[bs]), ro, BF16_TOL, "O")
    assert_lse_close(lse[bs].cpu().numpy(), rl, "LSE")
    del k, v, o
    torch.cuda.empty_cache()


def test_mla_decode_cache_past_2_31_elements():
    B, L, H = 64, 65536, 16  # latent cache: B * L * 576 > 2^31 elements
    say(f"case large MLA decode B={B} max_len={L} H={H} (cache: {B * L * 576} elements)")
    kv = _randn((B, L, 576), 51)
    q = _randn((B, H, 576), 52)
    lens = np.full(B, 5, np.int32)
    lens[B - 1], lens[0] = L, 1
    o, lse = fa.mla_decode(q, kv, dev(lens), dv=512, scale=576 ** -0.5, return_lse=True)
    torch.cuda.synchronize()
    bs = [0, B - 2, B - 1]
    ro, rl = oracle.mla_decode(host_f64(q[bs]), host_f64(kv[bs]), lens[bs], 512, 576 ** -0.5)
    assert_close(host_f64(o[bs]), ro, BF16_TOL, "O")
    assert_lse_close(lse[bs].cpu().numpy(), rl, "LSE")
    del kv, o
    torch.cuda.empty_cache()
