"""The C ABI without a GPU: libattn.so loads, exports every function include/attn.h
declares, and rejects invalid arguments with the documented status before any HIP
call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

import attention_flash_attn_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, EHIP, ESCALE, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first
NUL = None
S = ctypes.c_void_p(0)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    """libattn.so, or the library named by ATTN_ABI_TEST_LIB (the host-only sanitizer build of
    the same C ABI, see tests/test_abi_sanitized.py)."""
    path = os.environ.get("ATTN_ABI_TEST_LIB")
    if not path:
        return fa.lib()
    l = ctypes.CDLL(path)
    for name, (res, args) in fa.EXPORTS.items():
        f = getattr(l, name)
        f.restype, f.argtypes = res, args
    return l


def test_header_declares_the_four_entry_points():
    names = header_functions()
    for n in ("attn_prefill_fwd", "attn_decode_fwd", "mla_prefill_fwd", "mla_decode_fwd",
              "attn_decode_workspace_size", "mla_decode_workspace_size", "attn_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in header_functions():
        assert hasattr(lib, n), n
    assert set(header_functions()) == set(fa.EXPORTS)


def test_status_strings(lib):
    name = lambda code: lib.attn_status_string(code).decode()
    for code in (OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, EHIP, ESCALE, ESCRATCH):
        assert name(code) and name(code) != "unknown status"
    assert name(12345) == "unknown status"


def prefill(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=1, B=1, Sq=8, Skv=8, Hq=2, Hkv=1, D=128, causal=0, scale=0.1):
    return lib.attn_prefill_fwd(q, k, v, o, NUL, dtype, B, Sq, Skv, Hq, Hkv, D, causal, scale, S)


def test_prefill_validation(lib):
    assert prefill(lib, dtype=2) == EDTYPE
    assert prefill(lib, dtype=7) == EDTYPE
    assert prefill(lib, B=-1) == ESHAPE
    assert prefill(lib, Hq=3, Hkv=2) == ESHAPE
    assert prefill(lib, Hkv=0) == ESHAPE
    assert prefill(lib, Sq=-5) == ESHAPE
    assert prefill(lib, B=1 << 20, Sq=1 << 20, Hq=64, Hkv=64) == ESHAPE   # element count overflow
    assert prefill(lib, D=96) == EUNSUP
    assert prefill(lib, D=256) == EUNSUP
    assert prefill(lib, scale=0.0) == ESCALE
    assert prefill(lib, scale=float("nan")) == ESCALE
    assert prefill(lib, scale=float("inf")) == ESCALE
    assert prefill(lib, q=NUL) == ENULL
    assert prefill(lib, o=NUL) == ENULL
    assert prefill(lib, k=NUL) == ENULL
    # empty problems enqueue nothing and succeed, whatever the pointers
    assert prefill(lib, q=NUL, k=NUL, v=NUL, o=NUL, B=0) == OK
    assert prefill(lib, q=NUL, k=NUL, v=NUL, o=NUL, Sq=0) == OK


def decode(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lens=FAKE, ks=NUL, vs=NUL, dtype=1, B=4, Hq=32, Hkv=8, D=128, L=1024,
           scale=0.1, ws=FAKE, wsb=1 << 40):
    return lib.attn_decode_fwd(q, k, v, o, NUL, lens, ks, vs, dtype, B, Hq, Hkv, D, L, scale, ws, wsb, S)


def test_decode_validation(lib):
    need = lib.attn_decode_workspace_size(4, 32, 8, 128, 1024)
    assert need > 0
    assert lib.attn_decode_workspace_size(-1, 32, 8, 128, 1024) == 0
    assert lib.attn_decode_workspace_size(4, 32, 0, 128, 1024) == 0
    assert decode(lib, dtype=0) == EDTYPE
    assert decode(lib, Hq=30, Hkv=8) == ESHAPE
    assert decode(lib, L=-1) == ESHAPE
    assert decode(lib, D=96) == EUNSUP
    assert decode(lib, D=256) == EUNSUP
    assert decode(lib, Hq=64, Hkv=2) == EUNSUP       # 32 q heads per kv head > 16
    assert decode(lib, scale=-1.0) == ESCALE
    assert decode(lib, lens=NUL) == ENULL
    assert decode(lib, v=NUL) == ENULL
    assert decode(lib, ws=NUL) == EWS
    assert decode(lib, wsb=need - 1) == EWS
    assert decode(lib, B=0, q=NUL, o=NUL, lens=NUL, ws=NUL) == OK
    # head dim 64: the workspace of its own shape is enough, one byte less is not
    need64 = lib.attn_decode_workspace_size(4, 32, 8, 64, 1024)
    assert 0 < need64 < need
    assert decode(lib, D=64, wsb=need64 - 1) == EWS
    # e4m3 caches carry per-token scales; bf16 caches take none
    assert decode(lib, dtype=2, ks=NUL, vs=FAKE) == ENULL
    assert decode(lib, dtype=2, ks=FAKE, vs=NUL) == ENULL
    assert decode(lib, dtype=1, ks=FAKE, vs=FAKE) == EDTYPE
    assert decode(lib, dtype=2, ks=FAKE, vs=FAKE, D=96) == EUNSUP


def test_decode_split_plan_follows_the_kv_heads(lib):
    """One wave per (split, batch, kv head): fewer kv heads take more (shorter) splits, so the
    workspace (one partial row per (batch, q head, split)) grows as Hkv shrinks, and a long
    batch of many kv heads keeps its 1024-key splits."""
    row = 128 * 4 + 2 * 4           # fp32 partial O row + (m, l) per (batch, q head, split)
    ws = {hkv: lib.attn_decode_workspace_size(2, 16, hkv, 128, 65536) for hkv in (1, 2, 4, 8, 16)}
    assert ws[1] > ws[2] > ws[4] > ws[8] > ws[16]
    # B=64, Hkv=8, 8192 keys: 8 splits of 1024 keys give 4096 waves, no shortening needed
    big = lib.attn_decode_workspace_size(64, 32, 8, 128, 8192)
    assert abs(big - 64 * 32 * 8 * row) < 512


def decode_static(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lens=FAKE, ks=NUL, vs=NUL, dtype=1, B=4, Hq=32, Hkv=8, D=128,
                  L=1024, scale=0.1):
    return lib.attn_decode_fwd_static(q, k, v, o, NUL, lens, ks, vs, dtype, B, Hq, Hkv, D, L, scale, S)


def test_decode_static_validation(lib):
    """The entry point without a workspace validates like attn_decode_fwd and rejects, before any
    HIP call, partials larger than its static buffer (16 MiB)."""
    assert decode_static(lib, dtype=0) == EDTYPE
    assert decode_static(lib, Hq=30, Hkv=8) == ESHAPE
    assert decode_static(lib, D=96) == EUNSUP
    assert decode_static(lib, scale=0.0) == ESCALE
    assert decode_static(lib, lens=NUL) == ENULL
    assert decode_static(lib, dtype=2, ks=FAKE, vs=NUL) == ENULL
    assert decode_static(lib, B=0, q=NUL, o=NUL, lens=NUL) == OK
    limit = 16 << 20
    # B 64, 32/8 heads, D 128, 8192 keys: 8.5 MB of partials fit; 16384 keys (17 MB) do not
    assert lib.attn_decode_workspace_size(64, 32, 8, 128, 8192) <= limit
    assert lib.attn_decode_workspace_size(64, 32, 8, 128, 16384) > limit
    assert decode_static(lib, B=64, L=16384) == ESCRATCH
    assert decode_static(lib, B=512, Hq=64, Hkv=8, L=8192) == ESCRATCH


def mla_prefill(lib, qn=FAKE, qr=FAKE, kn=FAKE, kr=FAKE, v=FAKE, o=FAKE, vs=NUL, dt=2, vdt=1, B=1, Sq=64, Skv=64,
                H=4, Hr=1, Dn=128, Dr=64, Dv=128, causal=1, scale=0.07):
    return lib.mla_prefill_fwd(qn, qr, kn, kr, v, o, NUL, NUL, vs, NUL, dt, vdt, B, Sq, Skv, H, Hr, Dn, Dr, Dv,
                               causal, scale, S)


def test_mla_prefill_validation(lib):
    assert mla_prefill(lib, dt=0) == EDTYPE
    assert mla_prefill(lib, Hr=2) == ESHAPE
    assert mla_prefill(lib, H=-4) == ESHAPE
    assert mla_prefill(lib, Dn=64) == EUNSUP
    assert mla_prefill(lib, Dr=32) == EUNSUP
    assert mla_prefill(lib, Dv=64) == EUNSUP
    assert mla_prefill(lib, scale=0.0) == ESCALE
    assert mla_prefill(lib, qr=NUL) == ENULL
    assert mla_prefill(lib, kr=NUL) == ENULL
    assert mla_prefill(lib, B=0, qn=NUL, qr=NUL, kn=NUL, kr=NUL, v=NUL, o=NUL) == OK
    # e4m3 V carries one scale per row; bf16 V takes none
    assert mla_prefill(lib, vdt=0) == EDTYPE
    assert mla_prefill(lib, vdt=1, vs=FAKE) == EDTYPE
    assert mla_prefill(lib, vdt=2, vs=NUL) == ENULL
    assert mla_prefill(lib, vdt=2, vs=FAKE, Dv=64) == EUNSUP


def mla_decode(lib, q=FAKE, kv=FAKE, o=FAKE, lens=FAKE, ks=NUL, dtype=1, B=8, H=128, Dk=576, Dv=512, L=4096,
               scale=0.04, ws=FAKE, wsb=1 << 40):
    return lib.mla_decode_fwd(q, kv, o, NUL, lens, ks, dtype, B, H, Dk, Dv, L, scale, ws, wsb, S)


def test_mla_decode_validation(lib):
    need = lib.mla_decode_workspace_size(8, 128, 512, 4096)
    assert need >= 8 * 128 * 514 * 4
    assert mla_decode(lib, Dv=600) == ESHAPE
    assert mla_decode(lib, Dk=512) == EUNSUP
    assert mla_decode(lib, H=100) == EUNSUP
    assert mla_decode(lib, H=256) == EUNSUP
    assert mla_decode(lib, scale=float("nan")) == ESCALE
    assert mla_decode(lib, kv=NUL) == ENULL
    assert mla_decode(lib, wsb=need - 1) == EWS
    assert mla_decode(lib, B=0, q=NUL, kv=NUL, o=NUL, lens=NUL, ws=NUL) == OK
    # e4m3 latent caches carry one scale per row; bf16 caches take none
    assert mla_decode(lib, dtype=0) == EDTYPE
    assert mla_decode(lib, dtype=3, ks=FAKE) == EDTYPE
    assert mla_decode(lib, dtype=2, ks=NUL) == ENULL
    assert mla_decode(lib, dtype=1, ks=FAKE) == EDTYPE
    assert mla_decode(lib, dtype=2, ks=FAKE, Dk=512) == EUNSUP
    assert mla_decode(lib, dtype=2, ks=FAKE, wsb=need - 1) == EWS


def test_quantize_validation(lib):
    q = lambda x=FAKE, c=FAKE, s=FAKE, n=4, cols=128: lib.quantize_rows_e4m3(x, c, s, n, cols, S)
    assert q(n=-1) == ESHAPE
    assert q(cols=0) == ESHAPE
    assert q(cols=130) == EUNSUP       # not a multiple of 4
    assert q(cols=4100) == EUNSUP      # above 4096
    assert q(n=0) == OK                # empty: nothing to do, no HIP call
    assert q(x=NUL) == ENULL
    assert q(c=NUL) == ENULL
    assert q(s=NUL) == ENULL


def varlen(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, cq=FAKE, ck=FAKE, dtype=1, B=3, Tq=300, Tk=400, maxq=200, Hq=4,
           Hkv=2, D=128, causal=1, scale=0.1):
    return lib.attn_prefill_varlen_fwd(q, k, v, o, NUL, cq, ck, dtype, B, Tq, Tk, maxq, Hq, Hkv, D, causal, scale, S)


def test_prefill_varlen_validation(lib):
    assert varlen(lib, dtype=0) == EDTYPE           # ragged batches are bf16 only
    assert varlen(lib, dtype=2) == EDTYPE
    assert varlen(lib, B=-1) == ESHAPE
    assert varlen(lib, Tq=-1) == ESHAPE
    assert varlen(lib, maxq=-1) == ESHAPE
    assert varlen(lib, Hq=3) == ESHAPE
    assert varlen(lib, D=96) == EUNSUP
    assert varlen(lib, scale=0.0) == ESCALE
    assert varlen(lib, cq=NUL) == ENULL
    assert varlen(lib, ck=NUL) == ENULL
    assert varlen(lib, k=NUL) == ENULL
    assert varlen(lib, q=NUL) == ENULL
    assert varlen(lib, q=NUL, k=NUL, v=NUL, o=NUL, cq=NUL, ck=NUL, B=0) == OK
    assert varlen(lib, q=NUL, k=NUL, v=NUL, o=NUL, cq=NUL, ck=NUL, Tq=0) == OK
    assert varlen(lib, q=NUL, k=NUL, v=NUL, o=NUL, cq=NUL, ck=NUL, maxq=0) == OK


def merge(lib, oa=FAKE, la=FAKE, ob=FAKE, lb=FAKE, o=FAKE, dtype=1, B=2, S_=16, H=4, D=128):
    return lib.attn_merge_fwd(oa, la, ob, lb, o, NUL, dtype, B, S_, H, D, S)


def test_merge_validation(lib):
    assert merge(lib, dtype=2) == EDTYPE
    assert merge(lib, B=-1) == ESHAPE
    assert merge(lib, H=0) == ESHAPE
    assert merge(lib, D=100) == EUNSUP            # 200 bytes: not whole 16-byte chunks
    assert merge(lib, D=96) == EUNSUP             # 12 chunks: not a power of two
    assert merge(lib, D=1024) == EUNSUP           # 128 chunks per row
    assert merge(lib, dtype=0, D=512) == EUNSUP   # fp32: 128 chunks per row
    assert merge(lib, oa=NUL) == ENULL
    assert merge(lib, lb=NUL) == ENULL
    assert merge(lib, o=NUL) == ENULL
    assert merge(lib, oa=NUL, la=NUL, ob=NUL, lb=NUL, o=NUL, S_=0) == OK
