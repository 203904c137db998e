"""Python binding of libattn.so, the gfx950 forward-attention library.

Argument marshalling only: every step of attention runs in the HIP kernels behind
the C ABI declared in include/attn.h.  PyTorch supplies device memory (outputs and
workspaces are allocated with torch) and the current HIP stream.  If libattn.so is
missing, every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F32, ATTN_BF16, ATTN_FP8_E4M3 = 0, 1, 2

EXPORTS = {
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_prefill_fwd": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int] * 8 +
                         [ctypes.c_float, ctypes.c_void_p]),
    "attn_prefill_varlen_fwd": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 9 +
                                [ctypes.c_float, ctypes.c_void_p]),
    "attn_merge_fwd": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int] * 5 + [ctypes.c_void_p]),
    "attn_decode_workspace_size": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "attn_decode_fwd": (ctypes.c_int, [ctypes.c_void_p] * 8 + [ctypes.c_int] * 6 +
                        [ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "attn_decode_fwd_static": (ctypes.c_int, [ctypes.c_void_p] * 8 + [ctypes.c_int] * 6 +
                               [ctypes.c_float, ctypes.c_void_p]),
    "mla_prefill_fwd": (ctypes.c_int, [ctypes.c_void_p] * 10 + [ctypes.c_int] * 11 +
                        [ctypes.c_float, ctypes.c_void_p]),
    "mla_decode_workspace_size": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "mla_decode_fwd": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int] * 6 +
                       [ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "quantize_rows_e4m3": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 2 + [ctypes.c_void_p]),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with attention_flash_attn_fwd_amd.build.build()")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(l, name)
            f.restype, f.argtypes = res, args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, status):
    if status != 0:
        raise AttnError(fn, status)


def _need(t: torch.Tensor, name: str, dtypes, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t, name: str, dtype, shape, device):
    """A caller-supplied output: the kernels write it whole, so it must match exactly."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    return t


def _workspace(t, need: int, device):
    """A caller-supplied workspace of at least `need` bytes; returns (tensor, its size in bytes)."""
    if t is None:
        t = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    elif not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return t, t.numel() * t.element_size()


_FP8 = (torch.uint8, torch.float8_e4m3fn)


def prefill(q, k, v, causal: bool = False, scale: float | None = None, out=None, return_lse: bool = False):
    """Flash-attention forward.  q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] (bf16 or fp32) -> o [B,Sq,Hq,D]."""
    dts = (torch.bfloat16, torch.float32)
    _need(q, "q", dts, 4); _need(k, "k", (q.dtype,), 4); _need(v, "v", (q.dtype,), 4)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _out(out, "out", q.dtype, q.shape, q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    dt = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_F32
    st = lib().attn_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), dt, B, Sq, Skv, Hq, Hkv, D,
                                int(bool(causal)), scale, _stream())
    _check("attn_prefill_fwd", st)
    return (o, lse) if return_lse else o


def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                   scale: float | None = None, out=None, return_lse: bool = False):
    """Ragged-batch prefill over packed sequences.  q [Tq,Hq,D], k/v [Tk,Hkv,D] bf16;
    cu_seqlens_q/k int32 [B+1] (device) -> o [Tq,Hq,D] (and lse [Hq,Tq])."""
    _need(q, "q", (torch.bfloat16,), 3); _need(k, "k", (torch.bfloat16,), 3); _need(v, "v", (torch.bfloat16,), 3)
    _need(cu_seqlens_q, "cu_seqlens_q", (torch.int32,), 1); _need(cu_seqlens_k, "cu_seqlens_k", (torch.int32,), 1)
    Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.shape[0] - 1
    if B < 0 or cu_seqlens_k.shape[0] != B + 1 or k.shape[2] != D or v.shape != k.shape:
        raise ValueError("shape mismatch")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _out(out, "out", q.dtype, q.shape, q.device)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib().attn_prefill_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                                       _ptr(cu_seqlens_k), ATTN_BF16, B, Tq, Tk, int(max_seqlen_q), Hq, Hkv, D,
                                       int(bool(causal)), scale, _stream())
    _check("attn_prefill_varlen_fwd", st)
    return (o, lse) if return_lse else o


def merge(o_a, lse_a, o_b, lse_b, out=None, out_lse=None, return_lse: bool = False):
    """Merge two partial attention results over disjoint key sets: o_* [B,S,H,D] (bf16 or fp32),
    lse_* [B,H,S] fp32 -> o [B,S,H,D] (and lse [B,H,S]).  out / out_lse may be o_a / lse_a."""
    dts = (torch.bfloat16, torch.float32)
    _need(o_a, "o_a", dts, 4); _need(o_b, "o_b", (o_a.dtype,), 4)
    _need(lse_a, "lse_a", (torch.float32,), 3); _need(lse_b, "lse_b", (torch.float32,), 3)
    B, S, H, D = o_a.shape
    if o_b.shape != o_a.shape or tuple(lse_a.shape) != (B, H, S) or lse_b.shape != lse_a.shape:
        raise ValueError("shape mismatch")
    o = torch.empty_like(o_a) if out is None else _out(out, "out", o_a.dtype, o_a.shape, o_a.device)
    lse = None if out_lse is None else _out(out_lse, "out_lse", torch.float32, lse_a.shape, o_a.device)
    if lse is None and return_lse:
        lse = torch.empty_like(lse_a)
    st = lib().attn_merge_fwd(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse),
                              ATTN_BF16 if o_a.dtype == torch.bfloat16 else ATTN_F32, B, S, H, D, _stream())
    _check("attn_merge_fwd", st)
    return (o, lse) if (return_lse or out_lse is not None) else o


def decode_workspace_size(B: int, Hq: int, Hkv: int, D: int, max_kv_len: int) -> int:
    return int(lib().attn_decode_workspace_size(B, Hq, Hkv, D, max_kv_len))


def _decode_operands(q, k_cache, v_cache, kv_lens, k_scale, v_scale):
    _need(q, "q", (torch.bfloat16,), 3); _need(kv_lens, "kv_lens", (torch.int32,), 1)
    fp8 = k_cache.dtype in _FP8
    if fp8:
        _need(k_cache, "k_cache", _FP8, 4); _need(v_cache, "v_cache", _FP8, 4)
        _need(k_scale, "k_scale", (torch.float32,), 3); _need(v_scale, "v_scale", (torch.float32,), 3)
        if k_scale.shape != k_cache.shape[:3] or v_scale.shape != k_cache.shape[:3]:
            raise ValueError("k_scale / v_scale must be [B, Lmax, Hkv]")
    else:
        _need(k_cache, "k_cache", (torch.bfloat16,), 4); _need(v_cache, "v_cache", (torch.bfloat16,), 4)
        if k_scale is not None or v_scale is not None:
            raise ValueError("k_scale / v_scale go with e4m3 caches only")
    B, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != D or v_cache.shape != k_cache.shape or kv_lens.shape[0] != B:
        raise ValueError("shape mismatch")
    return fp8, B, Hq, Hkv, D, Lmax


def decode(q, k_cache, v_cache, kv_lens, scale: float | None = None, workspace=None, out=None,
           return_lse: bool = False, k_scale=None, v_scale=None):
    """Decode: q [B,Hq,D] bf16, caches [B,Lmax,Hkv,D], kv_lens int32 [B] (device) -> o [B,Hq,D] bf16.

    Caches are bf16, or e4m3 codes (uint8 / float8_e4m3fn) with per-token fp32 scales
    k_scale, v_scale [B,Lmax,Hkv]."""
    fp8, B, Hq, Hkv, D, Lmax = _decode_operands(q, k_cache, v_cache, kv_lens, k_scale, v_scale)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    workspace, ws_bytes = _workspace(workspace, decode_workspace_size(B, Hq, Hkv, D, Lmax), q.device)
    o = torch.empty_like(q) if out is None else _out(out, "out", torch.bfloat16, q.shape, q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib().attn_decode_fwd(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _ptr(kv_lens),
                               _ptr(k_scale), _ptr(v_scale), ATTN_FP8_E4M3 if fp8 else ATTN_BF16,
                               B, Hq, Hkv, D, Lmax, scale, _ptr(workspace), ws_bytes, _stream())
    _check("attn_decode_fwd", st)
    return (o, lse) if return_lse else o


DECODE_STATIC_SCRATCH_BYTES = 16 << 20


def decode_static(q, k_cache, v_cache, kv_lens, scale: float | None = None, out=None, lse=None,
                  k_scale=None, v_scale=None):
    """decode() without a workspace: the split partials live in the library's static per-GPU
    buffer (attn_decode_fwd_static).  Pass `out` (and `lse`) to keep the call free of
    allocations; calls that overlap in time on one GPU race for the buffer."""
    fp8, B, Hq, Hkv, D, Lmax = _decode_operands(q, k_cache, v_cache, kv_lens, k_scale, v_scale)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _out(out, "out", torch.bfloat16, q.shape, q.device)
    if lse is not None:
        _out(lse, "lse", torch.float32, (B, Hq), q.device)
    st = lib().attn_decode_fwd_static(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _ptr(kv_lens),
                                      _ptr(k_scale), _ptr(v_scale), ATTN_FP8_E4M3 if fp8 else ATTN_BF16,
                                      B, Hq, Hkv, D, Lmax, scale, _stream())
    _check("attn_decode_fwd_static", st)
    return o


def mla_prefill(q_nope, q_rope, k_nope, k_rope, v, q_scale=None, k_scale=None, causal: bool = True,
                scale: float | None = None, out=None, return_lse: bool = False, v_scale=None):
    """MLA prefill.  q_nope/k_nope [B,S,H,128] e4m3 (uint8 codes or float8_e4m3fn) or bf16;
    q_rope [B,Sq,H,64], k_rope [B,Skv,Hr,64]; q_scale [B,Sq,H], k_scale [B,Skv,H] fp32;
    v [B,Skv,H,128] bf16, or e4m3 codes with v_scale [B,Skv,H] fp32 (V = code * v_scale)."""
    fp8 = q_nope.dtype in _FP8
    ndt = _FP8 if fp8 else (torch.bfloat16,)
    _need(q_nope, "q_nope", ndt, 4); _need(k_nope, "k_nope", ndt, 4)
    _need(q_rope, "q_rope", (torch.bfloat16,), 4); _need(k_rope, "k_rope", (torch.bfloat16,), 4)
    v_fp8 = v.dtype in _FP8
    _need(v, "v", _FP8 if v_fp8 else (torch.bfloat16,), 4)
    if v_fp8:
        _need(v_scale, "v_scale", (torch.float32,), 3)
        if tuple(v_scale.shape) != tuple(v.shape[:3]):
            raise ValueError("v_scale must be [B, Skv, H]")
    elif v_scale is not None:
        raise ValueError("v_scale goes with e4m3 V only")
    B, Sq, H, Dn = q_nope.shape
    Skv, Dr, Hr, Dv = k_nope.shape[1], q_rope.shape[3], k_rope.shape[2], v.shape[3]
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale")):
        if t is not None:
            _need(t, n, (torch.float32,), 3)
    if q_scale is not None and tuple(q_scale.shape) != (B, Sq, H):
        raise ValueError("q_scale shape")
    if k_scale is not None and tuple(k_scale.shape) != (B, Skv, H):
        raise ValueError("k_scale shape")
    if (tuple(k_nope.shape) != (B, Skv, H, Dn) or tuple(q_rope.shape[:3]) != (B, Sq, H)
            or tuple(k_rope.shape) != (B, Skv, Hr, Dr) or tuple(v.shape[:3]) != (B, Skv, H)):
        raise ValueError("shape mismatch")
    scale = 1.0 / math.sqrt(Dn + Dr) if scale is None else float(scale)
    o = (torch.empty((B, Sq, H, Dv), dtype=torch.bfloat16, device=v.device) if out is None
         else _out(out, "out", torch.bfloat16, (B, Sq, H, Dv), v.device))
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=v.device) if return_lse else None
    st = lib().mla_prefill_fwd(_ptr(q_nope), _ptr(q_rope), _ptr(k_nope), _ptr(k_rope), _ptr(v), _ptr(o),
                               _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(lse),
                               ATTN_FP8_E4M3 if fp8 else ATTN_BF16, ATTN_FP8_E4M3 if v_fp8 else ATTN_BF16,
                               B, Sq, Skv, H, Hr, Dn, Dr, Dv, int(bool(causal)), scale, _stream())
    _check("mla_prefill_fwd", st)
    return (o, lse) if return_lse else o


def mla_decode_workspace_size(B: int, H: int, Dv: int, max_kv_len: int) -> int:
    return int(lib().mla_decode_workspace_size(B, H, Dv, max_kv_len))


def mla_decode(q, kv_cache, kv_lens, dv: int = 512, scale: float | None = None, workspace=None, out=None,
               return_lse: bool = False, kv_scale=None):
    """MLA decode: q [B,H,Dk] bf16, latent cache [B,Lmax,Dk] (V = first dv columns) -> o [B,H,dv].

    The cache is bf16, or e4m3 codes (uint8 / float8_e4m3fn) with one fp32 scale per row,
    kv_scale [B,Lmax]."""
    _need(q, "q", (torch.bfloat16,), 3); _need(kv_lens, "kv_lens", (torch.int32,), 1)
    fp8 = kv_cache.dtype in _FP8
    if fp8:
        _need(kv_cache, "kv_cache", _FP8, 3); _need(kv_scale, "kv_scale", (torch.float32,), 2)
        if kv_scale.shape != kv_cache.shape[:2]:
            raise ValueError("kv_scale must be [B, Lmax]")
    else:
        _need(kv_cache, "kv_cache", (torch.bfloat16,), 3)
        if kv_scale is not None:
            raise ValueError("kv_scale goes with an e4m3 cache only")
    B, H, Dk = q.shape
    Lmax = kv_cache.shape[1]
    if kv_cache.shape[0] != B or kv_cache.shape[2] != Dk or kv_lens.shape[0] != B:
        raise ValueError("shape mismatch")
    scale = 1.0 / math.sqrt(Dk) if scale is None else float(scale)
    workspace, ws_bytes = _workspace(workspace, mla_decode_workspace_size(B, H, dv, Lmax), q.device)
    o = (torch.empty((B, H, dv), dtype=torch.bfloat16, device=q.device) if out is None
         else _out(out, "out", torch.bfloat16, (B, H, dv), q.device))
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib().mla_decode_fwd(_ptr(q), _ptr(kv_cache), _ptr(o), _ptr(lse), _ptr(kv_lens), _ptr(kv_scale),
                              ATTN_FP8_E4M3 if fp8 else ATTN_BF16, B, H, Dk, dv, Lmax,
                              scale, _ptr(workspace), ws_bytes, _stream())
    _check("mla_decode_fwd", st)
    return (o, lse) if return_lse else o


def quantize_rows_e4m3(x, codes=None, scale=None):
    """Per-row e4m3 quantisation of fp32 x [..., cols]: returns (codes uint8 [..., cols],
    scale fp32 [...]) with scale = amax/448 per row and codes = e4m3fn(x / scale)."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous fp32 device tensor")
    if x.dim() < 1:
        raise ValueError("x needs a last (row) axis")
    cols = x.shape[-1]
    n_rows = x.numel() // cols if cols else 0
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if codes is None else codes
    scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if scale is None else scale
    if codes.shape != x.shape or scale.shape != x.shape[:-1]:
        raise ValueError("codes / scale shape mismatch")
    if codes.dtype not in _FP8 or scale.dtype != torch.float32 or not codes.is_contiguous() or not scale.is_contiguous():
        raise TypeError("codes must be contiguous uint8 / float8_e4m3fn, scale contiguous fp32")
    if codes.device != x.device or scale.device != x.device:
        raise ValueError(f"codes / scale must be on {x.device}")
    st = lib().quantize_rows_e4m3(_ptr(x), _ptr(codes), _ptr(scale), n_rows, cols, _stream())
    _check("quantize_rows_e4m3", st)
    return codes, scale
