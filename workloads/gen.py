"""Seeded draws of the workload tensors.

Every tensor is i.i.d. N(0, 1) in fp32, drawn with numpy's PCG64 in independent
streams of ``CHUNK`` tokens: the stream for (tensor t, batch b, token chunk c)
is seeded with ``[workload.seed, t, b, c]``.  Any batch entry can therefore be
redrawn alone (the oracle at full sizes checks sampled sequences), and large
tensors are drawn on several host threads.  The fp32 draws are then stored as
the workload's dtype: fp32 as is, bf16 by round-to-nearest-even, e4m3 by the
per-row amax/448 quantiser of :mod:`workloads.encode`.

Decode lengths are drawn from the stream ``[seed, 1000]`` as integers uniform
on the closed range [len_lo, len_hi]; cache positions at or past a sequence's
length are zero and never read.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .encode import bf16_bits, quantize_rows_e4m3
from .shapes import Workload

CHUNK = 256

# tensor ids of the streams
T_Q, T_K, T_V, T_QNOPE, T_KNOPE, T_QROPE, T_KROPE, T_KV = 1, 2, 3, 4, 5, 6, 7, 8
T_LSE_A, T_LSE_B = 9, 10


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def normal_f32(seed: int, tid: int, b: int, c: int, shape) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64([seed, tid, b, c]))
    return rng.standard_normal(shape, dtype=np.float32)


def _fill(seed, tid, batches, ntok, rest, store, out_arrays, lens=None):
    """Draw tokens [0, lens[b] or ntok) of tensor tid for each b in batches.

    store(x32) returns a tuple of arrays matching out_arrays (one per output);
    out_arrays[k] has shape [len(batches), ntok, ...].
    """
    jobs = []
    for i, b in enumerate(batches):
        n_b = ntok if lens is None else int(lens[i])
        for c in range((n_b + CHUNK - 1) // CHUNK):
            t0 = c * CHUNK
            jobs.append((i, b, c, t0, min(CHUNK, n_b - t0)))

    def work(job):
        i, b, c, t0, n = job
        x = normal_f32(seed, tid, b, c, (n,) + tuple(rest))
        for arr, val in zip(out_arrays, store(x)):
            arr[i, t0:t0 + n] = val

    if len(jobs) > 4:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, jobs))
    else:
        for j in jobs:
            work(j)


def _store_fn(dtype: str):
    if dtype == "f32":
        return lambda x: (x,)
    if dtype == "bf16":
        return lambda x: (bf16_bits(x),)
    raise ValueError(dtype)


def _np_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _batches(w: Workload, batches):
    return list(range(w.B)) if batches is None else list(batches)


def make_prefill(w: Workload, batches=None) -> dict:
    """q [nb, Sq, Hq, D], k/v [nb, Skv, Hkv, D] in storage form (fp32 values or bf16 bits)."""
    bs = _batches(w, batches)
    nb, st, dt = len(bs), _store_fn(w.dtype), _np_dtype(w.dtype)
    q = np.zeros((nb, w.Sq, w.Hq, w.D), dt)
    k = np.zeros((nb, w.Skv, w.Hkv, w.D), dt)
    v = np.zeros((nb, w.Skv, w.Hkv, w.Dv), dt)
    _fill(w.seed, T_Q, bs, w.Sq, (w.Hq, w.D), st, [q])
    _fill(w.seed, T_K, bs, w.Skv, (w.Hkv, w.D), st, [k])
    _fill(w.seed, T_V, bs, w.Skv, (w.Hkv, w.Dv), st, [v])
    return {"q": q, "k": k, "v": v, "batches": bs}


def decode_lengths(w: Workload) -> np.ndarray:
    """Per-sequence KV lengths, int32 [B], uniform on [len_lo, len_hi]."""
    if w.len_lo == w.len_hi:
        return np.full(w.B, w.len_lo, np.int32)
    rng = np.random.Generator(np.random.PCG64([w.seed, 1000]))
    return rng.integers(w.len_lo, w.len_hi + 1, size=w.B).astype(np.int32)


def varlen_lengths(w: Workload) -> np.ndarray:
    """Ragged prefill: per-sequence token counts, int32 [B], uniform on [len_lo, len_hi] (the
    same stream as the decode lengths)."""
    return decode_lengths(w)


def make_prefill_varlen(w: Workload) -> dict:
    """Ragged prefill: packed q [T, Hq, D], k/v [T, Hkv, D] (bf16 bits) for the sequences of
    varlen_lengths(w) laid end to end (each sequence's keys are its own tokens), and the
    offsets cu [B+1]."""
    lens = varlen_lengths(w)
    T = int(lens.sum())
    d = make_prefill(w.with_(B=1, Sq=T, Skv=T))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return {"q": d["q"][0], "k": d["k"][0], "v": d["v"][0], "cu": cu, "lens": lens}


def make_merge(w: Workload) -> dict:
    """Two partial states: o_a, o_b [B, S, H, D] (bf16 bits or fp32) and lse_a, lse_b [B, H, S]
    fp32, all i.i.d. N(0, 1)."""
    d = make_prefill(w.with_(Skv=w.Sq, Hkv=w.Hq))
    la = np.zeros((w.B, w.Hq, w.Sq), np.float32)
    lb = np.zeros((w.B, w.Hq, w.Sq), np.float32)
    for b in range(w.B):
        la[b] = normal_f32(w.seed, T_LSE_A, b, 0, (w.Hq, w.Sq))
        lb[b] = normal_f32(w.seed, T_LSE_B, b, 0, (w.Hq, w.Sq))
    return {"o_a": d["q"], "o_b": d["k"], "lse_a": la, "lse_b": lb}


def make_decode(w: Workload, batches=None, lens=None) -> dict:
    """GQA decode: q [nb, Hq, D]; k/v caches [nb, Lmax, Hkv, D]; kv_lens int32 [nb].

    dtype "fp8": q in bf16; the caches as e4m3 codes with per-(token, kv head) fp32 scales
    k_scale, v_scale [nb, Lmax, Hkv] (amax/448 of each fp32 row, the same per-row recipe as
    the MLA prefill nope operands)."""
    if w.dtype == "fp8":
        return _make_decode_fp8(w, batches, lens)
    bs = _batches(w, batches)
    all_lens = decode_lengths(w) if lens is None else np.asarray(lens, np.int32)
    lens_b = np.array([all_lens[b] for b in bs], np.int32)
    nb, st, dt = len(bs), _store_fn(w.dtype), _np_dtype(w.dtype)
    q = np.zeros((nb, 1, w.Hq, w.D), dt)
    k = np.zeros((nb, w.Skv, w.Hkv, w.D), dt)
    v = np.zeros((nb, w.Skv, w.Hkv, w.Dv), dt)
    _fill(w.seed, T_Q, bs, 1, (w.Hq, w.D), st, [q])
    _fill(w.seed, T_K, bs, w.Skv, (w.Hkv, w.D), st, [k], lens=lens_b)
    _fill(w.seed, T_V, bs, w.Skv, (w.Hkv, w.Dv), st, [v], lens=lens_b)
    return {"q": q[:, 0], "k": k, "v": v, "kv_lens": lens_b, "batches": bs}


def _make_decode_fp8(w: Workload, batches, lens) -> dict:
    bs = _batches(w, batches)
    all_lens = decode_lengths(w) if lens is None else np.asarray(lens, np.int32)
    lens_b = np.array([all_lens[b] for b in bs], np.int32)
    nb = len(bs)
    q = np.zeros((nb, 1, w.Hq, w.D), np.uint16)
    k = np.zeros((nb, w.Skv, w.Hkv, w.D), np.uint8)
    v = np.zeros((nb, w.Skv, w.Hkv, w.Dv), np.uint8)
    ks = np.zeros((nb, w.Skv, w.Hkv), np.float32)
    vs = np.zeros((nb, w.Skv, w.Hkv), np.float32)
    _fill(w.seed, T_Q, bs, 1, (w.Hq, w.D), lambda x: (bf16_bits(x),), [q])
    _fill(w.seed, T_K, bs, w.Skv, (w.Hkv, w.D), quantize_rows_e4m3, [k, ks], lens=lens_b)
    _fill(w.seed, T_V, bs, w.Skv, (w.Hkv, w.Dv), quantize_rows_e4m3, [v, vs], lens=lens_b)
    return {"q": q[:, 0], "k": k, "v": v, "k_scale": ks, "v_scale": vs, "kv_lens": lens_b, "batches": bs}


def make_mla_decode(w: Workload, batches=None, lens=None) -> dict:
    """MLA decode: q [nb, H, Dk]; latent cache kv [nb, Lmax, Dk]; kv_lens int32 [nb].

    V is not a tensor of its own: it is kv[..., :Dv].  dtype "fp8": q in bf16; the cache as
    e4m3 codes with one fp32 scale per row, kv_scale [nb, Lmax] (amax/448 of the whole
    fp32 latent row, the per-row recipe of the other e4m3 operands).
    """
    bs = _batches(w, batches)
    all_lens = decode_lengths(w) if lens is None else np.asarray(lens, np.int32)
    lens_b = np.array([all_lens[b] for b in bs], np.int32)
    nb = len(bs)
    if w.dtype == "fp8":
        q = np.zeros((nb, 1, w.Hq, w.D), np.uint16)
        kv = np.zeros((nb, w.Skv, w.D), np.uint8)
        kvs = np.zeros((nb, w.Skv), np.float32)
        _fill(w.seed, T_Q, bs, 1, (w.Hq, w.D), lambda x: (bf16_bits(x),), [q])
        _fill(w.seed, T_KV, bs, w.Skv, (w.D,), quantize_rows_e4m3, [kv, kvs], lens=lens_b)
        return {"q": q[:, 0], "kv": kv, "kv_scale": kvs, "kv_lens": lens_b, "batches": bs}
    st, dt = _store_fn(w.dtype), _np_dtype(w.dtype)
    q = np.zeros((nb, 1, w.Hq, w.D), dt)
    kv = np.zeros((nb, w.Skv, w.D), dt)
    _fill(w.seed, T_Q, bs, 1, (w.Hq, w.D), st, [q])
    _fill(w.seed, T_KV, bs, w.Skv, (w.D,), st, [kv], lens=lens_b)
    return {"q": q[:, 0], "kv": kv, "kv_lens": lens_b, "batches": bs}


def make_mla_prefill(w: Workload, batches=None) -> dict:
    """MLA prefill with per-token scales.

    q_nope/k_nope: e4m3 codes [nb, S, H, Dn] with fp32 scales [nb, S, H] (amax/448 of the fp32
    originals); q_rope [nb, S, H, Dr], k_rope [nb, S, Hr, Dr], v [nb, S, H, Dv] as bf16 bits.
    dtype "fp8v": v as e4m3 codes with per-(token, head) fp32 scales v_scale [nb, S, H] (the same
    draws, quantised by the same recipe).
    """
    bs = _batches(w, batches)
    nb = len(bs)
    H, S, Dn, Dr, Dv, Hr = w.Hq, w.Sq, w.Dn, w.Dr, w.Dv, w.Hr
    qn = np.zeros((nb, S, H, Dn), np.uint8)
    kn = np.zeros((nb, w.Skv, H, Dn), np.uint8)
    qs = np.zeros((nb, S, H), np.float32)
    ks = np.zeros((nb, w.Skv, H), np.float32)
    qr = np.zeros((nb, S, H, Dr), np.uint16)
    kr = np.zeros((nb, w.Skv, Hr, Dr), np.uint16)
    v = np.zeros((nb, w.Skv, H, Dv), np.uint16)
    _fill(w.seed, T_QNOPE, bs, S, (H, Dn), quantize_rows_e4m3, [qn, qs])
    _fill(w.seed, T_KNOPE, bs, w.Skv, (H, Dn), quantize_rows_e4m3, [kn, ks])
    _fill(w.seed, T_QROPE, bs, S, (H, Dr), lambda x: (bf16_bits(x),), [qr])
    _fill(w.seed, T_KROPE, bs, w.Skv, (Hr, Dr), lambda x: (bf16_bits(x),), [kr])
    out = {"q_nope": qn, "k_nope": kn, "q_scale": qs, "k_scale": ks, "q_rope": qr, "k_rope": kr, "batches": bs}
    if w.dtype == "fp8v":
        vc = np.zeros((nb, w.Skv, H, Dv), np.uint8)
        vs = np.zeros((nb, w.Skv, H), np.float32)
        _fill(w.seed, T_V, bs, w.Skv, (H, Dv), quantize_rows_e4m3, [vc, vs])
        out.update(v=vc, v_scale=vs)
    else:
        _fill(w.seed, T_V, bs, w.Skv, (H, Dv), lambda x: (bf16_bits(x),), [v])
        out.update(v=v)
    return out


def make_quantize(w: Workload, batches=None, tokens=None) -> dict:
    """fp32 rows to quantise: the q_nope draws of the MLA prefill stream of the same seed,
    x [nb, S, H, Dn] (tokens [0, tokens) only when given)."""
    bs = _batches(w, batches)
    S = w.Sq if tokens is None else int(tokens)
    x = np.zeros((len(bs), S, w.Hq, w.Dn), np.float32)
    _fill(w.seed, T_QNOPE, bs, S, (w.Hq, w.Dn), lambda v: (v,), [x])
    return {"x": x, "batches": bs}
