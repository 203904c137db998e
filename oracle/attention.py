"""fp64 reference attention (plain definition, materialised per query-row block).

Readings of the pages used here (they print no formula; the KVPipelineGeneric
page names the contractions S = Q.K^T and O += P.V over K/V tiles, the
MLASmemStorage page names the nope/rope parts of Q and K, the per-row
q_scale / per-key k_scale buffers and a per-row correction buffer):

* logits x[i, j] = scale * sum_d q[i, d] * k[j, d]; for MLA prefill
  x[i, j] = scale * ((q_nope[i] . k_nope[j]) * q_scale[i] * k_scale[j] + q_rope[i] . k_rope[j]).
* causal masking is aligned bottom-right: query i of Sq sees keys j <= i + (Skv - Sq).
* decode: the one query token sees keys [0, L_b) of its sequence.
* GQA: query head h reads kv head h // (Hq // Hkv).
* MLA decode: V is the first Dv columns of the latent cache row.
* P = softmax over visible keys; O = P . V; LSE = ln sum_j exp(x[i, j]) (natural log).
* a row with no visible key has O = 0 and LSE = -inf.

All arithmetic is float64 on the exact decoded input values.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 1024


def sdpa_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray | None,
              logits: np.ndarray | None = None, scale: float = 1.0):
    """Attention of a block of query rows against all keys of one head.

    q [M, D], k [N, D], v [N, Dv]; visible [M, N] bool (None = all visible).
    If ``logits`` [M, N] is given it is used as the already-scaled x and q/k are ignored.
    Returns O [M, Dv] and LSE [M] (float64).
    """
    if logits is None:
        x = scale * (q @ k.T)
    else:
        x = np.array(logits, dtype=np.float64, copy=True)
    if visible is not None:
        x = np.where(visible, x, -np.inf)
    row_max = x.max(axis=1, keepdims=True) if x.shape[1] else np.full((x.shape[0], 1), -np.inf)
    empty = ~np.isfinite(row_max)
    shift = np.where(empty, 0.0, row_max)
    e = np.exp(x - shift)                       # exp(-inf) = 0 for masked keys
    denom = e.sum(axis=1, keepdims=True)
    safe = np.where(denom > 0, denom, 1.0)
    p = np.where(denom > 0, e / safe, 0.0)
    o = p @ v
    lse = np.where(denom[:, 0] > 0, shift[:, 0] + np.log(safe[:, 0]), -np.inf)
    return o, lse


def causal_visible(rows: np.ndarray, Sq: int, Skv: int) -> np.ndarray:
    """Bottom-right causal mask: visible[i, j] = j <= rows[i] + (Skv - Sq)."""
    return np.arange(Skv)[None, :] <= (rows[:, None] + (Skv - Sq))


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """GQA grouping: consecutive groups of Hq // Hkv query heads share one kv head."""
    return h // (Hq // Hkv)


def mla_logits(qn, kn, qr, kr, qs, ks, scale: float) -> np.ndarray:
    """MLA prefill logits of a row block: scale * ((qn . kn^T) * qs[i] * ks[j] + qr . kr^T).

    The per-token scales multiply only the nope product (the MLASmemStorage page keeps
    q_scale per Q-tile row and k_scale per K-tile row next to the nope/rope operands).
    """
    nope = (qn @ kn.T) * qs[:, None] * ks[None, :]
    return scale * (nope + qr @ kr.T)


def mla_value(kv: np.ndarray, Dv: int) -> np.ndarray:
    """MLA decode: the value row of a latent cache row is its first Dv columns."""
    return kv[..., :Dv]


def prefill_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows: np.ndarray):
    """O [len(rows), Dv], LSE [len(rows)] for query rows ``rows`` of (batch b, q head h).

    q [B, Sq, Hq, D], k [B, Skv, Hkv, D], v [B, Skv, Hkv, Dv] float64.
    """
    Sq, Hq = q.shape[1], q.shape[2]
    Skv, Hkv = k.shape[1], k.shape[2]
    kvh = kv_head(h, Hq, Hkv)
    rows = np.asarray(rows)
    vis = causal_visible(rows, Sq, Skv) if causal else None
    return sdpa_rows(q[b, rows, h, :], k[b, :, kvh, :], v[b, :, kvh, :], vis, scale=scale)


def prefill(q, k, v, scale: float, causal: bool):
    """Full prefill: O [B, Sq, Hq, Dv], LSE [B, Hq, Sq]."""
    B, Sq, Hq, _ = q.shape
    Dv = v.shape[3]
    o = np.zeros((B, Sq, Hq, Dv))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, Sq, ROW_BLOCK):
                rows = np.arange(r0, min(Sq, r0 + ROW_BLOCK))
                ob, lb = prefill_rows(q, k, v, scale, causal, b, h, rows)
                o[b, rows, h, :] = ob
                lse[b, h, rows] = lb
    return o, lse


def decode(q, k_cache, v_cache, kv_lens, scale: float):
    """One query token per sequence: q [B, Hq, D]; caches [B, Lmax, Hkv, D]; kv_lens [B].

    Returns O [B, Hq, Dv], LSE [B, Hq].
    """
    B, Hq, _ = q.shape
    Hkv = k_cache.shape[2]
    Dv = v_cache.shape[3]
    o = np.zeros((B, Hq, Dv))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(min(max(int(kv_lens[b]), 0), k_cache.shape[1]))
        for h in range(Hq):
            kvh = kv_head(h, Hq, Hkv)
            ob, lb = sdpa_rows(q[b, h][None, :], k_cache[b, :L, kvh, :], v_cache[b, :L, kvh, :], None,
                               scale=scale)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def mla_prefill_rows(q_nope, q_rope, k_nope, k_rope, v, q_scale, k_scale, scale: float, causal: bool,
                     b: int, h: int, rows: np.ndarray):
    """MLA prefill rows of (b, h): logits scale*((qn.kn)*qs*ks + qr.kr), then softmax.V.

    q_nope [B,Sq,H,Dn], k_nope [B,Skv,H,Dn], q_rope [B,Sq,H,Dr], k_rope [B,Skv,Hr,Dr] (Hr = 1
    is shared by every head), v [B,Skv,H,Dv], q_scale [B,Sq,H], k_scale [B,Skv,H]; float64.
    """
    Sq, Skv = q_nope.shape[1], k_nope.shape[1]
    hr = 0 if k_rope.shape[2] == 1 else h
    rows = np.asarray(rows)
    x = mla_logits(q_nope[b, rows, h, :], k_nope[b, :, h, :], q_rope[b, rows, h, :], k_rope[b, :, hr, :],
                   q_scale[b, rows, h], k_scale[b, :, h], scale)
    vis = causal_visible(rows, Sq, Skv) if causal else None
    return sdpa_rows(None, None, v[b, :, h, :], vis, logits=x)


def mla_prefill(q_nope, q_rope, k_nope, k_rope, v, q_scale, k_scale, scale: float, causal: bool):
    """Full MLA prefill: O [B, Sq, H, Dv], LSE [B, H, Sq]."""
    B, Sq, H, _ = q_nope.shape
    Dv = v.shape[3]
    o = np.zeros((B, Sq, H, Dv))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, ROW_BLOCK):
                rows = np.arange(r0, min(Sq, r0 + ROW_BLOCK))
                ob, lb = mla_prefill_rows(q_nope, q_rope, k_nope, k_rope, v, q_scale, k_scale, scale,
                                          causal, b, h, rows)
                o[b, rows, h, :] = ob
                lse[b, h, rows] = lb
    return o, lse


def mla_decode(q, kv, kv_lens, Dv: int, scale: float, heads=None):
    """MLA decode: q [B, H, Dk], latent cache kv [B, Lmax, Dk]; V = kv[..., :Dv].

    Returns O [B, H, Dv], LSE [B, H] (rows of ``heads`` only, if given; others stay 0).
    """
    B, H, _ = q.shape
    o = np.zeros((B, H, Dv))
    lse = np.zeros((B, H))
    hs = np.arange(H) if heads is None else np.asarray(heads)
    for b in range(B):
        L = int(min(max(int(kv_lens[b]), 0), kv.shape[1]))
        keys = kv[b, :L, :]
        ob, lb = sdpa_rows(q[b, hs, :], keys, mla_value(keys, Dv), None, scale=scale)
        o[b, hs], lse[b, hs] = ob, lb
    return o, lse
