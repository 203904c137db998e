"""Pins of the fp64 attention oracle against things other than itself (CPU only).

* brute force: pure-Python loops with math.exp / math.fsum on tiny inputs;
* a library routine: torch.nn.functional.scaled_dot_product_attention on the CPU
  in float64 (GQA by repeating kv heads; MLA prefill as SDPA over the
  concatenated dequantised [nope*scale | rope] operands; MLA decode as SDPA
  with V = the first Dv latent columns);
* closed forms: zero queries give (prefix) means of V, two keys give a
  sigmoid mix, one visible key returns its V row, an empty row gives 0 / -inf;
* invariants: identical V rows, logit shifts (identical k_rope rows), per-token
  scale algebra, the bottom-right causal suffix, the split-KV merge identity.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(1234)


def rnd(*shape, s=1.0):
    return RNG.standard_normal(shape) * s


# ----------------------------------------------------------------- brute force

def brute_row(qrow, keys, vals, scale, nvis):
    xs = [scale * math.fsum(a * b for a, b in zip(qrow, keys[j])) for j in range(nvis)]
    if not xs:
        return [0.0] * len(vals[0]), -math.inf
    m = max(xs)
    w = [math.exp(x - m) for x in xs]
    s = math.fsum(w)
    o = [math.fsum(w[j] * vals[j][d] for j in range(nvis)) / s for d in range(len(vals[0]))]
    return o, m + math.log(s)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,Dv", [(2, 5, 5, 2, 1, 4, 3), (1, 3, 6, 4, 2, 3, 2), (1, 1, 4, 2, 2, 2, 2)])
def test_prefill_brute_force(causal, B, Sq, Skv, Hq, Hkv, D, Dv):
    q, k, v = rnd(B, Sq, Hq, D), rnd(B, Skv, Hkv, D), rnd(B, Skv, Hkv, Dv)
    scale = 0.7
    o, lse = oracle.prefill(q, k, v, scale, causal)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            for i in range(Sq):
                nvis = min(Skv, i + (Skv - Sq) + 1) if causal else Skv
                ob, lb = brute_row(q[b, i, h].tolist(), k[b, :, kvh].tolist(), v[b, :, kvh].tolist(), scale, nvis)
                assert np.allclose(o[b, i, h], ob, atol=1e-12, rtol=0)
                assert abs(lse[b, h, i] - lb) < 1e-12


def test_decode_brute_force():
    B, L, Hq, Hkv, D = 3, 7, 4, 2, 3
    q, kc, vc = rnd(B, Hq, D), rnd(B, L, Hkv, D), rnd(B, L, Hkv, D)
    lens = np.array([7, 1, 4])
    o, lse = oracle.decode(q, kc, vc, lens, 0.5)
    for b in range(B):
        for h in range(Hq):
            kvh = h // 2
            ob, lb = brute_row(q[b, h].tolist(), kc[b, :, kvh].tolist(), vc[b, :, kvh].tolist(), 0.5, lens[b])
            assert np.allclose(o[b, h], ob, atol=1e-12, rtol=0) and abs(lse[b, h] - lb) < 1e-12


def test_mla_prefill_brute_force():
    B, S, H, Dn, Dr, Dv = 1, 4, 2, 3, 2, 2
    qn, kn, qr, kr, v = rnd(B, S, H, Dn), rnd(B, S, H, Dn), rnd(B, S, H, Dr), rnd(B, S, 1, Dr), rnd(B, S, H, Dv)
    qs, ks = np.abs(rnd(B, S, H)) + 0.1, np.abs(rnd(B, S, H)) + 0.1
    o, lse = oracle.mla_prefill(qn, qr, kn, kr, v, qs, ks, 0.3, True)
    for h in range(H):
        for i in range(S):
            xs = [0.3 * (math.fsum(a * b for a, b in zip(qn[0, i, h], kn[0, j, h])) * qs[0, i, h] * ks[0, j, h]
                         + math.fsum(a * b for a, b in zip(qr[0, i, h], kr[0, j, 0]))) for j in range(i + 1)]
            m = max(xs)
            w = [math.exp(x - m) for x in xs]
            s = math.fsum(w)
            ob = [math.fsum(w[j] * v[0, j, h, d] for j in range(i + 1)) / s for d in range(Dv)]
            assert np.allclose(o[0, i, h], ob, atol=1e-12, rtol=0)
            assert abs(lse[0, h, i] - (m + math.log(s))) < 1e-12


def test_mla_decode_brute_force():
    B, L, H, Dk, Dv = 2, 5, 3, 4, 3
    q, kv = rnd(B, H, Dk), rnd(B, L, Dk)
    lens = np.array([5, 2])
    o, lse = oracle.mla_decode(q, kv, lens, Dv, 0.4)
    for b in range(B):
        for h in range(H):
            keys = kv[b].tolist()
            ob, lb = brute_row(q[b, h].tolist(), keys, [r[:Dv] for r in keys], 0.4, lens[b])
            assert np.allclose(o[b, h], ob, atol=1e-12, rtol=0) and abs(lse[b, h] - lb) < 1e-12


# ----------------------------------------------------------------- torch SDPA (fp64, CPU)

def sdpa_ref(q, k, v, scale, causal=False, mask=None):
    """q [B,Sq,Hq,D], k/v [B,Skv,Hkv,*] -> [B,Sq,Hq,Dv] via torch SDPA (kv heads repeated)."""
    g = q.shape[2] // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, is_causal=causal, scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1)])
def test_prefill_vs_torch_sdpa(causal, Hq, Hkv):
    B, S, D = 2, 97, 32
    q, k, v = rnd(B, S, Hq, D), rnd(B, S, Hkv, D), rnd(B, S, Hkv, D)
    o, lse = oracle.prefill(q, k, v, 1 / math.sqrt(D), causal)
    ref = sdpa_ref(q, k, v, 1 / math.sqrt(D), causal)
    assert np.abs(o - ref).max() < 1e-12
    # LSE against torch.logsumexp of the explicitly scaled logits
    g = Hq // Hkv
    for b, h in [(0, 0), (1, Hq - 1)]:
        x = torch.from_numpy(q[b, :, h] @ k[b, :, h // g].T / math.sqrt(D))
        if causal:
            x = x.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), -math.inf)
        assert np.abs(lse[b, h] - torch.logsumexp(x, dim=1).numpy()).max() < 1e-12


def test_prefill_large_logits_no_overflow():
    B, S, H, D = 1, 64, 2, 16
    q, k, v = rnd(B, S, H, D, s=30.0), rnd(B, S, H, D, s=30.0), rnd(B, S, H, D)
    o, lse = oracle.prefill(q, k, v, 1.0, False)   # logits of order 1e3..1e4
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert np.abs(o - sdpa_ref(q, k, v, 1.0)).max() < 1e-10


def test_decode_vs_torch_sdpa_with_lengths():
    B, L, Hq, Hkv, D = 4, 50, 8, 2, 16
    q, kc, vc = rnd(B, Hq, D), rnd(B, L, Hkv, D), rnd(B, L, Hkv, D)
    lens = np.array([50, 1, 17, 33])
    o, _ = oracle.decode(q, kc, vc, lens, 0.25)
    mask = torch.from_numpy(np.arange(L)[None, :] < lens[:, None])[:, None, None, :]  # [B,1,1,L]
    ref = sdpa_ref(q[:, None], kc, vc, 0.25, mask=mask)[:, 0]
    assert np.abs(o - ref).max() < 1e-12


def test_mla_prefill_vs_torch_sdpa_concat():
    """MLA logits = SDPA over q^ = [qn*qs | qr], k^ = [kn*ks | kr broadcast]."""
    B, S, H, Dn, Dr, Dv = 1, 80, 4, 16, 8, 12
    qn, kn, qr, kr, v = rnd(B, S, H, Dn), rnd(B, S, H, Dn), rnd(B, S, H, Dr), rnd(B, S, 1, Dr), rnd(B, S, H, Dv)
    qs, ks = np.abs(rnd(B, S, H)) + 0.05, np.abs(rnd(B, S, H)) + 0.05
    scale = 1 / math.sqrt(Dn + Dr)
    for causal in (False, True):
        o, _ = oracle.mla_prefill(qn, qr, kn, kr, v, qs, ks, scale, causal)
        qh = np.concatenate([qn * qs[..., None], qr], -1)
        kh = np.concatenate([kn * ks[..., None], np.broadcast_to(kr, (B, S, H, Dr))], -1)
        ref = sdpa_ref(qh, kh, v, scale, causal)
        assert np.abs(o - ref).max() < 1e-12


def test_mla_prefill_per_head_rope():
    B, S, H, Dn, Dr, Dv = 1, 20, 3, 8, 4, 5
    qn, kn, qr, kr, v = rnd(B, S, H, Dn), rnd(B, S, H, Dn), rnd(B, S, H, Dr), rnd(B, S, H, Dr), rnd(B, S, H, Dv)
    qs, ks = np.ones((B, S, H)), np.ones((B, S, H))
    o, _ = oracle.mla_prefill(qn, qr, kn, kr, v, qs, ks, 0.5, True)
    ref = sdpa_ref(np.concatenate([qn, qr], -1), np.concatenate([kn, kr], -1), v, 0.5, True)
    assert np.abs(o - ref).max() < 1e-12


def test_mla_decode_vs_torch_sdpa():
    B, L, H, Dk, Dv = 3, 40, 8, 24, 16
    q, kv = rnd(B, H, Dk), rnd(B, L, Dk)
    lens = np.array([40, 13, 1])
    o, _ = oracle.mla_decode(q, kv, lens, Dv, 1 / math.sqrt(Dk))
    mask = torch.from_numpy(np.arange(L)[None, :] < lens[:, None])[:, None, None, :]
    ref = sdpa_ref(q[:, None], kv[:, :, None, :], kv[:, :, None, :Dv], 1 / math.sqrt(Dk), mask=mask)[:, 0]
    assert np.abs(o - ref).max() < 1e-12


# ----------------------------------------------------------------- closed forms

def test_zero_query_gives_prefix_means():
    B, S, H, D = 1, 33, 2, 8
    q, k, v = np.zeros((B, S, H, D)), rnd(B, S, H, D), rnd(B, S, H, D)
    o, lse = oracle.prefill(q, k, v, 0.3, True)
    pref = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert np.abs(o - pref).max() < 1e-13
    assert np.abs(lse[0, 0] - np.log(np.arange(1, S + 1))).max() < 1e-13
    o, _ = oracle.prefill(q, k, v, 0.3, False)
    assert np.abs(o - v.mean(axis=1, keepdims=True)).max() < 1e-13


def test_zero_query_decode_gives_mean_of_visible():
    B, L, H, D = 3, 20, 2, 4
    q, kc, vc = np.zeros((B, H, D)), rnd(B, L, H, D), rnd(B, L, H, D)
    lens = np.array([20, 5, 1])
    o, _ = oracle.decode(q, kc, vc, lens, 1.0)
    for b in range(B):
        assert np.abs(o[b] - vc[b, :lens[b]].mean(axis=0)).max() < 1e-13


def test_first_causal_row_and_single_key():
    B, S, H, D = 2, 9, 3, 5
    q, k, v = rnd(B, S, H, D), rnd(B, S, H, D), rnd(B, S, H, D)
    o, lse = oracle.prefill(q, k, v, 0.5, True)
    assert np.abs(o[:, 0] - v[:, 0]).max() < 1e-15
    # logit of the single visible key is its LSE
    assert np.abs(lse[:, :, 0] - 0.5 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])).max() < 1e-13
    od, _ = oracle.decode(q[:, 0], k, v, np.array([1, 1]), 0.5)
    assert np.abs(od - v[:, 0]).max() < 1e-15


def test_two_keys_sigmoid():
    q = rnd(1, 1, 1, 6)
    k, v = rnd(1, 2, 1, 6), rnd(1, 2, 1, 4)
    o, lse = oracle.prefill(q, k, v, 0.8, False)
    x0, x1 = 0.8 * q[0, 0, 0] @ k[0, 0, 0], 0.8 * q[0, 0, 0] @ k[0, 1, 0]
    s0 = 1 / (1 + math.exp(x1 - x0))
    assert np.abs(o[0, 0, 0] - (s0 * v[0, 0, 0] + (1 - s0) * v[0, 1, 0])).max() < 1e-14
    assert abs(lse[0, 0, 0] - (max(x0, x1) + math.log1p(math.exp(-abs(x0 - x1))))) < 1e-13


def test_empty_rows():
    q, kc, vc = rnd(2, 2, 4), rnd(2, 8, 1, 4), rnd(2, 8, 1, 4)
    o, lse = oracle.decode(q, kc, vc, np.array([0, 3]), 1.0)
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(o[1]).all()


# ----------------------------------------------------------------- invariants

def test_identical_v_rows_return_that_row():
    B, S, H, D = 1, 40, 2, 8
    row = rnd(D)
    q, k = rnd(B, S, H, D, s=3.0), rnd(B, S, H, D, s=3.0)
    v = np.broadcast_to(row, (B, S, H, D)).copy()
    for causal in (False, True):
        o, _ = oracle.prefill(q, k, v, 1.0, causal)
        assert np.abs(o - row).max() < 1e-13


def test_causal_bottom_right_suffix():
    """Sq < Skv: the queries are the last Sq positions of a square causal problem."""
    B, Skv, H, D, Sq = 1, 30, 2, 8, 7
    qf, k, v = rnd(B, Skv, H, D), rnd(B, Skv, H, D), rnd(B, Skv, H, D)
    full, lfull = oracle.prefill(qf, k, v, 0.4, True)
    part, lpart = oracle.prefill(qf[:, -Sq:], k, v, 0.4, True)
    assert np.abs(part - full[:, -Sq:]).max() < 1e-14
    assert np.abs(lpart - lfull[:, :, -Sq:]).max() < 1e-13
    # ... and one query token (Sq = 1) sees every key, as decode does
    d, _ = oracle.decode(qf[:, -1], k, v, np.array([Skv]), 0.4)
    assert np.abs(d - full[:, -1]).max() < 1e-14


def test_identical_k_rope_rows_shift_logits_only():
    """Identical k_rope rows add a per-query constant to every logit: O equals nope-only attention."""
    B, S, H, Dn, Dr, Dv = 1, 30, 2, 8, 4, 6
    qn, kn, qr, v = rnd(B, S, H, Dn), rnd(B, S, H, Dn), rnd(B, S, H, Dr, s=5.0), rnd(B, S, H, Dv)
    kr = np.broadcast_to(rnd(Dr), (B, S, 1, Dr)).copy()
    qs, ks = np.abs(rnd(B, S, H)) + 0.1, np.abs(rnd(B, S, H)) + 0.1
    a, _ = oracle.mla_prefill(qn, qr, kn, kr, v, qs, ks, 0.5, True)
    b, _ = oracle.mla_prefill(qn, qr, kn, np.zeros_like(kr), v, qs, ks, 0.5, True)
    assert np.abs(a - b).max() < 1e-13


def test_per_token_scale_algebra():
    B, S, H, Dn, Dr, Dv = 1, 25, 2, 8, 4, 6
    qn, kn, qr, kr, v = rnd(B, S, H, Dn), rnd(B, S, H, Dn), rnd(B, S, H, Dr), rnd(B, S, 1, Dr), rnd(B, S, H, Dv)
    qs, ks = np.abs(rnd(B, S, H)) + 0.1, np.abs(rnd(B, S, H)) + 0.1
    base, _ = oracle.mla_prefill(qn, qr, kn, kr, v, qs, ks, 0.5, False)
    # k_scale == c everywhere is the same as scaling k_nope by c with unit k_scale
    c = 1.7
    a, _ = oracle.mla_prefill(qn, qr, kn, kr, v, qs, np.full_like(ks, c), 0.5, False)
    b, _ = oracle.mla_prefill(qn, qr, kn * c, kr, v, qs, np.ones_like(ks), 0.5, False)
    assert np.abs(a - b).max() < 1e-13
    # q_scale = 0 on a row removes the nope term of that row
    qs0 = qs.copy()
    qs0[0, 5, 1] = 0.0
    z, _ = oracle.mla_prefill(qn, qr, kn, kr, v, qs0, ks, 0.5, False)
    r, _ = oracle.mla_prefill(np.zeros_like(qn), qr, kn, kr, v, qs, ks, 0.5, False)
    assert np.abs(z[0, 5, 1] - r[0, 5, 1]).max() < 1e-13
    assert np.abs(z[0, 4] - base[0, 4]).max() == 0.0


def test_split_kv_merge_identity():
    """Partials (m = LSE of a key range, O of that range) merge exactly to the unsplit result."""
    B, L, H, D = 2, 100, 4, 16
    q, kc, vc = rnd(B, H, D), rnd(B, L, H, D), rnd(B, L, H, D)
    full, lfull = oracle.decode(q, kc, vc, np.array([L, L]), 0.3)
    cuts = [0, 13, 40, 41, 100]
    parts = []
    for a, b_ in zip(cuts[:-1], cuts[1:]):
        o, lse = oracle.decode(q, kc[:, a:b_], vc[:, a:b_], np.array([b_ - a] * B), 0.3)
        parts.append((o, lse))
    M = np.max([p[1] for p in parts], axis=0)
    w = [np.exp(p[1] - M) for p in parts]
    merged = sum(wi[..., None] * p[0] for wi, p in zip(w, parts)) / sum(w)[..., None]
    assert np.abs(merged - full).max() < 1e-12
    assert np.abs(M + np.log(sum(w)) - lfull).max() < 1e-12


def test_prefill_rows_match_full():
    B, S, Hq, Hkv, D = 2, 70, 4, 2, 8
    q, k, v = rnd(B, S, Hq, D), rnd(B, S, Hkv, D), rnd(B, S, Hkv, D)
    o, lse = oracle.prefill(q, k, v, 0.3, True)
    rows = np.array([0, 5, 69])
    ob, lb = oracle.prefill_rows(q, k, v, 0.3, True, 1, 3, rows)
    assert (ob == o[1, rows, 3]).all() and (lb == lse[1, 3, rows]).all()
