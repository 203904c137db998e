"""Pins of the ragged-prefill and state-merge oracle (CPU only), against things other than itself.

* brute force: pure-Python loops (math.exp / math.fsum) over tiny ragged batches,
  including empty sequences and query chunks shorter than their key ranges;
* a library routine: torch.nn.functional.scaled_dot_product_attention on the CPU in
  float64, one sequence at a time, with an explicit bottom-right causal mask;
* the split-key identity: attention over keys A u B equals the merge of the attention
  over A and over B -- checked against the unsplit oracle for arbitrary cuts and for the
  chunked-prefill case (cached prefix, non-causal, plus the chunk itself, causal);
* closed forms: an empty part leaves the other unchanged, equal LSEs average the outputs
  and add ln 2, two empty parts give 0 / -inf, LSEs of order 1e3 do not overflow.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.ragged as orag

RNG = np.random.default_rng(4321)


def rnd(*shape):
    return RNG.standard_normal(shape)


def brute_row(qrow, keys, vals, scale, nvis):
    xs = [scale * math.fsum(a * b for a, b in zip(qrow, keys[j])) for j in range(nvis)]
    if not xs:
        return [0.0] * len(vals[0]), -math.inf
    m = max(xs)
    w = [math.exp(x - m) for x in xs]
    s = math.fsum(w)
    return [math.fsum(w[j] * vals[j][d] for j in range(nvis)) / s for d in range(len(vals[0]))], m + math.log(s)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_brute_force(causal):
    lq = [3, 0, 1, 4]
    lk = [5, 2, 1, 4]        # sequence 0: a 3-row chunk after a 2-key prefix
    cu_q, cu_k = np.cumsum([0] + lq), np.cumsum([0] + lk)
    Hq, Hkv, D, Dv = 4, 2, 3, 2
    q, k, v = rnd(cu_q[-1], Hq, D), rnd(cu_k[-1], Hkv, D), rnd(cu_k[-1], Hkv, Dv)
    o, lse = oracle.prefill_varlen(q, k, v, cu_q, cu_k, 0.6, causal)
    for b in range(len(lq)):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            keys = k[cu_k[b]:cu_k[b + 1], kvh].tolist()
            vals = v[cu_k[b]:cu_k[b + 1], kvh].tolist() or [[0.0] * Dv]
            for i in range(lq[b]):
                nvis = min(lk[b], i + lk[b] - lq[b] + 1) if causal else lk[b]
                ob, lb = brute_row(q[cu_q[b] + i, h].tolist(), keys, vals, 0.6, max(nvis, 0))
                assert np.allclose(o[cu_q[b] + i, h], ob, atol=1e-12, rtol=0)
                assert lse[h, cu_q[b] + i] == lb or abs(lse[h, cu_q[b] + i] - lb) < 1e-12


def test_varlen_vs_torch_sdpa_per_sequence():
    lq = [70, 1, 33, 128]
    lk = [70, 9, 100, 128]
    cu_q, cu_k = np.cumsum([0] + lq), np.cumsum([0] + lk)
    Hq, Hkv, D = 6, 2, 16
    q, k, v = rnd(cu_q[-1], Hq, D), rnd(cu_k[-1], Hkv, D), rnd(cu_k[-1], Hkv, D)
    o, lse = oracle.prefill_varlen(q, k, v, cu_q, cu_k, 0.25, True)
    for b in range(len(lq)):
        qs = torch.from_numpy(q[cu_q[b]:cu_q[b + 1]]).permute(1, 0, 2)
        ks = torch.from_numpy(k[cu_k[b]:cu_k[b + 1]]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        vs = torch.from_numpy(v[cu_k[b]:cu_k[b + 1]]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        mask = torch.arange(lk[b])[None, :] <= (torch.arange(lq[b])[:, None] + lk[b] - lq[b])
        ref = F.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, scale=0.25).permute(1, 0, 2).numpy()
        assert np.abs(o[cu_q[b]:cu_q[b + 1]] - ref).max() < 1e-10
        x = 0.25 * torch.einsum("hid,hjd->hij", qs, ks).masked_fill(~mask, -math.inf)
        assert np.abs(lse[:, cu_q[b]:cu_q[b + 1]] - torch.logsumexp(x, -1).numpy()).max() < 1e-10


def test_varlen_rows_past_the_last_sequence_stay_empty():
    q, k, v = rnd(5, 2, 4), rnd(3, 2, 4), rnd(3, 2, 4)
    o, lse = oracle.prefill_varlen(q, k, v, np.array([0, 3]), np.array([0, 3]), 0.5, False)
    assert (o[3:] == 0).all() and np.isneginf(lse[:, 3:]).all()


@pytest.mark.parametrize("cut", [0, 1, 37, 63, 64])
def test_merge_identity_over_a_key_split(cut):
    """Attention over keys [0, 64) = merge(attention over [0, cut), over [cut, 64))."""
    B, S, H, D, L = 2, 9, 3, 8, 64
    q, k, v = rnd(B, S, H, D), rnd(B, L, H, D), rnd(B, L, H, D)
    full, lfull = oracle.prefill(q, k, v, 0.4, False)
    oa, la = oracle.prefill(q, k[:, :cut], v[:, :cut], 0.4, False)
    ob, lb = oracle.prefill(q, k[:, cut:], v[:, cut:], 0.4, False)
    o, lse = oracle.merge_states(oa, la, ob, lb)
    assert np.abs(o - full).max() < 1e-12
    assert np.abs(lse - lfull).max() < 1e-12
    o2, lse2 = oracle.merge_states(ob, lb, oa, la)   # symmetric
    assert np.abs(o2 - o).max() < 1e-14 and np.abs(lse2 - lse).max() < 1e-14


def test_merge_is_chunked_prefill():
    """A query chunk after a cached prefix: prefix (non-causal) merged with the chunk itself
    (causal) equals causal attention over the whole sequence, rows of the chunk."""
    P, C, H, D = 50, 20, 2, 8
    q, k, v = rnd(1, P + C, H, D), rnd(1, P + C, H, D), rnd(1, P + C, H, D)
    full, lfull = oracle.prefill(q, k, v, 0.3, True)
    oa, la = oracle.prefill(q[:, P:], k[:, :P], v[:, :P], 0.3, False)
    ob, lb = oracle.prefill(q[:, P:], k[:, P:], v[:, P:], 0.3, True)
    o, lse = oracle.merge_states(oa, la, ob, lb)
    assert np.abs(o - full[:, P:]).max() < 1e-12
    assert np.abs(lse - lfull[:, :, P:]).max() < 1e-12
    # the ragged path with Skv > Sq is the same computation in one call
    ov, lv = oracle.prefill_varlen(q[0, P:], k[0], v[0], np.array([0, C]), np.array([0, P + C]), 0.3, True)
    assert np.abs(ov - full[0, P:]).max() < 1e-12 and np.abs(lv - lfull[0, :, P:]).max() < 1e-12


def test_merge_closed_forms():
    B, S, H, D = 1, 4, 2, 3
    oa, ob = rnd(B, S, H, D), rnd(B, S, H, D)
    la = rnd(B, H, S)
    empty = np.full((B, H, S), -np.inf)
    o, lse = oracle.merge_states(oa, la, ob, empty)
    assert (o == oa).all() and (lse == la).all()
    o, lse = oracle.merge_states(oa, la, ob, la.copy())
    assert np.abs(o - 0.5 * (oa + ob)).max() < 1e-15 and np.abs(lse - (la + math.log(2))).max() < 1e-14
    o, lse = oracle.merge_states(oa, empty, ob, empty)
    assert (o == 0).all() and np.isneginf(lse).all()
    big = np.full((B, H, S), 1000.0)
    o, lse = oracle.merge_states(oa, big, ob, big - math.log(3))   # weights 3/4 and 1/4
    assert np.isfinite(o).all() and np.abs(o - (0.75 * oa + 0.25 * ob)).max() < 1e-13
    assert np.abs(lse - (1000.0 + math.log(4 / 3))).max() < 1e-12


def test_merge_mistakes_are_caught(monkeypatch):
    """Planted mistakes in the merge fail the pins above."""
    def swapped(o_a, lse_a, o_b, lse_b):
        m = np.maximum(lse_a, lse_b)
        wa, wb = np.exp(lse_a - m), np.exp(lse_b - m)
        t = lambda w: np.transpose(w / (wa + wb), (0, 2, 1))[..., None]
        return t(wb) * o_a + t(wa) * o_b, m + np.log(wa + wb)

    def unshifted(o_a, lse_a, o_b, lse_b):
        wa, wb = np.exp(lse_a), np.exp(lse_b)
        t = lambda w: np.transpose(w / (wa + wb), (0, 2, 1))[..., None]
        return t(wa) * o_a + t(wb) * o_b, np.log(wa + wb)

    for bad in (swapped, unshifted):
        monkeypatch.setattr(oracle, "merge_states", bad)
        caught = []
        for fn, args in ((test_merge_identity_over_a_key_split, (37,)), (test_merge_closed_forms, ())):
            try:
                with np.errstate(all="ignore"):
                    fn(*args)
                caught.append(False)
            except (AssertionError, FloatingPointError):
                caught.append(True)
        assert any(caught), bad.__name__


def test_varlen_off_by_one_offsets_are_caught(monkeypatch):
    monkeypatch.setattr(orag, "seq_bounds", lambda cu, b: (int(cu[b]) + (1 if b > 0 else 0), int(cu[b + 1])))
    with pytest.raises(AssertionError):
        test_varlen_vs_torch_sdpa_per_sequence()
