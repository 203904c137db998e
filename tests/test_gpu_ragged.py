"""GPU parity of the ragged-batch prefill (attn_prefill_varlen_fwd) and of the merge of partial
attention states (attn_merge_fwd) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as fa
import oracle
from tests.helpers import BF16_TOL, F32_TOL, assert_close, assert_lse_close, dev, dev_bf16, host_f64, say
from workloads import make_prefill, workload

pytestmark = pytest.mark.gpu


def _packed(Tq, Tk, Hq, Hkv, D):
    """Seeded bf16 q [Tq,Hq,D], k/v [Tk,Hkv,D] on the device (the prefill workload's draws)."""
    w = workload("mha_prefill_causal_bf16_b4_h32_s4096_d128", B=1, Sq=Tq, Skv=Tk, Hq=Hq, Hkv=Hkv, D=D, Dv=D)
    d = make_prefill(w)
    return dev_bf16(d["q"][0]), dev_bf16(d["k"][0]), dev_bf16(d["v"][0])


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


VARLEN_CASES = [
    # query lengths, key lengths, Hq, Hkv, D
    ([300, 1, 0, 129, 64], [300, 1, 5, 400, 64], 4, 2, 128),   # empty query sequence, chunk after prefix
    ([77, 200], [77, 50], 2, 1, 64),                           # Sq > Skv: leading rows see no key
    ([10, 33], [0, 33], 2, 2, 128),                            # a sequence with no key at all
    ([513, 1000, 7], [513, 1000, 7], 8, 2, 128),
    ([128, 0, 128, 0, 256], [128, 0, 128, 3, 256], 2, 2, 64),  # sequences of equal work (ties in the work order)
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lk,Hq,Hkv,D", VARLEN_CASES)
def test_varlen_vs_oracle(lq, lk, Hq, Hkv, D, causal):
    say(f"case varlen lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} D={D} causal={causal}")
    cq, ck = _cu(lq), _cu(lk)
    q, k, v = _packed(int(cq[-1]), int(ck[-1]), Hq, Hkv, D)
    o, lse = fa.prefill_varlen(q, k, v, dev(cq), dev(ck), max(lq), causal=causal, scale=D ** -0.5,
                               return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(host_f64(q), host_f64(k), host_f64(v), cq, ck, D ** -0.5, causal)
    assert_close(host_f64(o), ro, BF16_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


@pytest.mark.parametrize("n_seq", [200, 300])
def test_varlen_many_sequences(n_seq):
    """Many short sequences of random lengths (some empty, keys up to two past the queries):
    most (sequence, head) work items exit at once, the grid covering the longest."""
    rng = np.random.default_rng(n_seq)
    lq = rng.integers(0, 40, n_seq)
    lk = lq + rng.integers(0, 3, n_seq)
    say(f"case varlen n_seq={n_seq} total_q={lq.sum()} total_k={lk.sum()}")
    cq, ck = _cu(lq), _cu(lk)
    q, k, v = _packed(int(cq[-1]), int(ck[-1]), 2, 1, 64)
    o, lse = fa.prefill_varlen(q, k, v, dev(cq), dev(ck), int(lq.max()), causal=True, scale=0.125, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(host_f64(q), host_f64(k), host_f64(v), cq, ck, 0.125, True)
    assert_close(host_f64(o), ro, BF16_TOL, "O")
    assert_lse_close(lse.cpu().numpy(), rl, "LSE")


def test_varlen_equals_fixed_shape_prefill_bitwise():
    """Equal-length sequences: the ragged call computes exactly what the batched call does."""
    B, S, Hq, Hkv, D = 3, 333, 4, 2, 128
    q, k, v = _packed(B * S, B * S, Hq, Hkv, D)
    fixed, lf = fa.prefill(q.view(B, S, Hq, D), k.view(B, S, Hkv, D), v.view(B, S, Hkv, D), causal=True,
                           return_lse=True)
    cu = dev(_cu([S] * B))
    rag, lr = fa.prefill_varlen(q, k, v, cu, cu, S, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(fixed.view(B * S, Hq, D).view(torch.int16), rag.view(torch.int16))
    assert torch.equal(lf.permute(1, 0, 2).reshape(Hq, B * S), lr)


def test_varlen_leaves_rows_outside_the_sequences_untouched():
    q, k, v = _packed(200, 200, 2, 2, 128)
    o = torch.full_like(q, 7.0)
    cq = dev(np.array([0, 50, 120], np.int32))  # rows 120..199 belong to no sequence
    fa.prefill_varlen(q, k, v, cq, cq, 70, causal=True, out=o)
    torch.cuda.synchronize()
    assert (o[120:].float() == 7.0).all()
    ro, _ = oracle.prefill_varlen(host_f64(q), host_f64(k), host_f64(v), np.array([0, 50, 120]),
                                  np.array([0, 50, 120]), 128 ** -0.5, True)
    assert_close(host_f64(o[:120]), ro[:120], BF16_TOL, "O")


def test_varlen_full_size_sampled():
    """The ragged workload the bench times (8 sequences, lengths uniform on [512, 3584], 32 heads,
    D 128, causal), sampled rows checked against the oracle one sequence at a time."""
    from workloads import make_prefill_varlen
    w = workload("mha_prefill_varlen_causal_bf16_b8_len512to3584_h32_d128")
    d = make_prefill_varlen(w)
    lens, cu = d["lens"], d["cu"]
    say(f"case {w.name} lens={list(lens)}")
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    o, lse = fa.prefill_varlen(q, k, v, dev(cu), dev(cu), int(max(lens)), causal=True, scale=w.scale,
                               return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    got, ref, gl, rlse = [], [], [], []
    for b, h in [(0, 0), (3, 9), (len(lens) - 1, 31)]:
        s0, s1 = int(cu[b]), int(cu[b + 1])
        rows = np.unique(np.concatenate([[0, 1, s1 - s0 - 1], rng.integers(0, s1 - s0, 12)]))
        qs = host_f64(q[s0:s1, h:h + 1])[None]
        ks = host_f64(k[s0:s1, h:h + 1])[None]
        vs = host_f64(v[s0:s1, h:h + 1])[None]
        ro, rl = oracle.prefill_rows(qs, ks, vs, w.scale, True, 0, 0, rows)
        got.append(host_f64(o[s0 + rows, h]))
        ref.append(ro)
        gl.append(lse[h, s0 + rows].cpu().numpy())
        rlse.append(rl)
    assert_close(np.concatenate(got), np.concatenate(ref), BF16_TOL, "O sampled")
    assert_lse_close(np.concatenate(gl), np.concatenate(rlse), "LSE sampled")


@pytest.mark.parametrize("in_place", [False, True])
def test_chunked_prefill_by_merge(in_place):
    """A 300-row query chunk after a 1000-key cached prefix: prefill over the prefix
    (non-causal) merged with prefill over the chunk (causal) = causal attention over all."""
    P, C, H, D = 1000, 300, 4, 128
    say(f"case chunked prefill P={P} C={C} in_place={in_place}")
    q, k, v = _packed(P + C, P + C, H, H, D)
    q4, k4, v4 = q[None], k[None], v[None]
    qc = q4[:, P:].contiguous()
    oa, la = fa.prefill(qc, k4[:, :P].contiguous(), v4[:, :P].contiguous(), causal=False, return_lse=True)
    ob, lb = fa.prefill(qc, k4[:, P:].contiguous(), v4[:, P:].contiguous(), causal=True, return_lse=True)
    if in_place:
        o, lse = fa.merge(oa, la, ob, lb, out=oa, out_lse=la)
    else:
        o, lse = fa.merge(oa, la, ob, lb, return_lse=True)
    torch.cuda.synchronize()
    rows = np.arange(P, P + C)
    ro_all = np.stack([oracle.prefill_rows(host_f64(q4), host_f64(k4), host_f64(v4), D ** -0.5, True, 0, h, rows)[0]
                       for h in range(H)], axis=1)
    rl_all = np.stack([oracle.prefill_rows(host_f64(q4), host_f64(k4), host_f64(v4), D ** -0.5, True, 0, h, rows)[1]
                       for h in range(H)], axis=0)
    assert_close(host_f64(o[0]), ro_all, BF16_TOL, "O merged")
    assert_lse_close(lse[0].cpu().numpy(), rl_all, "LSE merged")
    # the ragged path does the same in one call
    ov = fa.prefill_varlen(qc[0], k, v, dev(_cu([C])), dev(_cu([P + C])), C, causal=True)
    torch.cuda.synchronize()
    assert_close(host_f64(ov), ro_all, BF16_TOL, "O ragged")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_vs_oracle_with_empty_parts(dtype):
    """Random partial states, some rows with one or both parts empty (lse = -inf).  Partial
    outputs are averages of value rows, so they are drawn at that scale (std 0.5); each bf16
    result must also be the exact merge rounded once (within half a bf16 ulp, 2^-8 relative)."""
    B, S, H, D = 2, 77, 3, 128 if dtype == "bf16" else 64
    rng = np.random.default_rng(5)
    oa32 = (0.5 * rng.standard_normal((B, S, H, D))).astype(np.float32)
    ob32 = (0.5 * rng.standard_normal((B, S, H, D))).astype(np.float32)
    la, lb = (rng.standard_normal((B, H, S)) * 3).astype(np.float32), (rng.standard_normal((B, H, S)) * 3).astype(np.float32)
    la[0, 0, :5] = -np.inf
    lb[0, 0, 3:8] = -np.inf          # rows 3, 4: both empty
    la[1, 2, 10] = 80.0              # large lse: no overflow
    if dtype == "bf16":
        ta, tb = torch.from_numpy(oa32).to(torch.bfloat16).cuda(), torch.from_numpy(ob32).to(torch.bfloat16).cuda()
        tol = BF16_TOL
    else:
        ta, tb = dev(oa32), dev(ob32)
        tol = F32_TOL
    o, lse = fa.merge(ta, dev(la), tb, dev(lb), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_states(host_f64(ta), la.astype(np.float64), host_f64(tb), lb.astype(np.float64))
    assert_close(host_f64(o), ro, tol, f"merge {dtype}")
    if dtype == "bf16":
        assert (np.abs(host_f64(o) - ro) <= 2.0 ** -8 * np.abs(ro) + 1e-6).all(), "not correctly rounded"
    assert_lse_close(lse.cpu().numpy(), rl, "merge LSE", tol=1e-5)
    assert (host_f64(o)[0, 3:5, 0] == 0).all()
