"""fp64 reference of ragged (variable-length) prefill and of merging partial attention states.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): nothing on the product path imports it.

Readings used here.  The pages pipeline K/V tiles through S = Q.K^T and O += P.V
("KVPipelineGeneric", sm100 MLA decode utilities: description and Parameters) and keep a
per-row correction for the running softmax ("MLASmemStorage": correction_smem); they print
no batching convention and no merge rule, so:

* ragged batch: sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 of a packed q [Tq, Hq, D]
  and key rows cu_k[b] .. cu_k[b+1]-1 of packed k, v [Tk, Hkv, D]; every sequence is an
  independent prefill with the bottom-right causal alignment of its own lengths (a query
  chunk that follows a cached prefix of Skv_b - Sq_b keys sees that whole prefix);
* merging two attention results over disjoint key sets A and B of the same query rows is
  the plain identity softmax over A u B = the LSE-weighted mix of the two softmaxes:
  O = (e^lse_a O_a + e^lse_b O_b) / (e^lse_a + e^lse_b), lse = ln(e^lse_a + e^lse_b),
  evaluated with the larger lse subtracted; two empty parts (both -inf) give O = 0,
  lse = -inf.

parity pins: tests/test_oracle_ragged.py (pure-Python brute force, torch CPU fp64 SDPA
per sequence, the split-key identity against the unsplit oracle, closed forms).
"""
from __future__ import annotations

import numpy as np

from .attention import prefill


def seq_bounds(cu: np.ndarray, b: int) -> tuple[int, int]:
    """Row range [start, end) of sequence b in a packed tensor with offsets cu [B+1]."""
    return int(cu[b]), int(cu[b + 1])


def prefill_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool):
    """Ragged prefill.  q [Tq, Hq, D], k [Tk, Hkv, D], v [Tk, Hkv, Dv] float64;
    cu_q, cu_k int [B+1] (non-decreasing, from 0).

    Returns O [Tq, Hq, Dv] and LSE [Hq, Tq]; rows past cu_q[B] stay O = 0, LSE = -inf.
    """
    Tq, Hq, _ = q.shape
    Dv = v.shape[2]
    o = np.zeros((Tq, Hq, Dv))
    lse = np.full((Hq, Tq), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1 = seq_bounds(cu_q, b)
        k0, k1 = seq_bounds(cu_k, b)
        if q1 == q0:
            continue
        ob, lb = prefill(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], scale, causal)
        o[q0:q1] = ob[0]
        lse[:, q0:q1] = lb[0]
    return o, lse


def merge_states(o_a, lse_a, o_b, lse_b):
    """Merge two partial attention results of the same query rows over disjoint key sets.

    o_a, o_b [B, S, H, D]; lse_a, lse_b [B, H, S] (natural log, -inf for an empty part).
    Returns O [B, S, H, D] and LSE [B, H, S] of the union of the two key sets.
    """
    la = np.asarray(lse_a, np.float64)
    lb = np.asarray(lse_b, np.float64)
    m = np.maximum(la, lb)
    empty = np.isneginf(m)
    shift = np.where(empty, 0.0, m)
    wa = np.exp(la - shift)              # exp(-inf) = 0 for an empty part
    wb = np.exp(lb - shift)
    den = wa + wb
    safe = np.where(empty, 1.0, den)
    # weights are per (b, h, s); o is laid out (b, s, h, d)
    ta = np.transpose(wa / safe, (0, 2, 1))[..., None]
    tb = np.transpose(wb / safe, (0, 2, 1))[..., None]
    o = np.where(np.transpose(empty, (0, 2, 1))[..., None], 0.0, ta * o_a + tb * o_b)
    lse = np.where(empty, -np.inf, shift + np.log(safe))
    return o, lse
