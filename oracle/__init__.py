"""CPU fp64 oracle of the forward-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP path.

What it computes is the plain definition of scaled-dot-product attention,
materialised in full for every query row: logits x = scale * q.k (or the MLA
logit with per-token scales), masked keys at -inf, P = softmax over keys, and
O = P.V, with LSE = log sum exp of the row.  The pages (Modular's Mojo kernel
docs: "KVPipelineGeneric", "MLASmemStorage", AMD attention "buffers") name the
two contractions S = Q.K^T and O += P.V, a per-row correction buffer (the
online-softmax rescale) and the nope/rope + q_scale/k_scale split of MLA; they
never print the softmax, so the textbook definition stands in for it.  The
oracle never blocks over keys (that would be the online algorithm it checks).

It also holds the per-token e4m3 quantiser (oracle/quantize.py) that produces the
MLA prefill nope operands and their fp32 scales, and (oracle/ragged.py) ragged-batch
prefill over packed sequences and the merge of two partial attention results by
their LSE.

parity pins: see tests/test_oracle_*.py (brute force, torch CPU fp64 SDPA,
closed forms, invariants, the OCP e4m3 code table, torch float8 casts).
"""
from .codecs import bf16_to_f64, e4m3_to_f64, E4M3_TABLE
from .quantize import e4m3_round, quantize_rows, row_scale
from .attention import (
    sdpa_rows,
    prefill,
    prefill_rows,
    decode,
    mla_prefill,
    mla_prefill_rows,
    mla_decode,
)
from .ragged import merge_states, prefill_varlen

__all__ = [
    "bf16_to_f64", "e4m3_to_f64", "E4M3_TABLE", "e4m3_round", "quantize_rows", "row_scale",
    "sdpa_rows", "prefill", "prefill_rows", "decode", "mla_prefill", "mla_prefill_rows", "mla_decode",
    "prefill_varlen", "merge_states",
]
