"""Seeded synthetic inputs for the forward-attention path.

This package is shared by the CPU oracle tests, the GPU parity tests and the
benchmark. It holds no attention arithmetic: only random draws, the storage
encodings of the inputs (bfloat16 round-to-nearest-even, OCP e4m3fn with a
per-row amax/448 scale -- the recipe of the MLA prefill inputs) and the shapes of
the workloads.  The oracle's quantiser (oracle/quantize.py) is written separately and
is what the GPU quantiser is checked against.
"""
from .encode import bf16_bits, bf16_bits_to_f32, e4m3_encode, quantize_rows_e4m3
from .shapes import WORKLOADS, Workload, workload
from .gen import (
    normal_f32,
    make_prefill,
    make_decode,
    make_mla_prefill,
    make_mla_decode,
    make_quantize,
    decode_lengths,
    varlen_lengths,
    make_prefill_varlen,
    make_merge,
)

__all__ = [
    "bf16_bits", "bf16_bits_to_f32", "e4m3_encode", "quantize_rows_e4m3",
    "WORKLOADS", "Workload", "workload",
    "normal_f32", "make_prefill", "make_decode", "make_mla_prefill", "make_mla_decode", "make_quantize",
    "decode_lengths", "varlen_lengths", "make_prefill_varlen", "make_merge",
]
