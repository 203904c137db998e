"""The synthetic workloads of the forward-attention path, by name.

Each one is a shape, a storage dtype and a seed; the tensors are drawn by
:mod:`workloads.gen`.  Layouts are token-major and row-major throughout:
q/o ``[B, S, H, D]``, k/v ``[B, S, Hkv, D]``, decode caches ``[B, Lmax, Hkv, D]``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "prefill_varlen" | "merge" | "decode" | "mla_prefill" | "mla_decode" | "quantize"
    seed: int
    dtype: str                # storage dtype of q/k/v: "f32" | "bf16" | "fp8+bf16" | "fp8v" (MLA nope and V) | "fp8" (decode cache)
    B: int
    Hq: int
    Hkv: int
    Sq: int = 1
    Skv: int = 1
    D: int = 128              # q/k head dim (MHA/GQA), Dk for MLA decode
    Dv: int = 128
    causal: bool = False
    Dn: int = 0               # MLA prefill nope depth
    Dr: int = 0               # MLA prefill rope depth
    Hr: int = 1               # MLA prefill k_rope heads (1 = shared by every head)
    len_lo: int = 0           # decode (KV) and ragged prefill: per-sequence lengths uniform on [len_lo, len_hi]
    len_hi: int = 0
    scale: float = 0.0
    notes: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # MHA forward, non-causal, fp32: batch 1, 4 heads, seq 128, head_dim 64.
    "mha_fp32_b1_h4_s128_d64": Workload(
        name="mha_fp32_b1_h4_s128_d64", kind="prefill", seed=1, dtype="f32",
        B=1, Hq=4, Hkv=4, Sq=128, Skv=128, D=64, Dv=64, causal=False, scale=1.0 / 64 ** 0.5),
    # MHA prefill, causal, bf16: batch 4, 32 heads, seq 4096, head_dim 128.
    "mha_prefill_causal_bf16_b4_h32_s4096_d128": Workload(
        name="mha_prefill_causal_bf16_b4_h32_s4096_d128", kind="prefill", seed=2, dtype="bf16",
        B=4, Hq=32, Hkv=32, Sq=4096, Skv=4096, D=128, Dv=128, causal=True, scale=1.0 / 128 ** 0.5),
    # GQA decode, bf16 contiguous cache: batch 64, 32 q heads over 8 kv heads, max length 8192,
    # per-sequence lengths uniform on [1024, 8192].
    "gqa_decode_bf16_b64_hq32_hkv8_d128_l8192": Workload(
        name="gqa_decode_bf16_b64_hq32_hkv8_d128_l8192", kind="decode", seed=3, dtype="bf16",
        B=64, Hq=32, Hkv=8, Skv=8192, D=128, Dv=128, len_lo=1024, len_hi=8192,
        scale=1.0 / 128 ** 0.5),
    # The same GQA decode over an e4m3 cache with per-(token, kv head) fp32 scales.
    "gqa_decode_fp8_b64_hq32_hkv8_d128_l8192": Workload(
        name="gqa_decode_fp8_b64_hq32_hkv8_d128_l8192", kind="decode", seed=3, dtype="fp8",
        B=64, Hq=32, Hkv=8, Skv=8192, D=128, Dv=128, len_lo=1024, len_hi=8192,
        scale=1.0 / 128 ** 0.5),
    # MLA decode: batch 64, 128 q heads over one latent head, K = [latent 512 | rope 64],
    # V = K[..., :512], length 4096 for every sequence.
    "mla_decode_bf16_b64_h128_dk576_dv512_l4096": Workload(
        name="mla_decode_bf16_b64_h128_dk576_dv512_l4096", kind="mla_decode", seed=4, dtype="bf16",
        B=64, Hq=128, Hkv=1, Skv=4096, D=576, Dv=512, len_lo=4096, len_hi=4096,
        scale=1.0 / 576 ** 0.5),
    # The same MLA decode over an e4m3 latent cache with one fp32 scale per cache row (token).
    "mla_decode_fp8_b64_h128_dk576_dv512_l4096": Workload(
        name="mla_decode_fp8_b64_h128_dk576_dv512_l4096", kind="mla_decode", seed=4, dtype="fp8",
        B=64, Hq=128, Hkv=1, Skv=4096, D=576, Dv=512, len_lo=4096, len_hi=4096,
        scale=1.0 / 576 ** 0.5),
    # MLA prefill, causal, per-token scales: batch 1, 128 heads, seq 8192; nope 128 in e4m3 with
    # per-(token, head) fp32 scales, rope 64 in bf16 (one shared k_rope head), V 128 in bf16.
    "mla_prefill_fp8_causal_b1_h128_s8192": Workload(
        name="mla_prefill_fp8_causal_b1_h128_s8192", kind="mla_prefill", seed=5, dtype="fp8+bf16",
        B=1, Hq=128, Hkv=128, Sq=8192, Skv=8192, D=192, Dv=128, causal=True, Dn=128, Dr=64, Hr=1,
        scale=1.0 / 192 ** 0.5),
    # The same MLA prefill with V also in e4m3 (per-(token, head) fp32 value scales), as the
    # per-token-scale MLA page types V like Q and K_nope.
    "mla_prefill_fp8v_causal_b1_h128_s8192": Workload(
        name="mla_prefill_fp8v_causal_b1_h128_s8192", kind="mla_prefill", seed=5, dtype="fp8v",
        B=1, Hq=128, Hkv=128, Sq=8192, Skv=8192, D=192, Dv=128, causal=True, Dn=128, Dr=64, Hr=1,
        scale=1.0 / 192 ** 0.5),
    # Ragged-batch causal prefill: 8 packed sequences with lengths uniform on [512, 3584]
    # (16384 tokens on average, the token count of the B4 S4096 prefill), 32 heads, D 128, bf16.
    "mha_prefill_varlen_causal_bf16_b8_len512to3584_h32_d128": Workload(
        name="mha_prefill_varlen_causal_bf16_b8_len512to3584_h32_d128", kind="prefill_varlen", seed=6,
        dtype="bf16", B=8, Hq=32, Hkv=32, D=128, Dv=128, causal=True, len_lo=512, len_hi=3584,
        scale=1.0 / 128 ** 0.5),
    # Merge of two partial attention results of the B4 S4096 H32 D128 prefill's shape (bf16 outputs,
    # fp32 LSEs), e.g. a cached-prefix part and a chunk part.
    "merge_bf16_b4_s4096_h32_d128": Workload(
        name="merge_bf16_b4_s4096_h32_d128", kind="merge", seed=7, dtype="bf16",
        B=4, Hq=32, Hkv=32, Sq=4096, Skv=4096, D=128, Dv=128),
    # Per-token e4m3 quantisation of the MLA prefill q_nope originals: 8192 tokens x 128 heads
    # rows of 128 fp32 values (the same draws the MLA prefill workload quantises).
    "quantize_e4m3_rows_b1_s8192_h128_d128": Workload(
        name="quantize_e4m3_rows_b1_s8192_h128_d128", kind="quantize", seed=5, dtype="f32",
        B=1, Hq=128, Hkv=128, Sq=8192, Skv=8192, D=128, Dv=128, Dn=128),
}

# The headline workload of the benchmark.
BENCH_DEFAULT = "mha_prefill_causal_bf16_b4_h32_s4096_d128"
# Every workload the benchmark times by default, in order: the five workloads of the path,
# then those of the next rows (e4m3 caches, e4m3 V, ragged prefill, merge, quantiser).
BENCH_ORDER = [
    "mha_prefill_causal_bf16_b4_h32_s4096_d128",
    "mha_fp32_b1_h4_s128_d64",
    "gqa_decode_bf16_b64_hq32_hkv8_d128_l8192",
    "mla_decode_bf16_b64_h128_dk576_dv512_l4096",
    "mla_prefill_fp8_causal_b1_h128_s8192",
    "gqa_decode_fp8_b64_hq32_hkv8_d128_l8192",
    "mla_decode_fp8_b64_h128_dk576_dv512_l4096",
    "mla_prefill_fp8v_causal_b1_h128_s8192",
    "mha_prefill_varlen_causal_bf16_b8_len512to3584_h32_d128",
    "merge_bf16_b4_s4096_h32_d128",
    "quantize_e4m3_rows_b1_s8192_h128_d128",
]


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally resized (e.g. ``workload(n, B=1, Sq=300, Skv=300)``)."""
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w
