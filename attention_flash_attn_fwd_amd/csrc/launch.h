// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Keys per K/V tile of the decode kernels (the split sizes of the decode plans are multiples).
constexpr int kDecodeTileKeys = 32;
// Size of the static split-partials buffer of attn_decode_fwd_static (per GPU).
constexpr size_t kDecodeStaticScratchBytes = size_t(16) << 20;

struct PrefillArgs {
  const void* q;        // MHA: q; MLA: q_nope
  const void* k;        // MHA: k; MLA: k_nope
  const void* v;
  void* o;
  float* lse;           // nullable
  const void* q_rope;   // MLA only
  const void* k_rope;   // MLA only
  const float* q_scale; // MLA only, nullable (= 1)
  const float* k_scale; // MLA only, nullable (= 1)
  const float* v_scale; // MLA with e4m3 V only: one fp32 scale per V row
  const int32_t* cu_q;  // ragged batches only: query / key row offsets [B+1] of each sequence
  const int32_t* cu_k;
  int total_q, total_k; // ragged batches: rows of the packed q and k/v tensors
  int B, Sq, Skv, Hq, Hkv, Hr;  // ragged batches: Sq = the longest query sequence
  int causal;
  float scale;
};

struct DecodeArgs {
  const void* q;
  const void* k;        // GQA: k cache; MLA: latent cache
  const void* v;        // GQA: v cache; MLA: unused (V = first Dv columns of k)
  void* o;
  float* lse;
  const int32_t* kv_lens;
  const float* k_scale; // e4m3 caches: GQA [B, max_len, Hkv] per key row, MLA [B, max_len]; else NULL
  const float* v_scale; // e4m3 GQA cache: [B, max_len, Hkv]; else NULL
  float* part_o;        // workspace: [B, Hq, n_split, Dv] fp32 (GQA: Dv = D); MLA: int16 + exponents
  float* part_ml;       // workspace: [B, Hq, n_split, 2] fp32 (row max, row sum)
  int B, Hq, Hkv, max_len;
  int n_split, chunk;   // keys per split
  float scale;
};

struct MergeArgs {
  const void* o_a;      // [B, S, H, D] partial outputs over two disjoint key sets
  const float* lse_a;   // [B, H, S]
  const void* o_b;
  const float* lse_b;
  void* o;              // [B, S, H, D] merged output (may alias o_a or o_b)
  float* lse;           // [B, H, S] merged LSE, nullable (may alias lse_a or lse_b)
  int B, S, H, D;
  int log2_chunks;      // log2 of the 16-byte chunks per output row (0..6)
};

struct QuantArgs {
  const float* x;       // [n_rows, cols] fp32
  uint8_t* codes;       // [n_rows, cols] e4m3fn
  float* scale;         // [n_rows] fp32
  int n_rows, cols;
  int lanes_per_row;    // power of two, from quantize_lanes_per_row(cols)
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, int D, hipStream_t s);
// bf16 MHA / GQA prefill of head dim 128 without the causal mask: 64 query rows per wave, one
// wave per SIMD.
hipError_t launch_prefill_w64(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, int D, hipStream_t s);
hipError_t launch_prefill_varlen_bf16(const PrefillArgs& a, int D, hipStream_t s);
hipError_t launch_mla_prefill(const PrefillArgs& a, bool nope_fp8, bool v_fp8, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t s);
int quantize_lanes_per_row(int cols);
hipError_t launch_quantize_rows(const QuantArgs& a, hipStream_t s);

// Split plan of the decode kernels (host-only arithmetic, shared with the workspace query).
struct SplitPlan {
  int chunk;
  int n_split;
};
SplitPlan gqa_decode_plan(int B, int Hkv, int max_len);
SplitPlan mla_decode_plan(int B, int H, int max_len);
size_t decode_workspace_bytes(int B, int Hq, int Dv, int n_split);

hipError_t launch_gqa_decode(const DecodeArgs& a, int D, bool fp8, hipStream_t s);
// The GQA split kernels alone (gqa_decode.hip); launch_gqa_decode adds the combine.
hipError_t launch_gqa_split_kernels(const DecodeArgs& a, int D, bool fp8, hipStream_t s);
// The same with the partials in the library's static per-GPU buffer (a.part_o / a.part_ml are
// set here); the caller has checked that they fit in kDecodeStaticScratchBytes.
hipError_t launch_gqa_decode_static(DecodeArgs a, int D, bool fp8, hipStream_t s);
hipError_t launch_mla_decode(const DecodeArgs& a, bool fp8, hipStream_t s);

}  // namespace fa
