/*
 * attn.h -- C ABI of the MI355X (gfx950) forward-attention library (libattn.so).
 *
 * What is computed.  Scaled-dot-product attention, forward only:
 *     x[i,j] = scale * q_i . k_j          (MLA prefill: see mla_prefill_fwd)
 *     P[i,:] = softmax over the keys j visible to query i
 *     O[i,:] = sum_j P[i,j] v_j,   LSE[i] = ln sum_j exp(x[i,j])
 * evaluated as tiled flash attention: S = Q.K^T on a K tile, an online softmax with a
 * running row max and sum whose per-row correction rescales the O accumulator, then
 * O += P.V on the matching V tile.  Modular's Mojo kernel pages describe this path:
 * "KVPipelineGeneric" (NVIDIA sm100, MLA decode utilities; description and Parameters:
 * the S = Q.K' and O += P.V products pipelined over K/V tiles), "MLASmemStorage" (sm100
 * per-token-scale MLA prefill; description, Parameters and Fields: Q and K split into
 * nope and rope parts, a q_scale per Q-tile row and a k_scale per K-tile row, a per-row
 * correction buffer) and the AMD attention "buffers" module (K/V tile buffers with a
 * token_gen (decode) variant, Q/P/O operands held in registers).
 *
 * Conventions shared by every entry point.
 *  - Every tensor pointer is a DEVICE pointer owned by the caller; the library never
 *    allocates, frees or retains memory and keeps no state between calls.
 *  - Layouts are row-major and contiguous, token-major: q/o [B, Sq, Hq, D],
 *    k/v [B, Skv, Hkv, D], decode caches [B, max_kv_len, Hkv, D].
 *  - Query head h reads kv head h / (Hq / Hkv) (consecutive GQA groups).
 *  - Causal masking is aligned bottom-right: query i sees key j iff j <= i + (Skv - Sq).
 *    A query row that sees no key gets O = 0 and LSE = -inf.
 *  - softmax_scale multiplies the logits; it must be finite and > 0.
 *  - lse (nullable) receives fp32 natural-log LSE, [B, Hq, Sq] (prefill) or [B, Hq] (decode).
 *  - Every call enqueues its kernels on `stream` (0 = the null stream) and returns
 *    before they finish; there is no host synchronisation inside the library.
 *  - Errors: arguments are validated on the host BEFORE any HIP call, and a non-OK
 *    status is returned with nothing enqueued.  A failed launch returns ATTN_ERR_HIP.
 *    Device faults surface at the caller's next synchronisation.
 *  - Concurrent calls are safe; calls that run concurrently need distinct workspaces.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F32 = 0,       /* IEEE binary32 */
  ATTN_BF16 = 1,      /* bfloat16 */
  ATTN_FP8_E4M3 = 2   /* OCP 8-bit e4m3fn: bias 7, max 448, no infinities */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,         /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,        /* a size is negative, or Hq % Hkv != 0, or sizes overflow */
  ATTN_ERR_DTYPE = -3,        /* dtype not accepted by this entry point */
  ATTN_ERR_UNSUPPORTED = -4,  /* head dims / options outside the compiled set */
  ATTN_ERR_WORKSPACE = -5,    /* workspace NULL or smaller than *_workspace_size() */
  ATTN_ERR_HIP = -6,          /* a HIP launch failed */
  ATTN_ERR_SCALE = -7,        /* softmax_scale not finite and positive */
  ATTN_ERR_SCRATCH = -8       /* attn_decode_fwd_static: partials larger than its static buffer */
} attn_status_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char* attn_status_string(int status);

/*
 * Prefill / MHA / GQA forward (KVPipelineGeneric page: S = Q.K' then O += P.V over
 * pipelined K/V tiles; AMD buffers page: Q held in registers, K/V tiles staged in LDS).
 *   q [B,Sq,Hq,D], k [B,Skv,Hkv,D], v [B,Skv,Hkv,D], o [B,Sq,Hq,D]: all `dtype`
 *   (ATTN_BF16 or ATTN_F32); bf16 output is rounded to nearest even.
 *   lse: NULL or fp32 [B,Hq,Sq].
 *   Supported: D in {64, 128}; Hq % Hkv == 0; any Sq, Skv >= 0 (0 sizes enqueue nothing
 *   except, for Skv == 0, the zero output).
 */
int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int dtype, int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal,
                     float softmax_scale, hipStream_t stream);

/*
 * Ragged-batch prefill over packed sequences (KVPipelineGeneric page: S = Q.K' then
 * O += P.V over pipelined K/V tiles, here per sequence).  Sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and key rows cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1 of k and v; each is an independent attention with its own causal
 * alignment (bottom-right: a query chunk of Sq_b rows after a cached prefix sees keys
 * j <= i + (Skv_b - Sq_b), so chunked prefill over a contiguous prefix is one call).
 *   q, o [total_q, Hq, D]; k, v [total_k, Hkv, D]: bf16 (dtype must be ATTN_BF16).
 *   cu_seqlens_q, cu_seqlens_k: DEVICE int32 [B+1], non-decreasing from 0, last entry
 *   <= total_q (resp. total_k); every query length <= max_seqlen_q.  The kernel clamps
 *   the offsets into [0, total], so inconsistent arrays give unspecified values but no
 *   access outside the tensors; rows of o outside every sequence are not written.
 *   lse: NULL or fp32 [Hq, total_q].
 *   Supported: D in {64, 128}; Hq % Hkv == 0.
 */
int attn_prefill_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype, int B,
                            int total_q, int total_k, int max_seqlen_q, int Hq, int Hkv, int D, int causal,
                            float softmax_scale, hipStream_t stream);

/*
 * Merge of two partial attention results of the same query rows over disjoint key sets
 * (the per-row correction of the running softmax, MLASmemStorage page correction_smem,
 * applied to two finished parts):
 *   M = max(lse_a, lse_b), w = exp(lse - M),
 *   o = (w_a o_a + w_b o_b) / (w_a + w_b),  lse = M + ln(w_a + w_b);
 * both parts empty (lse = -inf) gives o = 0, lse = -inf.  Used to finish a query chunk
 * from a prefill over its cached prefix (non-causal) and one over the chunk (causal).
 *   o_a, o_b, o [B, S, H, D] of `dtype` (ATTN_BF16 or ATTN_F32); lse_a, lse_b [B, H, S]
 *   fp32 (the layout attn_prefill_fwd writes; a ragged batch is B = 1, S = total_q);
 *   lse: NULL or fp32 [B, H, S].  o may be o_a or o_b and lse may be lse_a or lse_b
 *   (in place); other overlaps are not allowed.
 *   Supported: D * element size a multiple of 16 bytes, D * element size / 16 a power of
 *   two <= 64 (bf16 D in {8, ..., 512}, fp32 D in {4, ..., 256}).
 */
int attn_merge_fwd(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o,
                   float* lse, int dtype, int B, int S, int H, int D, hipStream_t stream);

/*
 * Decode (token generation; AMD buffers page, token_gen variant of the K/V buffers):
 * one query token per sequence attends to keys [0, kv_lens[b]) of its cache.
 *   q [B,Hq,D] bf16; o [B,Hq,D] bf16;
 *   k_cache, v_cache [B,max_kv_len,Hkv,D] of the cache dtype:
 *     ATTN_BF16: bf16 values; k_scale and v_scale must be NULL.
 *     ATTN_FP8_E4M3: e4m3fn codes with per-token fp32 scales k_scale, v_scale
 *       [B,max_kv_len,Hkv] (one per key row and kv head, as the per-token-scale pages keep
 *       one k_scale per K row): K = code * k_scale, V = code * v_scale.  Both required.
 *   kv_lens: DEVICE int32 [B], clamped in-kernel to [0, max_kv_len] (0 gives O = 0).
 *   lse: NULL or fp32 [B,Hq].
 * The KV range of every sequence is split across workgroups; each writes a partial
 * (row max, row sum, unnormalised O) to `workspace`, and a second kernel on the same
 * stream merges the partials.  workspace: device memory of at least
 * attn_decode_workspace_size(B, Hq, Hkv, D, max_kv_len) bytes, owned by the caller (the
 * split count, and so the size, depends on the number of kv heads: one workgroup per
 * (split, batch, kv head)).  The size query returns 0 for invalid sizes.
 *   Supported: dtype ATTN_BF16 or ATTN_FP8_E4M3, D in {64, 128}, Hq % Hkv == 0,
 *   Hq / Hkv <= 16.
 */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_kv_len);
int attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, void* o,
                    float* lse, const int32_t* kv_lens, const float* k_scale,
                    const float* v_scale, int dtype, int B, int Hq, int Hkv, int D,
                    int max_kv_len, float softmax_scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no workspace argument; the
 * split partials go to a static buffer of ATTN_DECODE_STATIC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  The caller still passes q, the
 * caches, kv_lens and o (and lse), exactly as for attn_decode_fwd, with the same results.
 * The call allocates nothing.  It returns ATTN_ERR_SCRATCH, with nothing enqueued, when
 * attn_decode_workspace_size(B, Hq, Hkv, D, max_kv_len) exceeds the buffer (for example B 64,
 * Hq 32, Hkv 8, D 128 and 8192 keys need 8.5 MB).  All calls on one GPU share its buffer: calls
 * that overlap in time there (on different streams without ordering) race and give undefined
 * results; order them (one stream, or events).  The first call on a GPU resolves the buffer's
 * address there (hipGetSymbolAddress); a failure of that returns ATTN_ERR_HIP.
 */
#define ATTN_DECODE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int attn_decode_fwd_static(const void* q, const void* k_cache, const void* v_cache, void* o,
                           float* lse, const int32_t* kv_lens, const float* k_scale,
                           const float* v_scale, int dtype, int B, int Hq, int Hkv, int D,
                           int max_kv_len, float softmax_scale, hipStream_t stream);

/*
 * MLA prefill with per-token scales (MLASmemStorage page: Q and KV tiles each hold a
 * nope part in the qkv dtype and a rope part in the rope dtype, plus one fp32 q_scale
 * per Q row and one k_scale per K row of the tile; V is typed like Q and K_nope).  Logits:
 *   x[i,j] = scale * ( (q_nope_i . k_nope_j) * q_scale_i * k_scale_j + q_rope_i . k_rope_j )
 *   q_nope [B,Sq,H,Dn], k_nope [B,Skv,H,Dn]: `nope_dtype` (ATTN_FP8_E4M3 or ATTN_BF16);
 *   q_rope [B,Sq,H,Dr], k_rope [B,Skv,Hr,Dr] (Hr = 1: one rope head shared by all H,
 *   or Hr = H): bf16; o [B,Sq,H,Dv]: bf16;
 *   v [B,Skv,H,Dv] of `v_dtype`: ATTN_BF16 (v_scale must be NULL), or ATTN_FP8_E4M3 codes
 *   with one fp32 scale per V row, v_scale [B,Skv,H] (required): V = code * v_scale.  The
 *   products P.V run on bf16 matrix cores after an exact code conversion, with v_scale
 *   folded into P (P stays bf16: e4m3 P would cost ~2.5% relative error on O);
 *   q_scale [B,Sq,H], k_scale [B,Skv,H]: fp32, or NULL for all-ones;
 *   lse: NULL or fp32 [B,H,Sq].
 *   Supported: (Dn, Dr, Dv) == (128, 64, 128).
 */
int mla_prefill_fwd(const void* q_nope, const void* q_rope, const void* k_nope,
                    const void* k_rope, const void* v, void* o, const float* q_scale,
                    const float* k_scale, const float* v_scale, float* lse, int nope_dtype,
                    int v_dtype, int B, int Sq, int Skv, int H, int Hr, int Dn, int Dr, int Dv,
                    int causal, float softmax_scale, hipStream_t stream);

/*
 * MLA decode (KVPipelineGeneric page, MLA decode utilities): H query heads share one
 * latent KV head; a cache row is [latent Dv | rope Dk-Dv] and serves as K (all Dk
 * columns) and as V (its first Dv columns), read from HBM once.
 *   q [B,H,Dk] bf16; o [B,H,Dv] bf16;
 *   kv_cache [B,max_kv_len,Dk] of the cache dtype:
 *     ATTN_BF16: bf16 values; kv_scale must be NULL.
 *     ATTN_FP8_E4M3: e4m3fn codes with one fp32 scale per cache row, kv_scale
 *       [B,max_kv_len] (the row is one token's latent K and V, so its scale serves both):
 *       K = code * kv_scale, V = code[:Dv] * kv_scale.  Required.
 *   kv_lens DEVICE int32 [B] (clamped to [0, max_kv_len]); lse NULL or fp32 [B,H].
 *   workspace: at least mla_decode_workspace_size(B, H, Dv, max_kv_len) bytes.
 *   Supported: dtype ATTN_BF16 or ATTN_FP8_E4M3, (Dk, Dv) == (576, 512), H % 16 == 0,
 *   H <= 128.
 */
size_t mla_decode_workspace_size(int B, int H, int Dv, int max_kv_len);
int mla_decode_fwd(const void* q, const void* kv_cache, void* o, float* lse,
                   const int32_t* kv_lens, const float* kv_scale, int dtype, int B, int H,
                   int Dk, int Dv, int max_kv_len, float softmax_scale, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * Per-token e4m3 quantisation: produces the nope operands and scales that
 * mla_prefill_fwd consumes (MLASmemStorage page: one fp32 scale per Q-tile row,
 * q_scale_smem, and per K-tile row, k_scale_smem, beside the fp8 nope tiles).
 * For each of n_rows rows of cols fp32 values:
 *   scale[r]    = fp32(max_j |x[r][j]| / 448)   (1.0 for an all-zero row)
 *   codes[r][j] = e4m3fn(fp32(x[r][j] / scale[r])), round to nearest even
 * (OCP e4m3fn: bias 7, 3 mantissa bits, max 448, no infinity.)
 *   x: device fp32 [n_rows, cols]; codes: device uint8 [n_rows, cols];
 *   scale: device fp32 [n_rows]; all contiguous, owned by the caller.
 *   Rows must be finite; a row holding inf or NaN gives unspecified codes and scale.
 *   Supported: cols % 4 == 0 and 4 <= cols <= 4096 (else ATTN_ERR_UNSUPPORTED).
 */
int quantize_rows_e4m3(const float* x, uint8_t* codes, float* scale, int n_rows, int cols,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
