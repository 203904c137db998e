// C ABI of libattn.so: argument validation (host only, before any HIP call) and dispatch
// to the kernel launchers.  Declarations and contracts: include/attn.h.
#include "attn.h"

#include <cmath>
#include <cstdint>

#include "launch.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;

bool bad_scale(float s) { return !(std::isfinite(s) && s > 0.f); }

// product of non-negative sizes, or -1 on overflow past kMaxElems
int64_t elems(std::initializer_list<int64_t> dims) {
  int64_t n = 1;
  for (int64_t d : dims) {
    if (d < 0) return -1;
    if (d != 0 && n > kMaxElems / d) return -1;
    n *= d;
  }
  return n;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (negative size, Hq % Hkv != 0, or too large)";
    case ATTN_ERR_DTYPE: return "dtype not supported by this entry point";
    case ATTN_ERR_UNSUPPORTED: return "head dims or options outside the supported set";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch failed";
    case ATTN_ERR_SCALE: return "softmax_scale must be finite and positive";
    case ATTN_ERR_SCRATCH: return "decode partials larger than the static scratch buffer";
    default: return "unknown status";
  }
}

int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int B, int Sq,
                     int Skv, int Hq, int Hkv, int D, int causal, float softmax_scale, hipStream_t stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (B < 0 || Sq < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (elems({B, Sq, Hq, D}) < 0 || elems({B, Skv, Hkv, D}) < 0) return ATTN_ERR_SHAPE;
  if (elems({(Sq + 127) / 128, B, Hq}) > INT32_MAX) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (bad_scale(softmax_scale)) return ATTN_ERR_SCALE;
  if (B == 0 || Sq == 0) return ATTN_OK;
  if (!q || !o || (Skv > 0 && (!k || !v))) return ATTN_ERR_NULL;
  fa::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Sq = Sq; a.Skv = Skv; a.Hq = Hq; a.Hkv = Hkv; a.Hr = 1;
  a.causal = causal ? 1 : 0;
  a.scale = softmax_scale;
  return hip_status(dtype == ATTN_BF16 ? fa::launch_prefill_bf16(a, D, stream) : fa::launch_prefill_f32(a, D, stream));
}

int attn_prefill_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype, int B, int total_q,
                            int total_k, int max_seqlen_q, int Hq, int Hkv, int D, int causal, float softmax_scale,
                            hipStream_t stream) {
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (B < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0)
    return ATTN_ERR_SHAPE;
  if (elems({total_q, Hq, D}) < 0 || elems({total_k, Hkv, D}) < 0) return ATTN_ERR_SHAPE;
  if (elems({(max_seqlen_q + 127) / 128, (int64_t)(B * (int64_t)Hq + 7) / 8 * 8}) > INT32_MAX) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (bad_scale(softmax_scale)) return ATTN_ERR_SCALE;
  if (B == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_OK;
  if (!q || !o || !cu_seqlens_q || !cu_seqlens_k || (total_k > 0 && (!k || !v))) return ATTN_ERR_NULL;
  fa::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.total_q = total_q; a.total_k = total_k;
  a.B = B; a.Sq = max_seqlen_q; a.Skv = 0; a.Hq = Hq; a.Hkv = Hkv; a.Hr = 1;
  a.causal = causal ? 1 : 0;
  a.scale = softmax_scale;
  return hip_status(fa::launch_prefill_varlen_bf16(a, D, stream));
}

int attn_merge_fwd(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
                   int dtype, int B, int S, int H, int D, hipStream_t stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (B < 0 || S < 0 || H <= 0 || D <= 0) return ATTN_ERR_SHAPE;
  const int64_t n = elems({B, S, H, D});
  if (n < 0 || n > (int64_t)INT32_MAX * 64) return ATTN_ERR_SHAPE;
  const int esz = dtype == ATTN_BF16 ? 2 : 4;
  const int chunks = D * esz / 16;  // 16-byte chunks per row: a power of two up to 64
  if ((D * esz) % 16 != 0 || chunks > 64 || (chunks & (chunks - 1)) != 0) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o) return ATTN_ERR_NULL;
  fa::MergeArgs a{};
  a.o_a = o_a; a.lse_a = lse_a; a.o_b = o_b; a.lse_b = lse_b; a.o = o; a.lse = lse;
  a.B = B; a.S = S; a.H = H; a.D = D;
  a.log2_chunks = __builtin_ctz((unsigned)chunks);
  return hip_status(fa::launch_merge(a, dtype == ATTN_BF16, stream));
}

size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_kv_len) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_kv_len < 0) return 0;
  const fa::SplitPlan p = fa::gqa_decode_plan(B, Hkv, max_kv_len);
  return fa::decode_workspace_bytes(B, Hq, D, p.n_split);
}

}  // extern "C"

namespace {

// Host validation of a GQA decode call and its launch arguments (all but the partials).
int decode_args(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                const int32_t* kv_lens, const float* k_scale, const float* v_scale, int dtype, int B, int Hq,
                int Hkv, int D, int max_kv_len, float softmax_scale, fa::DecodeArgs& a, size_t& need) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_DTYPE;
  const bool fp8 = dtype == ATTN_FP8_E4M3;
  if (!fp8 && (k_scale || v_scale)) return ATTN_ERR_DTYPE;  // scales belong to e4m3 caches only
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_kv_len < 0 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (elems({B, max_kv_len, Hkv, D}) < 0 || elems({B, Hq, D}) < 0) return ATTN_ERR_SHAPE;
  if ((D != 64 && D != 128) || Hq / Hkv > 16) return ATTN_ERR_UNSUPPORTED;
  if (bad_scale(softmax_scale)) return ATTN_ERR_SCALE;
  if (B == 0) return ATTN_OK;
  if (!q || !o || !kv_lens || (max_kv_len > 0 && (!k_cache || !v_cache))) return ATTN_ERR_NULL;
  if (fp8 && max_kv_len > 0 && (!k_scale || !v_scale)) return ATTN_ERR_NULL;
  const fa::SplitPlan p = fa::gqa_decode_plan(B, Hkv, max_kv_len);
  if (B > 65535 || p.n_split > 65535 || elems({p.n_split, Hkv, (B + 7) / 8 * 8}) > INT32_MAX) return ATTN_ERR_SHAPE;
  if (elems({B, Hq, D}) / 8 > INT32_MAX - 256) return ATTN_ERR_SHAPE;  // combine: one thread per 8 columns
  need = fa::decode_workspace_bytes(B, Hq, D, p.n_split);
  a = fa::DecodeArgs{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse; a.kv_lens = kv_lens;
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.max_len = max_kv_len;
  a.n_split = p.n_split; a.chunk = p.chunk;
  a.scale = softmax_scale;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                    const int32_t* kv_lens, const float* k_scale, const float* v_scale, int dtype, int B,
                    int Hq, int Hkv, int D, int max_kv_len, float softmax_scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  fa::DecodeArgs a;
  size_t need = 0;
  const int st = decode_args(q, k_cache, v_cache, o, lse, kv_lens, k_scale, v_scale, dtype, B, Hq, Hkv, D,
                             max_kv_len, softmax_scale, a, need);
  if (st != ATTN_OK || B == 0) return st;
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + ((size_t)B * Hq * a.n_split * D * 4 + 255) / 256 * 256);
  return hip_status(fa::launch_gqa_decode(a, D, dtype == ATTN_FP8_E4M3, stream));
}

static_assert(ATTN_DECODE_STATIC_SCRATCH_BYTES == fa::kDecodeStaticScratchBytes, "static scratch size");

int attn_decode_fwd_static(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                           const int32_t* kv_lens, const float* k_scale, const float* v_scale, int dtype, int B,
                           int Hq, int Hkv, int D, int max_kv_len, float softmax_scale, hipStream_t stream) {
  fa::DecodeArgs a;
  size_t need = 0;
  const int st = decode_args(q, k_cache, v_cache, o, lse, kv_lens, k_scale, v_scale, dtype, B, Hq, Hkv, D,
                             max_kv_len, softmax_scale, a, need);
  if (st != ATTN_OK || B == 0) return st;
  if (need > fa::kDecodeStaticScratchBytes) return ATTN_ERR_SCRATCH;
  return hip_status(fa::launch_gqa_decode_static(a, D, dtype == ATTN_FP8_E4M3, stream));
}

int mla_prefill_fwd(const void* q_nope, const void* q_rope, const void* k_nope, const void* k_rope, const void* v,
                    void* o, const float* q_scale, const float* k_scale, const float* v_scale, float* lse,
                    int nope_dtype, int v_dtype, int B, int Sq, int Skv, int H, int Hr, int Dn, int Dr, int Dv,
                    int causal, float softmax_scale, hipStream_t stream) {
  if (nope_dtype != ATTN_FP8_E4M3 && nope_dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (v_dtype != ATTN_FP8_E4M3 && v_dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  const bool v_fp8 = v_dtype == ATTN_FP8_E4M3;
  if (!v_fp8 && v_scale) return ATTN_ERR_DTYPE;  // the value scale belongs to e4m3 V only
  if (B < 0 || Sq < 0 || Skv < 0 || H <= 0 || Hr <= 0 || Dn <= 0 || Dr <= 0 || Dv <= 0) return ATTN_ERR_SHAPE;
  if (Hr != 1 && Hr != H) return ATTN_ERR_SHAPE;
  if (elems({B, Sq, H, Dn + Dr + Dv}) < 0 || elems({B, Skv, H, Dn + Dr + Dv}) < 0) return ATTN_ERR_SHAPE;
  if (elems({(Sq + 127) / 128, B, H}) > INT32_MAX) return ATTN_ERR_SHAPE;
  if (Dn != 128 || Dr != 64 || Dv != 128) return ATTN_ERR_UNSUPPORTED;
  if (bad_scale(softmax_scale)) return ATTN_ERR_SCALE;
  if (B == 0 || Sq == 0) return ATTN_OK;
  if (!q_nope || !q_rope || !o || (Skv > 0 && (!k_nope || !k_rope || !v))) return ATTN_ERR_NULL;
  if (v_fp8 && Skv > 0 && !v_scale) return ATTN_ERR_NULL;
  fa::PrefillArgs a{};
  a.q = q_nope; a.k = k_nope; a.v = v; a.o = o; a.lse = lse;
  a.q_rope = q_rope; a.k_rope = k_rope; a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.B = B; a.Sq = Sq; a.Skv = Skv; a.Hq = H; a.Hkv = H; a.Hr = Hr;
  a.causal = causal ? 1 : 0;
  a.scale = softmax_scale;
  return hip_status(fa::launch_mla_prefill(a, nope_dtype == ATTN_FP8_E4M3, v_fp8, stream));
}

size_t mla_decode_workspace_size(int B, int H, int Dv, int max_kv_len) {
  if (B < 0 || H <= 0 || Dv <= 0 || max_kv_len < 0) return 0;
  const fa::SplitPlan p = fa::mla_decode_plan(B, H, max_kv_len);
  return fa::decode_workspace_bytes(B, H, Dv, p.n_split);
}

int mla_decode_fwd(const void* q, const void* kv_cache, void* o, float* lse, const int32_t* kv_lens,
                   const float* kv_scale, int dtype, int B, int H, int Dk, int Dv, int max_kv_len,
                   float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_DTYPE;
  const bool fp8 = dtype == ATTN_FP8_E4M3;
  if (!fp8 && kv_scale) return ATTN_ERR_DTYPE;  // the scale belongs to e4m3 caches only
  if (B < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || max_kv_len < 0 || Dv > Dk) return ATTN_ERR_SHAPE;
  if (elems({B, max_kv_len, Dk}) < 0 || elems({B, H, Dk}) < 0) return ATTN_ERR_SHAPE;
  if (Dk != 576 || Dv != 512 || H % 16 != 0 || H > 128) return ATTN_ERR_UNSUPPORTED;
  if (bad_scale(softmax_scale)) return ATTN_ERR_SCALE;
  if (B == 0) return ATTN_OK;
  if (!q || !o || !kv_lens || (max_kv_len > 0 && !kv_cache)) return ATTN_ERR_NULL;
  if (fp8 && max_kv_len > 0 && !kv_scale) return ATTN_ERR_NULL;
  const fa::SplitPlan p = fa::mla_decode_plan(B, H, max_kv_len);
  if (B > 65535 || elems({p.n_split, (B + 7) / 8 * 8}) > INT32_MAX) return ATTN_ERR_SHAPE;
  if (elems({B, H, Dv}) / 8 > INT32_MAX - 256) return ATTN_ERR_SHAPE;  // combine: one thread per 8 columns
  const size_t need = fa::decode_workspace_bytes(B, H, Dv, p.n_split);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  fa::DecodeArgs a{};
  a.q = q; a.k = kv_cache; a.v = nullptr; a.o = o; a.lse = lse; a.kv_lens = kv_lens;
  a.k_scale = kv_scale;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + ((size_t)B * H * p.n_split * Dv * 4 + 255) / 256 * 256);
  a.B = B; a.Hq = H; a.Hkv = 1; a.max_len = max_kv_len;
  a.n_split = p.n_split; a.chunk = p.chunk;
  a.scale = softmax_scale;
  return hip_status(fa::launch_mla_decode(a, fp8, stream));
}

int quantize_rows_e4m3(const float* x, uint8_t* codes, float* scale, int n_rows, int cols, hipStream_t stream) {
  if (n_rows < 0 || cols <= 0) return ATTN_ERR_SHAPE;
  if (elems({n_rows, cols}) < 0) return ATTN_ERR_SHAPE;
  if (cols % 4 != 0 || cols > 4096) return ATTN_ERR_UNSUPPORTED;
  if (n_rows == 0) return ATTN_OK;
  if (!x || !codes || !scale) return ATTN_ERR_NULL;
  fa::QuantArgs a{};
  a.x = x; a.codes = codes; a.scale = scale;
  a.n_rows = n_rows; a.cols = cols;
  a.lanes_per_row = fa::quantize_lanes_per_row(cols);
  return hip_status(fa::launch_quantize_rows(a, stream));
}

}  // extern "C"
