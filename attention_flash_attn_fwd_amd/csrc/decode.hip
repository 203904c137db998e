// Decode (token generation) kernels: split-KV partials and their combine.
//
// The AMD "buffers" page gives its K/V tile buffers a token_gen variant; Modular's
// "KVPipelineGeneric" page (MLA decode utilities) pipelines K/V tiles through S = Q.K'
// and O += P.V.  With one query token per sequence there is no query-row parallelism
// to fill the GPU, so the KV range of each sequence is cut into splits processed by
// independent waves; each writes (row max m, row sum l, unnormalised O) and a combine
// kernel merges them: M = max_s m_s, w_s = 2^((m_s - M) c), O = sum w_s O_s / sum w_s l_s.
//
// Both products use v_mfma_f32_16x16x32_bf16 in transposed form (S^T = K.Q^T and
// O^T = V^T.P^T); the 16 MFMA columns hold query heads (the Hq/Hkv heads of a GQA group,
// or 16 of the MLA heads).
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int TK = 32;  // keys per tile

// ------------------------------------------------------------------------------------
// GQA decode split: one wave per workgroup = one split of one (batch, kv head); the wave
// owns a private STAGES-deep LDS ring of K and V tiles (32 keys x 128 bf16 each), filled by
// direct global->LDS loads, so no workgroup barrier is needed.

template <int G>
__global__ __launch_bounds__(64) void gqa_decode_split(DecodeArgs a) {
  constexpr int D = 128, ROWB = 256, TILE = TK * ROWB, STAGES = 3;
  constexpr int OPS = 2 * TILE / 1024;  // vector-memory instructions per tile (K + V)
  __shared__ __attribute__((aligned(1024))) char smem_raw[STAGES * 2 * TILE];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = min(max(a.kv_lens[b], 0), a.max_len);
  const int start = split * a.chunk;
  if (start >= L) return;
  const int end = min(start + a.chunk, L);
  const int n_tiles = (end - start + TK - 1) / TK;

  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;
  const float c = a.scale * kLog2e;

  i32x4_t qf[D / 32];
  {
    const int hq = kvh * G + (l16 < G ? l16 : 0);
    const char* qp = (const char*)a.q + ((size_t)b * a.Hq + hq) * ROWB;
#pragma unroll
    for (int cc = 0; cc < D / 32; cc++) {
      i32x4_t x = *(const i32x4_t*)(qp + cc * 64 + g * 16);
      qf[cc] = l16 < G ? x : i32x4_t{};
    }
  }

  auto issue = [&](int t) {
    FA_LDS char* dst = smem + (t % STAGES) * 2 * TILE;
    const int key0 = start + t * TK;
#pragma unroll
    for (int i = 0; i < TILE / 1024; i++) {
      const int row = i * 4 + (lane >> 4);
      const int lch = (lane & 15) ^ swz256(row);
      const int key = min(key0 + row, L - 1);
      const size_t gi = (((size_t)b * a.max_len + key) * a.Hkv + kvh) * ROWB + lch * 16;
      dma16((const char*)a.k + gi, dst + i * 1024);
      dma16((const char*)a.v + gi, dst + TILE + i * 1024);
    }
  };

  RowState st{-INFINITY, 0.f};
  f32x4_t o[D / 16];
#pragma unroll
  for (int d = 0; d < D / 16; d++) o[d] = f32x4_t{};

#pragma unroll
  for (int t = 0; t < STAGES - 1; t++)
    if (t < n_tiles) issue(t);

  for (int t = 0; t < n_tiles; t++) {
    if (t + STAGES - 1 < n_tiles) issue(t + STAGES - 1);
    const int after = min(STAGES - 1, n_tiles - 1 - t);  // tiles issued after tile t
    if (after >= 2) wait_vmcnt<2 * OPS>();
    else if (after == 1) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");

    const FA_LDS char* kt = smem + (t % STAGES) * 2 * TILE;
    const FA_LDS char* vt = kt + TILE;
    f32x4_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      const int row = 16 * kb + l16;
      const FA_LDS char* r = kt + row * ROWB;
      const uint32_t sw = swz256(row);
      s[kb] = f32x4_t{};
#pragma unroll
      for (int cc = 0; cc < D / 32; cc++) s[kb] = mfma16x16x32_bf16(lds_b128(r + (((4 * cc + g) ^ sw) << 4)), qf[cc], s[kb]);
    }
    const int key0 = start + t * TK;
    if (key0 + TK > end) {
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int v = 0; v < 4; v++)
          if (key0 + 16 * kb + 4 * g + v >= end) s[kb][v] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = xor32_max(xor16_max(mx));
    float neg;
    const float alpha = softmax_rescale(st, mx, c, neg);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const float e = exp2_fast(fmaf(s[kb][v], c, neg));
        s[kb][v] = e;
        rs += e;
      }
    st.l = st.l * alpha + rs;
    const i32x4_t pb = {pack_bf16(s[0][0], s[0][1]), pack_bf16(s[0][2], s[0][3]), pack_bf16(s[1][0], s[1][1]),
                        pack_bf16(s[1][2], s[1][3])};
#pragma unroll
    for (int db = 0; db < D / 16; db++) {
      o[db] *= alpha;
      const int col = 16 * db + 4 * (l16 & 3);
      i32x2_t part[2];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int row = 16 * u + 4 * g + (l16 >> 2);
        part[u] = lds_tr16(vt + row * ROWB + ((((uint32_t)col >> 3) ^ swz256(row)) << 4) + (((col >> 2) & 1) << 3));
      }
      o[db] = mfma16x16x32_bf16(cat(part[0], part[1]), pb, o[db]);
    }
  }

  const float l_tot = xor32_sum(xor16_sum(st.l));
  if (l16 < G) {
    const int hq = kvh * G + l16;
    const size_t pidx = ((size_t)b * a.Hq + hq) * a.n_split + split;
    float* po = a.part_o + pidx * D;
#pragma unroll
    for (int db = 0; db < D / 16; db++) *(f32x4_t*)(po + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      a.part_ml[2 * pidx] = st.m;
      a.part_ml[2 * pidx + 1] = l_tot;
    }
  }
}

// ------------------------------------------------------------------------------------
// MLA decode split: workgroup = H/16 waves sharing one LDS ring of latent tiles
// (32 keys x 576 bf16 = 36 KiB, two stages); wave w owns heads 16w..16w+15.  The tile feeds
// S^T over all 576 columns and, through transposing reads of its first 512 columns,
// O^T = V^T.P^T: the latent cache is read from HBM once.

constexpr int MLA_DK = 576, MLA_DV = 512, MLA_ROWB = 1152, MLA_TILE = TK * MLA_ROWB;

__global__ __launch_bounds__(512) void mla_decode_split(DecodeArgs a) {
  constexpr int STAGES = 2;
  __shared__ __attribute__((aligned(1024))) char smem_raw[STAGES * MLA_TILE];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;

  const int split = blockIdx.x, b = blockIdx.y;
  const int nw = blockDim.x >> 6;
  const int L = min(max(a.kv_lens[b], 0), a.max_len);
  const int start = split * a.chunk;
  if (start >= L) return;  // uniform over the workgroup
  const int end = min(start + a.chunk, L);
  const int n_tiles = (end - start + TK - 1) / TK;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const int h = 16 * wave + l16;
  const float c = a.scale * kLog2e;

  i32x4_t qf[MLA_DK / 32];
  {
    const char* qp = (const char*)a.q + ((size_t)b * a.Hq + h) * MLA_ROWB;
#pragma unroll
    for (int cc = 0; cc < MLA_DK / 32; cc++) qf[cc] = *(const i32x4_t*)(qp + cc * 64 + g * 16);
  }

  auto issue = [&](int t) {
    FA_LDS char* dst = smem + (t % STAGES) * MLA_TILE;
    const int key0 = start + t * TK;
    for (int blk = wave; blk < MLA_TILE / 1024; blk += nw) {
      const int o = blk * 1024 + lane * 16;
      const int row = o / MLA_ROWB;
      const int lch = ((o % MLA_ROWB) >> 4) ^ swz_half(row);
      const int key = min(key0 + row, L - 1);
      dma16((const char*)a.k + ((size_t)b * a.max_len + key) * MLA_ROWB + lch * 16, dst + blk * 1024);
    }
  };

  RowState st{-INFINITY, 0.f};
  f32x4_t o[MLA_DV / 16];
#pragma unroll
  for (int d = 0; d < MLA_DV / 16; d++) o[d] = f32x4_t{};

  issue(0);
  for (int t = 0; t < n_tiles; t++) {
    wait_vmcnt<0>();
    barrier();
    if (t + 1 < n_tiles) issue(t + 1);
    const FA_LDS char* kt = smem + (t % STAGES) * MLA_TILE;

    f32x4_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      const int row = 16 * kb + l16;
      const FA_LDS char* r = kt + row * MLA_ROWB;
      const uint32_t sw = swz_half(row);
      s[kb] = f32x4_t{};
#pragma unroll
      for (int cc = 0; cc < MLA_DK / 32; cc++)
        s[kb] = mfma16x16x32_bf16(lds_b128(r + (((4 * cc + g) ^ sw) << 4)), qf[cc], s[kb]);
    }
    const int key0 = start + t * TK;
    if (key0 + TK > end) {
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int v = 0; v < 4; v++)
          if (key0 + 16 * kb + 4 * g + v >= end) s[kb][v] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = xor32_max(xor16_max(mx));
    float neg;
    const float alpha = softmax_rescale(st, mx, c, neg);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const float e = exp2_fast(fmaf(s[kb][v], c, neg));
        s[kb][v] = e;
        rs += e;
      }
    st.l = st.l * alpha + rs;
    const i32x4_t pb = {pack_bf16(s[0][0], s[0][1]), pack_bf16(s[0][2], s[0][3]), pack_bf16(s[1][0], s[1][1]),
                        pack_bf16(s[1][2], s[1][3])};
#pragma unroll
    for (int db = 0; db < MLA_DV / 16; db++) {
      o[db] *= alpha;
      const int col = 16 * db + 4 * (l16 & 3);
      i32x2_t part[2];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int row = 16 * u + 4 * g + (l16 >> 2);
        part[u] = lds_tr16(kt + row * MLA_ROWB + ((((uint32_t)col >> 3) ^ swz_half(row)) << 4) + (((col >> 2) & 1) << 3));
      }
      o[db] = mfma16x16x32_bf16(cat(part[0], part[1]), pb, o[db]);
    }
  }

  const float l_tot = xor32_sum(xor16_sum(st.l));
  const size_t pidx = ((size_t)b * a.Hq + h) * a.n_split + split;
  float* po = a.part_o + pidx * MLA_DV;
#pragma unroll
  for (int db = 0; db < MLA_DV / 16; db++) *(f32x4_t*)(po + 16 * db + 4 * g) = o[db];
  if (g == 0) {
    a.part_ml[2 * pidx] = st.m;
    a.part_ml[2 * pidx + 1] = l_tot;
  }
}

// ------------------------------------------------------------------------------------
// Combine: one workgroup per (batch, head); merges the splits that cover [0, L_b) in
// split order (deterministic, no atomics).

__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a, int Dv) {
  const int bh = blockIdx.x, b = bh / a.Hq, h = bh % a.Hq;
  const int L = min(max(a.kv_lens[b], 0), a.max_len);
  const int ns = (L + a.chunk - 1) / a.chunk;
  const float c = a.scale * kLog2e;
  const float* ml = a.part_ml + (size_t)bh * a.n_split * 2;
  const float* po = a.part_o + (size_t)bh * a.n_split * Dv;
  float M = -INFINITY;
  for (int s = 0; s < ns; s++) M = fmaxf(M, ml[2 * s]);
  float den = 0.f;
  for (int s = 0; s < ns; s++) den += exp2_fast((ml[2 * s] - M) * c) * ml[2 * s + 1];
  const float inv = den > 0.f ? 1.f / den : 0.f;
  __bf16* out = (__bf16*)a.o + (size_t)bh * Dv;
  for (int d = 2 * threadIdx.x; d < Dv; d += 2 * blockDim.x) {
    float x0 = 0.f, x1 = 0.f;
    for (int s = 0; s < ns; s++) {
      const float w = exp2_fast((ml[2 * s] - M) * c);
      x0 = fmaf(w, po[(size_t)s * Dv + d], x0);
      x1 = fmaf(w, po[(size_t)s * Dv + d + 1], x1);
    }
    *(int*)(out + d) = pack_bf16(x0 * inv, x1 * inv);
  }
  if (a.lse && threadIdx.x == 0) a.lse[bh] = den > 0.f ? M * a.scale + logf(den) : -INFINITY;
}

}  // namespace

SplitPlan gqa_decode_plan(int B, int Hq, int max_len) {
  (void)Hq;
  int chunk = 256;
  // keep at least ~2048 waves in flight for small batches
  while (chunk > TK && (long)B * 8 * ((max_len + chunk - 1) / chunk) < 2048) chunk /= 2;
  SplitPlan p;
  p.chunk = chunk;
  p.n_split = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
  return p;
}

SplitPlan mla_decode_plan(int B, int H, int max_len) {
  (void)H;
  // one workgroup per CU: aim for >= 256 workgroups in total
  int want = B > 0 ? (256 + B - 1) / B : 1;
  int n_tiles = max_len > 0 ? (max_len + TK - 1) / TK : 1;
  want = max(1, min(want, n_tiles));
  int chunk = ((n_tiles + want - 1) / want) * TK;
  SplitPlan p;
  p.chunk = chunk;
  p.n_split = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
  return p;
}

size_t decode_workspace_bytes(int B, int Hq, int Dv, int n_split) {
  const size_t rows = (size_t)B * Hq * n_split;
  const size_t o_bytes = (rows * Dv * 4 + 255) / 256 * 256;
  return o_bytes + rows * 2 * 4;
}

hipError_t launch_gqa_decode(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid(a.n_split, a.Hkv, a.B);
  switch (G) {
#define FA_G(n) case n: gqa_decode_split<n><<<grid, 64, 0, s>>>(a); break;
    FA_G(1) FA_G(2) FA_G(3) FA_G(4) FA_G(5) FA_G(6) FA_G(7) FA_G(8)
    FA_G(9) FA_G(10) FA_G(11) FA_G(12) FA_G(13) FA_G(14) FA_G(15) FA_G(16)
#undef FA_G
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_kernel<<<a.B * a.Hq, 64, 0, s>>>(a, 128);
  return hipGetLastError();
}

hipError_t launch_mla_decode(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.B);
  mla_decode_split<<<grid, 64 * (a.Hq / 16), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_kernel<<<a.B * a.Hq, 256, 0, s>>>(a, MLA_DV);
  return hipGetLastError();
}

}  // namespace fa
