// fp32 prefill forward (MHA / GQA), the small-problem path.
//
// Same method as the bf16 kernel (S = Q.K' and O += P.V per K/V tile with the online-softmax
// correction, as Modular's "KVPipelineGeneric" page pipelines them), on fp32 matrix cores:
// v_mfma_f32_32x32x2_f32 for both products, in the transposed form that lets a lane own one
// query column (S^T = K.Q^T, O^T = V^T.P^T).  K/V tiles of 32 keys are staged through LDS with
// ordinary loads, one stage: the fp32 workload is small and latency-bound.
//
// This file is compiled with the matrix-core accumulators in ordinary vector registers
// (-mllvm -amdgpu-mfma-vgpr-form): at head dim 64 the kernels then run four waves per SIMD
// instead of two or three (5.7 % faster on a causal B4 H8 S1100 D64 call).
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int BM = 128;

// fp32 prefill: v_mfma_f32_32x32x2_f32 for both products, K/V tiles of 32 keys staged
// through LDS with ordinary loads (one stage).  S^T MFMA number c contracts head-dim
// columns c (lanes 0-31) and c + D/2 (lanes 32-63).

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs p, int n_qblocks) {
  constexpr int BNF = 32, LD = D + 4;
  __shared__ float kt[BNF][LD];
  __shared__ float vt[BNF][LD];
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int BH = p.B * p.Hq;
  const int rank = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int qb = CAUSAL ? (n_qblocks - 1 - rank) : rank;
  const int b = bh / p.Hq, h = bh % p.Hq, kvh = h / (p.Hq / p.Hkv);
  const int q0 = qb * BM, off = p.Skv - p.Sq;
  int kv_end = p.Skv;
  if (CAUSAL) kv_end = max(0, min(p.Skv, min(q0 + BM, p.Sq) - 1 + off + 1));
  const int n_tiles = (kv_end + BNF - 1) / BNF;
  const int qrow = q0 + 32 * wave + l32, qrow_c = min(qrow, p.Sq - 1);
  const float c = p.scale * kLog2e;

  float q[D / 2];
  {
    const float* qp = (const float*)p.q + (((size_t)b * p.Sq + qrow_c) * p.Hq + h) * D + (D / 2) * hl;
#pragma unroll
    for (int i = 0; i < D / 2; i += 4) {
      f32x4_t x = *(const f32x4_t*)(qp + i);
      q[i] = x.x; q[i + 1] = x.y; q[i + 2] = x.z; q[i + 3] = x.w;
    }
  }
  RowState st{-INFINITY, 0.f};
  f32x16_t o[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; d++) o[d] = f32x16_t{};

  for (int t = 0; t < n_tiles; t++) {
    __syncthreads();
    for (int e = tid * 4; e < BNF * D; e += 256 * 4) {
      const int row = e / D, col = e % D;
      const int key = min(t * BNF + row, p.Skv - 1);
      const size_t gi = (((size_t)b * p.Skv + key) * p.Hkv + kvh) * D + col;
      *(f32x4_t*)&kt[row][col] = *(const f32x4_t*)((const float*)p.k + gi);
      *(f32x4_t*)&vt[row][col] = *(const f32x4_t*)((const float*)p.v + gi);
    }
    __syncthreads();
    f32x16_t s{};
#pragma unroll
    for (int cc = 0; cc < D / 2; cc++) s = mfma32x32x2_f32(kt[l32][cc + (D / 2) * hl], q[cc], s);
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int key = t * BNF + 8 * (v >> 2) + 4 * hl + (v & 3);
      const bool vis = key < p.Skv && (!CAUSAL || key <= qrow + off);
      s[v] = vis ? s[v] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; v++) mx = fmaxf(mx, s[v]);
    mx = xor32_max(mx);
    float neg;
    const float alpha = softmax_rescale(st, mx, c, neg);
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < 16; v++) {
      s[v] = exp2_fast(fmaf(s[v], c, neg));
      rs += s[v];
    }
    st.l = st.l * alpha + rs;
#pragma unroll
    for (int d = 0; d < D / 32; d++) o[d] *= alpha;
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int key = 8 * (v >> 2) + 4 * hl + (v & 3);
#pragma unroll
      for (int d = 0; d < D / 32; d++) o[d] = mfma32x32x2_f32(vt[key][32 * d + l32], s[v], o[d]);
    }
  }
  const float l_tot = xor32_sum(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < p.Sq) {
    float* op = (float*)p.o + (((size_t)b * p.Sq + qrow) * p.Hq + h) * D;
#pragma unroll
    for (int d = 0; d < D / 32; d++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        *(f32x4_t*)(op + 32 * d + 8 * j + 4 * hl) =
            f32x4_t{o[d][4 * j] * inv, o[d][4 * j + 1] * inv, o[d][4 * j + 2] * inv, o[d][4 * j + 3] * inv};
    if (p.lse && hl == 0)
      p.lse[((size_t)b * p.Hq + h) * p.Sq + qrow] = l_tot > 0.f ? st.m * p.scale + logf(l_tot) : -INFINITY;
  }
}

// Small fp32 problems (fewer 128-row blocks than CUs): one workgroup per (batch, head, 32 query
// rows), whose four waves take every fourth K/V tile each, so that a row block's key range is
// worked on by four SIMDs at once.  A wave reads its tiles straight from memory into the MFMA
// operand registers (a lane's K operands are half of one key row, contiguous; its V^T operands
// are one column of 16 key rows, read 128 bytes per row across the half-wave), so the loop has
// no LDS stage and no barrier.  The waves' partial results (row max m_w, lane-partial row sum
// l_w, unnormalised O^T) meet in LDS at the end, where wave 0 merges them in wave order:
// O = sum_w 2^((m_w - M) c) O_w / sum_w 2^((m_w - M) c) l_w with M = max_w m_w.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void prefill_f32_split_kernel(PrefillArgs p) {
  constexpr int BNF = 32, NW = 4, NB = D / 32;
  __shared__ float xo[NW - 1][NB * 16][64];  // O^T registers of waves 1..3, [register][lane]
  __shared__ float xm[NW - 1][64], xl[NW - 1][64];
  const int wave = wave_id(), lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
  const int BH = p.B * p.Hq;
  const int rb = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int b = bh / p.Hq, h = bh % p.Hq, kvh = h / (p.Hq / p.Hkv);
  const int q0 = rb * 32, off = p.Skv - p.Sq;
  int kv_end = p.Skv;
  if (CAUSAL) kv_end = max(0, min(p.Skv, min(q0 + 32, p.Sq) - 1 + off + 1));
  const int n_tiles = (kv_end + BNF - 1) / BNF;
  const int qrow = q0 + l32, qrow_c = min(qrow, p.Sq - 1);
  const float c = p.scale * kLog2e;

  float q[D / 2];
  {
    const float* qp = (const float*)p.q + (((size_t)b * p.Sq + qrow_c) * p.Hq + h) * D + (D / 2) * hl;
#pragma unroll
    for (int i = 0; i < D / 2; i += 4) {
      const f32x4_t x = *(const f32x4_t*)(qp + i);
      q[i] = x.x; q[i + 1] = x.y; q[i + 2] = x.z; q[i + 3] = x.w;
    }
  }
  RowState st{-INFINITY, 0.f};
  f32x16_t o[NB];
#pragma unroll
  for (int d = 0; d < NB; d++) o[d] = f32x16_t{};
  const size_t kv_row0 = (size_t)b * p.Skv * p.Hkv + kvh;  // row index of (batch, key 0, kv head)

  for (int t = wave; t < n_tiles; t += NW) {
    // S^T A operands: key row t*32 + l32 (keys past Skv repeat the last one; they are masked),
    // head-dim columns (D/2) hl ..
    float kr[D / 2];
    {
      const int key = min(t * BNF + l32, p.Skv - 1);
      const float* kp = (const float*)p.k + (kv_row0 + (size_t)key * p.Hkv) * D + (D / 2) * hl;
#pragma unroll
      for (int i = 0; i < D / 2; i += 4) {
        const f32x4_t x = *(const f32x4_t*)(kp + i);
        kr[i] = x.x; kr[i + 1] = x.y; kr[i + 2] = x.z; kr[i + 3] = x.w;
      }
    }
    f32x16_t s{};
#pragma unroll
    for (int cc = 0; cc < D / 2; cc++) s = mfma32x32x2_f32(kr[cc], q[cc], s);
    // register v holds key t*32 + 8(v/4) + 4hl + v%4
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int key = t * BNF + 8 * (v >> 2) + 4 * hl + (v & 3);
      const bool vis = key < p.Skv && (!CAUSAL || key <= qrow + off);
      s[v] = vis ? s[v] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; v++) mx = fmaxf(mx, s[v]);
    mx = xor32_max(mx);
    float neg;
    const float alpha = softmax_rescale(st, mx, c, neg);
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < 16; v++) {
      s[v] = exp2_fast(fmaf(s[v], c, neg));
      rs += s[v];
    }
    st.l = st.l * alpha + rs;
#pragma unroll
    for (int d = 0; d < NB; d++) o[d] *= alpha;
    // O^T += V^T P^T: the A operand of register v is V[key of v][32 d + l32]
#pragma unroll
    for (int v = 0; v < 16; v++) {
      const int key = min(t * BNF + 8 * (v >> 2) + 4 * hl + (v & 3), p.Skv - 1);
      const float* vp = (const float*)p.v + (kv_row0 + (size_t)key * p.Hkv) * D + l32;
#pragma unroll
      for (int d = 0; d < NB; d++) o[d] = mfma32x32x2_f32(vp[32 * d], s[v], o[d]);
    }
  }

  if (wave > 0) {
    xm[wave - 1][lane] = st.m;
    xl[wave - 1][lane] = st.l;
#pragma unroll
    for (int d = 0; d < NB; d++)
#pragma unroll
      for (int v = 0; v < 16; v++) xo[wave - 1][16 * d + v][lane] = o[d][v];
  }
  __syncthreads();
  if (wave != 0) return;
  float M = st.m;
#pragma unroll
  for (int w = 0; w < NW - 1; w++) M = fmaxf(M, xm[w][lane]);
  const float m_use = M == -INFINITY ? 0.f : M;
  {
    const float a0 = st.m == -INFINITY ? 0.f : exp2_fast((st.m - m_use) * c);
    st.l *= a0;
#pragma unroll
    for (int d = 0; d < NB; d++) o[d] *= a0;
  }
#pragma unroll
  for (int w = 0; w < NW - 1; w++) {
    const float mw = xm[w][lane];
    const float aw = mw == -INFINITY ? 0.f : exp2_fast((mw - m_use) * c);
    st.l = fmaf(aw, xl[w][lane], st.l);
#pragma unroll
    for (int d = 0; d < NB; d++)
#pragma unroll
      for (int v = 0; v < 16; v++) o[d][v] = fmaf(aw, xo[w][16 * d + v][lane], o[d][v]);
  }
  const float l_tot = xor32_sum(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < p.Sq) {
    float* op = (float*)p.o + (((size_t)b * p.Sq + qrow) * p.Hq + h) * D;
#pragma unroll
    for (int d = 0; d < NB; d++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        *(f32x4_t*)(op + 32 * d + 8 * j + 4 * hl) =
            f32x4_t{o[d][4 * j] * inv, o[d][4 * j + 1] * inv, o[d][4 * j + 2] * inv, o[d][4 * j + 3] * inv};
    if (p.lse && hl == 0)
      p.lse[((size_t)b * p.Hq + h) * p.Sq + qrow] = l_tot > 0.f ? M * p.scale + logf(l_tot) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int D, hipStream_t s) {
  const int nqb = (a.Sq + BM - 1) / BM;
  const int grid = nqb * a.B * a.Hq;
  if (grid == 0) return hipSuccess;
  if (grid < 256) {
    // fewer 128-row blocks than CUs: 32-row blocks whose waves split the keys
    const int g32 = (a.Sq + 31) / 32 * a.B * a.Hq;
    if (D == 128) {
      if (a.causal) prefill_f32_split_kernel<128, true><<<g32, 256, 0, s>>>(a);
      else prefill_f32_split_kernel<128, false><<<g32, 256, 0, s>>>(a);
    } else {
      if (a.causal) prefill_f32_split_kernel<64, true><<<g32, 256, 0, s>>>(a);
      else prefill_f32_split_kernel<64, false><<<g32, 256, 0, s>>>(a);
    }
    return hipGetLastError();
  }
  if (D == 128) {
    if (a.causal) prefill_f32_kernel<128, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_f32_kernel<128, false><<<grid, 256, 0, s>>>(a, nqb);
  } else {
    if (a.causal) prefill_f32_kernel<64, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_f32_kernel<64, false><<<grid, 256, 0, s>>>(a, nqb);
  }
  return hipGetLastError();
}

}  // namespace fa
