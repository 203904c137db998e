// Prefill forward kernels (MHA / GQA in bf16 or fp32, and MLA with e4m3 nope + bf16 rope).
//
// Method: the flash-attention forward that Modular's "KVPipelineGeneric" page describes
// (S = Q.K' and O += P.V per K/V tile, over a pipeline of K/V stages), with the online
// softmax whose per-row correction the "MLASmemStorage" page keeps in a correction
// buffer: here the correction factor stays in the lane that owns the row.  The AMD
// "buffers" page's roles map as follows: QRegisterBuffer -> Q fragments in VGPRs;
// KBufferLDS / KVBufferLDS (direct DRAM->LDS, no register staging) -> global_load_lds
// into a swizzled two-stage LDS ring; VBufferTransposeLoads -> ds_read_b64_tr_b16;
// PRegisterBuffer -> P packed to bf16 in VGPRs; OutputRegisterBuffer -> O^T accumulators.
//
// Workgroup: 4 waves, BM = 128 query rows (32 per wave), K/V tiles of BN = 64 keys.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NW = 4;

// ------------------------------------------------------------------------------------
// Q.K^T policies: how Q is held in registers, how the K part of a tile is laid out in
// LDS, and how one 32-key block of S^T is formed.

// MHA / GQA: bf16 q/k of head dim D.
template <int D>
struct QkBf16 {
  static constexpr int ROWB = D * 2;
  static constexpr int KBYTES = BN * ROWB;
  struct QFrag {
    i32x4_t c[D / 16];
  };
  __device__ static uint32_t swz(uint32_t row) { return D == 128 ? swz256(row) : swz_half(row); }

  __device__ static void load_q(const PrefillArgs& p, int b, int h, int qrow, int hl, QFrag& q) {
    const char* base = (const char*)p.q + (((size_t)b * p.Sq + qrow) * p.Hq + h) * (size_t)ROWB;
#pragma unroll
    for (int c = 0; c < D / 16; c++) q.c[c] = *(const i32x4_t*)(base + c * 32 + hl * 16);
  }

  __device__ static void load_k(const PrefillArgs& p, int b, int h, int kvh, int key0, FA_LDS char* dst,
                                int wave, int lane) {
    constexpr int RPI = 1024 / ROWB, CPR = ROWB / 16, NI = KBYTES / 1024 / NW;
#pragma unroll
    for (int i = 0; i < NI; i++) {
      int blk = i * NW + wave;
      int row = blk * RPI + lane / CPR;
      int lch = (lane % CPR) ^ swz(row);
      int key = min(key0 + row, p.Skv - 1);
      const char* g = (const char*)p.k + (((size_t)b * p.Skv + key) * p.Hkv + kvh) * (size_t)ROWB + lch * 16;
      dma16(g, dst + blk * 1024);
    }
  }

  __device__ static void scores(const QFrag& q, const FA_LDS char* kt, int kb, int l32, int hl, f32x16_t& s,
                                bool /*has_kscale*/) {
    const int row = 32 * kb + l32;
    const FA_LDS char* r = kt + row * ROWB;
    const uint32_t sw = swz(row);
    s = f32x16_t{};
#pragma unroll
    for (int c = 0; c < D / 16; c++) {
      i32x4_t a = lds_b128(r + (((2 * c + hl) ^ sw) << 4));
      s = mfma32x32x16_bf16(a, q.c[c], s);
    }
  }
};

// MLA prefill with per-token scales: nope part (Dn = 128) in e4m3 or bf16, rope part
// (Dr = 64) in bf16 with Hr rope heads, fp32 q_scale per query row and k_scale per key.
// K part of a stage: k_nope [BN][Dn] | k_rope [BN][64] bf16 (128-byte rows) | k_scale [BN] fp32.
template <bool FP8>
struct QkMla {
  static constexpr int NROWB = FP8 ? 128 : 256;
  static constexpr int KN = 0;
  static constexpr int KR = BN * NROWB;
  static constexpr int KS = KR + BN * 128;
  static constexpr int KBYTES = KS + BN * 4;
  struct QFrag {
    i32x8_t n8[2];        // e4m3: 2 x (32 bytes) per lane
    i32x4_t n16[FP8 ? 1 : 8];
    i32x4_t r[4];
    float qs;
  };
  __device__ static uint32_t nswz(uint32_t row) { return FP8 ? swz_half(row) : swz256(row); }

  __device__ static void load_q(const PrefillArgs& p, int b, int h, int qrow, int hl, QFrag& q) {
    const size_t tok = ((size_t)b * p.Sq + qrow) * p.Hq + h;
    const char* n = (const char*)p.q + tok * NROWB;
    if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < 2; c++) {
        i32x4_t lo = *(const i32x4_t*)(n + c * 64 + hl * 32);
        i32x4_t hi = *(const i32x4_t*)(n + c * 64 + hl * 32 + 16);
        q.n8[c] = i32x8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; c++) q.n16[c] = *(const i32x4_t*)(n + c * 32 + hl * 16);
    }
    const char* r = (const char*)p.q_rope + tok * 128;
#pragma unroll
    for (int c = 0; c < 4; c++) q.r[c] = *(const i32x4_t*)(r + c * 32 + hl * 16);
    q.qs = p.q_scale ? p.q_scale[tok] : 1.f;
  }

  __device__ static void load_k(const PrefillArgs& p, int b, int h, int kvh, int key0, FA_LDS char* dst,
                                int wave, int lane) {
    (void)kvh;
    {  // nope
      constexpr int RPI = 1024 / NROWB, CPR = NROWB / 16, NI = BN * NROWB / 1024 / NW;
#pragma unroll
      for (int i = 0; i < NI; i++) {
        int blk = i * NW + wave;
        int row = blk * RPI + lane / CPR;
        int lch = (lane % CPR) ^ nswz(row);
        int key = min(key0 + row, p.Skv - 1);
        const char* g = (const char*)p.k + (((size_t)b * p.Skv + key) * p.Hq + h) * (size_t)NROWB + lch * 16;
        dma16(g, dst + KN + blk * 1024);
      }
    }
    {  // rope: 128-byte rows, 8 per wave instruction
      const int hr = p.Hr == 1 ? 0 : h;
#pragma unroll
      for (int i = 0; i < BN * 128 / 1024 / NW; i++) {
        int blk = i * NW + wave;
        int row = blk * 8 + lane / 8;
        int lch = (lane % 8) ^ swz_half(row);
        int key = min(key0 + row, p.Skv - 1);
        const char* g = (const char*)p.k_rope + (((size_t)b * p.Skv + key) * p.Hr + hr) * 128 + lch * 16;
        dma16(g, dst + KR + blk * 1024);
      }
    }
    if (p.k_scale && wave == 0) {
      int key = min(key0 + lane, p.Skv - 1);
      dma4(p.k_scale + ((size_t)b * p.Skv + key) * p.Hq + h, dst + KS);
    }
  }

  __device__ static void scores(const QFrag& q, const FA_LDS char* kt, int kb, int l32, int hl, f32x16_t& s,
                                bool has_kscale) {
    const int row = 32 * kb + l32;
    f32x16_t sn{};
    {
      const FA_LDS char* r = kt + KN + row * NROWB;
      const uint32_t sw = nswz(row);
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < 2; c++) {
          i32x4_t lo = lds_b128(r + (((4 * c + 2 * hl) ^ sw) << 4));
          i32x4_t hi = lds_b128(r + (((4 * c + 2 * hl + 1) ^ sw) << 4));
          sn = mfma32x32x64_e4m3(i32x8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, q.n8[c], sn);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; c++) sn = mfma32x32x16_bf16(lds_b128(r + (((2 * c + hl) ^ sw) << 4)), q.n16[c], sn);
      }
    }
    f32x16_t sr{};
    {
      const FA_LDS char* r = kt + KR + row * 128;
      const uint32_t sw = swz_half(row);
#pragma unroll
      for (int c = 0; c < 4; c++) sr = mfma32x32x16_bf16(lds_b128(r + (((2 * c + hl) ^ sw) << 4)), q.r[c], sr);
    }
    // lane holds keys 32kb + 8j + 4hl + i for register 4j + i
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f32x4_t ks = has_kscale ? lds_f32x4(kt + KS + (32 * kb + 8 * j + 4 * hl) * 4) : f32x4_t{1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int i = 0; i < 4; i++) s[4 * j + i] = fmaf(sn[4 * j + i], q.qs * ks[i], sr[4 * j + i]);
    }
  }
};

// V tile [BN][DV] bf16 of kv head `kvh`, rows swizzled like K.
template <int DV>
__device__ __forceinline__ void load_v(const PrefillArgs& p, int b, int kvh, int key0, FA_LDS char* dst, int wave,
                                       int lane) {
  constexpr int ROWB = DV * 2, RPI = 1024 / ROWB, CPR = ROWB / 16, NI = BN * ROWB / 1024 / NW;
#pragma unroll
  for (int i = 0; i < NI; i++) {
    int blk = i * NW + wave;
    int row = blk * RPI + lane / CPR;
    int lch = (lane % CPR) ^ (DV == 128 ? swz256(row) : swz_half(row));
    int key = min(key0 + row, p.Skv - 1);
    const char* g = (const char*)p.v + (((size_t)b * p.Skv + key) * p.Hkv + kvh) * (size_t)ROWB + lch * 16;
    dma16(g, dst + blk * 1024);
  }
}

// ------------------------------------------------------------------------------------
// The bf16 / MLA prefill kernel.

template <class QK, int DV, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs p, int n_qblocks) {
  constexpr int KPART = (QK::KBYTES + 1023) / 1024 * 1024;
  constexpr int VROWB = DV * 2;
  constexpr int STAGE = KPART + BN * VROWB;
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * STAGE];
  FA_LDS char* smem = (FA_LDS char*)smem_raw;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;

  // work item: q-blocks with the most keys first when causal
  const int BH = p.B * p.Hq;
  const int rank = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int qb = CAUSAL ? (n_qblocks - 1 - rank) : rank;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int kvh = h / (p.Hq / p.Hkv);
  const int q0 = qb * BM;
  const int off = p.Skv - p.Sq;

  int kv_end = p.Skv;
  if (CAUSAL) kv_end = max(0, min(p.Skv, min(q0 + BM, p.Sq) - 1 + off + 1));
  const int n_tiles = (kv_end + BN - 1) / BN;

  const int wrow0 = q0 + 32 * wave;                      // first query row of this wave
  int wave_end = kv_end, mask_from = p.Skv / BN;
  if (CAUSAL) {
    wave_end = max(0, min(kv_end, wrow0 + 31 + off + 1));
    const int lim = wrow0 + off + 1;
    mask_from = min(mask_from, lim > 0 ? lim / BN : 0);
  }
  const int wave_tiles = (wave_end + BN - 1) / BN;

  const int qrow = wrow0 + l32;
  const int qrow_c = min(qrow, p.Sq - 1);
  const float c = p.scale * kLog2e;
  const bool has_ks = p.k_scale != nullptr;

  typename QK::QFrag qf;
  QK::load_q(p, b, h, qrow_c, hl, qf);

  RowState st{-INFINITY, 0.f};
  f32x16_t o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; d++) o[d] = f32x16_t{};

  if (n_tiles > 0) {
    QK::load_k(p, b, h, kvh, 0, smem, wave, lane);
    load_v<DV>(p, b, kvh, 0, smem + KPART, wave, lane);
  }

  const int g = lane >> 4, i16 = lane & 15;
  for (int t = 0; t < n_tiles; t++) {
    FA_LDS char* cur = smem + (t & 1) * STAGE;
    wait_vmcnt<0>();
    barrier();
    if (t + 1 < n_tiles) {
      FA_LDS char* nxt = smem + ((t + 1) & 1) * STAGE;
      QK::load_k(p, b, h, kvh, (t + 1) * BN, nxt, wave, lane);
      load_v<DV>(p, b, kvh, (t + 1) * BN, nxt + KPART, wave, lane);
    }
    if (t >= wave_tiles) continue;

    f32x16_t s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; kb++) QK::scores(qf, cur, kb, l32, hl, s[kb], has_ks);

    if (t >= mask_from) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const int key = t * BN + 32 * kb + 8 * (v >> 2) + 4 * hl + (v & 3);
          const bool vis = key < p.Skv && (!CAUSAL || key <= qrow + off);
          s[kb][v] = vis ? s[kb][v] : -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
      for (int v = 0; v < 16; v++) mx = fmaxf(mx, s[kb][v]);
    mx = xor32_max(mx);
    float neg;
    const float alpha = softmax_rescale(st, mx, c, neg);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const float e = exp2_fast(fmaf(s[kb][v], c, neg));
        s[kb][v] = e;
        rs += e;
      }
    st.l = st.l * alpha + rs;
#pragma unroll
    for (int d = 0; d < DV / 32; d++) o[d] *= alpha;

    // O^T += V^T . P^T
    const FA_LDS char* vt = cur + KPART;
#pragma unroll
    for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
      for (int tp = 0; tp < 2; tp++) {
        const i32x4_t pb = {pack_bf16(s[kb][8 * tp + 0], s[kb][8 * tp + 1]), pack_bf16(s[kb][8 * tp + 2], s[kb][8 * tp + 3]),
                            pack_bf16(s[kb][8 * tp + 4], s[kb][8 * tp + 5]), pack_bf16(s[kb][8 * tp + 6], s[kb][8 * tp + 7])};
        const int row0 = 32 * kb + 16 * tp + 4 * (g >> 1) + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < DV / 32; db++) {
          const int col = 32 * db + 16 * (g & 1) + 4 * (i16 & 3);
          i32x2_t part[2];
#pragma unroll
          for (int u = 0; u < 2; u++) {
            const int row = row0 + 8 * u;
            const uint32_t sw = DV == 128 ? swz256(row) : swz_half(row);
            part[u] = lds_tr16(vt + row * VROWB + ((((uint32_t)col >> 3) ^ sw) << 4) + (((col >> 2) & 1) << 3));
          }
          o[db] = mfma32x32x16_bf16(cat(part[0], part[1]), pb, o[db]);
        }
      }
  }

  // epilogue: O = O^T / l, LSE = m * scale + ln l
  const float l_tot = xor32_sum(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < p.Sq) {
    char* ob = (char*)p.o + (((size_t)b * p.Sq + qrow) * p.Hq + h) * (size_t)VROWB;
#pragma unroll
    for (int db = 0; db < DV / 32; db++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int d = 32 * db + 8 * j + 4 * hl;
        i32x2_t w = {pack_bf16(o[db][4 * j] * inv, o[db][4 * j + 1] * inv), pack_bf16(o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv)};
        *(i32x2_t*)(ob + d * 2) = w;
      }
    if (p.lse && hl == 0)
      p.lse[((size_t)b * p.Hq + h) * p.Sq + qrow] = l_tot > 0.f ? st.m * p.scale + logf(l_tot) : -INFINITY;
  }
}

// ------------------------------------------------------------------------------------
// fp32 prefill: v_mfma_f32_32x32x2_f32 for both products, K/V tiles of 32 keys staged
// through LDS with ordinary loads (one stage).  S^T MFMA number c contracts head-dim
// columns c (lanes 0-31) and c + D/2 (lanes 32-63).

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs p, int n_qblocks) {
  constexpr int BNF = 32, LD = D + 4;
  __shared__ float kt[BNF][LD];
  __shared__ float vt[BNF][LD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
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

int grid_of(const PrefillArgs& a, int& n_qblocks) {
  n_qblocks = (a.Sq + BM - 1) / BM;
  return n_qblocks * a.B * a.Hq;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int D, hipStream_t s) {
  int nqb;
  const int grid = grid_of(a, nqb);
  if (grid == 0) return hipSuccess;
  if (D == 128) {
    if (a.causal) prefill_kernel<QkBf16<128>, 128, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_kernel<QkBf16<128>, 128, false><<<grid, 256, 0, s>>>(a, nqb);
  } else {
    if (a.causal) prefill_kernel<QkBf16<64>, 64, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_kernel<QkBf16<64>, 64, false><<<grid, 256, 0, s>>>(a, nqb);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, int D, hipStream_t s) {
  int nqb;
  const int grid = grid_of(a, nqb);
  if (grid == 0) return hipSuccess;
  if (D == 128) {
    if (a.causal) prefill_f32_kernel<128, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_f32_kernel<128, false><<<grid, 256, 0, s>>>(a, nqb);
  } else {
    if (a.causal) prefill_f32_kernel<64, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_f32_kernel<64, false><<<grid, 256, 0, s>>>(a, nqb);
  }
  return hipGetLastError();
}

hipError_t launch_mla_prefill(const PrefillArgs& a, bool nope_fp8, hipStream_t s) {
  int nqb;
  const int grid = grid_of(a, nqb);
  if (grid == 0) return hipSuccess;
  if (nope_fp8) {
    if (a.causal) prefill_kernel<QkMla<true>, 128, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_kernel<QkMla<true>, 128, false><<<grid, 256, 0, s>>>(a, nqb);
  } else {
    if (a.causal) prefill_kernel<QkMla<false>, 128, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_kernel<QkMla<false>, 128, false><<<grid, 256, 0, s>>>(a, nqb);
  }
  return hipGetLastError();
}

}  // namespace fa
