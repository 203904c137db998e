// GQA decode split kernels (bf16 and e4m3 caches, head dim 64 or 128): the split half of
// split-KV decode; decode.hip holds the combine and the launcher that runs both.
//
// The AMD "buffers" page gives its K/V tile buffers a token_gen variant; Modular's
// "KVPipelineGeneric" page pipelines K/V tiles through S = Q.K' and O += P.V.  With one query
// token per sequence there is no query-row parallelism to fill the GPU, so the KV range of each
// sequence is cut into splits processed by independent waves; each writes (row max m, row sum l,
// unnormalised O) for the combine.  Both products use v_mfma_f32_16x16x32_bf16 in transposed
// form (S^T = K.Q^T and O^T = V^T.P^T); the 16 MFMA columns hold the Hq/Hkv query heads of a
// GQA group.
//
// This file is compiled with the matrix-core accumulators in ordinary vector registers
// (-mllvm -amdgpu-mfma-vgpr-form): the kernels need under 160 registers, and with the
// accumulators in AGPRs the compiler moved them through vector registers around every softmax
// step (1.3-1.8 % slower).
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int TK = kDecodeTileKeys;  // keys per tile

// Work item of a GQA split kernel (one wave = one split of one (batch, kv head)).  The grid
// is 1-D; workgroup i runs on XCD i % 8.  The Hkv waves of one (split, batch) pair take
// consecutive positions on one XCD, so each token's kv-head rows -- adjacent in the cache --
// are read together through that XCD's L2 (one 128-byte e4m3 row per head would otherwise
// be fetched by eight XCDs apart).  Pair (split, b) runs on XCD (split + b) % 8, splits in
// order: every sequence's splits spread over all XCDs and early (full) splits go first.
// Batch entries are padded to a multiple of 8; items past B exit.
__device__ __forceinline__ bool gqa_item(const DecodeArgs& a, int& kvh, int& split, int& b) {
  const int i = blockIdx.x, x = i & 7, j = i >> 3;
  kvh = j % a.Hkv;
  const int gi = j / a.Hkv, nb8 = (a.B + 7) / 8;
  split = gi / nb8;
  b = ((x - split) & 7) + 8 * (gi % nb8);
  return b < a.B;
}

// ------------------------------------------------------------------------------------
// GQA decode split: one wave per workgroup = one split of one (batch, kv head).  K and V
// tiles of 32 keys go HBM -> LDS by direct loads into a private ring of GQA_NS stages (no
// barriers: the wave is alone in its workgroup).  Each copy instruction reads whole cache
// rows that nothing reads again, so the copies carry the non-temporal policy (kStream).
// Every LDS read of a tile is an asm block
// that waits for itself (lds_* in device.h), so no instruction the compiler sees consumes
// a load result inside the loop: the only vector-memory waits are the explicit ones, and
// GQA_NS - 1 tiles stay in flight while a tile is computed.  In the last GQA_NS - 1 steps
// no tile is left to issue, and each waits for exactly the copies of the tiles still younger
// than its own, so no copy is ever in flight into a stage being read.  Head dim D = 128 or 64.

constexpr int GQA_NS = 4;  // LDS stages per wave

// s_waitcnt vmcnt(younger * OPS): tile t has landed when at most the copies of the `younger`
// tiles issued after it are still in flight (0 <= younger < GQA_NS; vector-memory loads
// complete in order)
template <int OPS>
__device__ __forceinline__ void wait_tile(int younger) {
  static_assert(GQA_NS == 4, "one case per count of younger tiles");
  switch (younger) {
    case 3: wait_vmcnt<3 * OPS>(); break;
    case 2: wait_vmcnt<2 * OPS>(); break;
    case 1: wait_vmcnt<OPS>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// 16-byte chunk swizzles of the GQA tiles not covered by device.h:
//  * bf16 rows of 128 bytes (D = 64) alternate bank halves by parity.  With t = (row / 2) % 8,
//    the 16 rows of an S^T A-operand read need an XOR one-to-one over t, and the 8 rows read
//    together by a transposing V read (32 lanes: rows 8k .. 8k+7) need distinct chunk pairs
//    (xor >> 1) over t % 4 within each parity: ((t % 4) << 1) | (t / 4) is both.
//  * e4m3 rows of 64 bytes (D = 64) put four rows in a bank row.  The 16 rows of an S^T read
//    (rows 16kb .. 16kb+15) and the 16 rows of a transposing V read pass (row / 4 in {0, 1, 4, 5}
//    or {2, 3, 6, 7}) both need an XOR one-to-one over row / 4 within each class of row % 4:
//    ((row / 4) % 4) ^ (2 * ((row / 16) % 2)) is.
__device__ __forceinline__ uint32_t swz_b64(uint32_t row) {
  const uint32_t t = (row >> 1) & 7u;
  return ((t & 3u) << 1) | (t >> 2);
}
__device__ __forceinline__ uint32_t swz_q64(uint32_t row) { return ((row >> 2) & 3u) ^ ((row >> 3) & 2u); }

template <int D>
__device__ __forceinline__ uint32_t gqa_swz_bf16(uint32_t row) {
  return D == 128 ? swz16(row) : swz_b64(row);
}

template <int D, int G>
__global__ __launch_bounds__(64) void gqa_decode_split(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int ROWB = 2 * D, TILE = TK * ROWB;     // K or V tile: 8 KiB (D = 128), 4 KiB (D = 64)
  constexpr int STAGE = 2 * TILE;                   // K tile | V tile
  constexpr int NCP = TILE / 1024;                  // direct copies per K or V tile
  constexpr int OPS = 2 * NCP;                      // direct copies per tile
  constexpr int RPI = 1024 / ROWB, CPR = ROWB / 16; // rows per copy instruction, chunks per row
  constexpr int NC = D / 32;                        // S^T contraction steps
  constexpr int NB = D / 16;                        // 16-column blocks of O^T
  __shared__ __attribute__((aligned(1024))) char ring_raw[GQA_NS * STAGE];
  FA_LDS char* const ring = (FA_LDS char*)ring_raw;

  int kvh, split, b;
  if (!gqa_item(a, kvh, split, b)) return;
  const int L = min(max(a.kv_lens[b], 0), a.max_len);
  const int start = split * a.chunk;
  if (start >= L) return;
  const int end = min(start + a.chunk, L);
  const int n_tiles = (end - start + TK - 1) / TK;

  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;
  const float c = a.scale * kLog2e;
  const uint32_t rstride = (uint32_t)a.Hkv * ROWB;  // bytes between consecutive keys

  // Q^T as the B operand: column l16 = query head kvh*G + l16 (zero past the group),
  // k = head-dim 32cc + 8g .. +7
  i32x4_t qf[NC];
  {
    const int hq = kvh * G + (l16 < G ? l16 : 0);
    const char* qp = (const char*)a.q + ((size_t)b * a.Hq + hq) * ROWB;
#pragma unroll
    for (int cc = 0; cc < NC; cc++) {
      const i32x4_t x = *(const i32x4_t*)(qp + cc * 64 + g * 16);
      qf[cc] = l16 < G ? x : i32x4_t{};
    }
  }
  const char* kbase = (const char*)a.k + ((size_t)b * a.max_len * a.Hkv + kvh) * ROWB;
  const char* vbase = (const char*)a.v + ((size_t)b * a.max_len * a.Hkv + kvh) * ROWB;
  // direct copy: LDS row RPI*i + lane/CPR holds that key row with its 16-byte chunks
  // XOR-permuted
  uint32_t coff[NCP];
#pragma unroll
  for (int i = 0; i < NCP; i++) {
    const uint32_t row = RPI * i + lane / CPR;
    coff[i] = row * rstride + (((lane % CPR) ^ gqa_swz_bf16<D>(row)) << 4);
  }
  // S^T A operand of key block kb, step cc: row 16kb + l16, chunk 4cc + g
  uint32_t ka[2 * NC];
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int cc = 0; cc < NC; cc++) {
      const uint32_t row = 16 * kb + l16;
      ka[NC * kb + cc] = row * ROWB + (((4 * cc + g) ^ gqa_swz_bf16<D>(row)) << 4);
    }
  // transposing V reads: rows 16u + 4g + l16/4, columns 16db + 4(l16%4) .. +3, i.e. chunk
  // 2db + (l16%4)/2 of the row (before the XOR), byte 8(l16%2) of the chunk
  uint32_t va[NB][2];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const uint32_t row = 16 * u + 4 * g + (l16 >> 2), sw = gqa_swz_bf16<D>(row);
#pragma unroll
    for (int db = 0; db < NB; db++)
      va[db][u] = TILE + row * ROWB + (((2 * db + ((l16 & 3) >> 1)) ^ sw) << 4) + ((l16 & 1) << 3);
  }

  // tile t -> stage t % GQA_NS; rows past the sequence repeat its last row (masked below)
  auto issue = [&](int t) {
    const int key0 = start + t * TK, valid = min(TK, end - key0);
    FA_LDS char* dst = ring + (t % GQA_NS) * STAGE;
    const uint32_t bytes = (uint32_t)(valid - 1) * rstride + ROWB;
    const auto rk = make_rsrc(kbase + (size_t)key0 * rstride, bytes);
    const auto rv = make_rsrc(vbase + (size_t)key0 * rstride, bytes);
    if (valid == TK) {
#pragma unroll
      for (int i = 0; i < NCP; i++) dma16_buf<kStream>(rk, dst + i * 1024, coff[i]);
#pragma unroll
      for (int i = 0; i < NCP; i++) dma16_buf<kStream>(rv, dst + TILE + i * 1024, coff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NCP; i++) {
        const uint32_t row = RPI * i + lane / CPR, rc = min(row, (uint32_t)(valid - 1));
        const uint32_t off = rc * rstride + (((lane % CPR) ^ gqa_swz_bf16<D>(row)) << 4);
        dma16_buf<kStream>(rk, dst + i * 1024, off);
        dma16_buf<kStream>(rv, dst + TILE + i * 1024, off);
      }
    }
  };

  float m_ref = -INFINITY, neg = 0.f, l = 0.f;
  f32x4_t o[NB];
#pragma unroll
  for (int d = 0; d < NB; d++) o[d] = f32x4_t{};

  // prologue: tiles 0 .. GQA_NS-2; then every step issues tile t + GQA_NS - 1 while there is
  // one, so min(GQA_NS - 1, n_tiles - 1 - t) tiles of copies are younger than tile t's
#pragma unroll
  for (int p = 0; p < GQA_NS - 1; p++)
    if (p < n_tiles) issue(p);
  for (int t = 0; t < n_tiles; t++) {
    // the stage refilled here held tile t - 1, whose reads completed in their asm blocks
    if (t + GQA_NS - 1 < n_tiles) {
      issue(t + GQA_NS - 1);
      wait_vmcnt<(GQA_NS - 1) * OPS>();
    } else {
      wait_tile<OPS>(n_tiles - 1 - t);
    }
    asm volatile("" ::: "memory");
    const uint32_t st = lds_addr(ring) + (t % GQA_NS) * STAGE;

    i32x4_t kf[2 * NC];
    {
      uint32_t ad[2 * NC];
#pragma unroll
      for (int i = 0; i < 2 * NC; i++) ad[i] = st + ka[i];
      if constexpr (NC == 4) lds_b128_x8(kf, ad);
      else lds_b128_x4(kf, ad);
    }
    f32x4_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      s[kb] = f32x4_t{};
#pragma unroll
      for (int cc = 0; cc < NC; cc++) s[kb] = mfma16x16x32_bf16(kf[NC * kb + cc], qf[cc], s[kb]);
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
    if (__builtin_amdgcn_ballot_w64(mx * c > m_ref * c + 8.f)) {  // lazy rescale (P <= 2^8)
      const float m_new = fmaxf(m_ref, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast((m_ref - m_use) * c);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < NB; d++) o[d] *= alpha;
      m_ref = m_new;
      neg = -m_use * c;
    }
    float e[8];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int v = 0; v < 4; v++) e[4 * kb + v] = exp2_fast(fmaf(s[kb][v], c, neg));
    const i32x4_t pb = {pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]), pack_bf16(e[4], e[5]), pack_bf16(e[6], e[7])};
#pragma unroll
    for (int i = 0; i < 4; i++) l = dot2_bf16(pb[i], kBf16PairOne, l);
#pragma unroll
    for (int half = 0; half < NB / 4; half++) {
      uint32_t ad[8];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        ad[2 * j] = st + va[4 * half + j][0];
        ad[2 * j + 1] = st + va[4 * half + j][1];
      }
      i32x2_t vr[8];
      lds_tr16_x8(vr, ad);
#pragma unroll
      for (int j = 0; j < 4; j++)
        o[4 * half + j] = mfma16x16x32_bf16(cat(vr[2 * j], vr[2 * j + 1]), pb, o[4 * half + j]);
    }
  }

  const float l_tot = xor32_sum(xor16_sum(l));
  if (l16 < G) {
    const int hq = kvh * G + l16;
    const size_t pidx = ((size_t)b * a.Hq + hq) * a.n_split + split;
    float* po = a.part_o + pidx * D;
#pragma unroll
    for (int db = 0; db < NB; db++) *(f32x4_t*)(po + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      a.part_ml[2 * pidx] = m_ref;
      a.part_ml[2 * pidx + 1] = l_tot;
    }
  }
}

// ------------------------------------------------------------------------------------
// GQA decode split over an e4m3 cache with per-token scales (k_scale, v_scale per key row
// and kv head).  Same structure as the bf16 kernel, at half the bytes per key:
//  * K codes go through the LDS ring; the contraction order is permuted so that a lane's K
//    fragments are one contiguous run of its key row (step cc, lane group g, element i covers
//    head dim (D/4)g + 8cc + i; Q^T uses the same order), and e4m3 -> bf16 is exact, so
//    S^T = K_code.Q^T runs on the bf16 matrix cores and the key scale multiplies S afterwards;
//  * V codes are read transposed one byte wide (ds_read_b64_tr_b8: 8 keys of one column per
//    lane, one read per product instead of two), converted exactly, and the value scale is
//    folded into P: O += (P . v_scale) V_code.

template <int D>
__device__ __forceinline__ uint32_t gqa_swz_k8(uint32_t row) {
  return D == 128 ? swz_half(row) : swz_q64(row);
}
template <int D>
__device__ __forceinline__ uint32_t gqa_swz_v8(uint32_t row) {
  return D == 128 ? swz_fp8v(row) : swz_q64(row);
}

template <int D, int G>
__global__ __launch_bounds__(64) void gqa_decode_split_fp8(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int ROWB = D, TILE = TK * ROWB;         // 4 KiB (D = 128), 2 KiB (D = 64) per K or V tile
  constexpr int SCB = 256;                          // one scale copy: 64 lanes x 4 bytes
  constexpr int STAGE = 2 * TILE + 2 * SCB;         // K codes | V codes | k_scale | v_scale
  constexpr int NCP = TILE / 1024;                  // direct copies per K or V tile
  constexpr int OPS = 2 * NCP + 2;                  // direct copies per tile
  constexpr int RPI = 1024 / ROWB, CPR = ROWB / 16; // rows per copy instruction, chunks per row
  constexpr int KCH = D / 64;                       // 16-byte K reads per lane per 16-key block
  constexpr int NC = D / 32;                        // S^T contraction steps
  constexpr int NB = D / 16;                        // 16-column blocks of O^T
  __shared__ __attribute__((aligned(1024))) char ring_raw[GQA_NS * STAGE];
  FA_LDS char* const ring = (FA_LDS char*)ring_raw;

  int kvh, split, b;
  if (!gqa_item(a, kvh, split, b)) return;
  const int L = min(max(a.kv_lens[b], 0), a.max_len);
  const int start = split * a.chunk;
  if (start >= L) return;
  const int end = min(start + a.chunk, L);
  const int n_tiles = (end - start + TK - 1) / TK;

  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;
  const float c = a.scale * kLog2e;
  const uint32_t rstride = (uint32_t)a.Hkv * ROWB;  // bytes between consecutive keys
  const uint32_t sstride = (uint32_t)a.Hkv * 4;     // scale bytes between consecutive keys

  // Q^T as the B operand: column l16 = query head kvh*G + l16 (zero past the group); step cc
  // holds head dims (D/4)g + 8cc .. +7
  i32x4_t qf[NC];
  {
    const int hq = kvh * G + (l16 < G ? l16 : 0);
    const char* qp = (const char*)a.q + ((size_t)b * a.Hq + hq) * (D * 2);
#pragma unroll
    for (int cc = 0; cc < NC; cc++) {
      const i32x4_t x = *(const i32x4_t*)(qp + ((D / 4) * g + 8 * cc) * 2);
      qf[cc] = l16 < G ? x : i32x4_t{};
    }
  }
  const size_t row0 = (size_t)b * a.max_len * a.Hkv + kvh;  // (batch, key 0, kv head) row index
  const char* kbase = (const char*)a.k + row0 * ROWB;
  const char* vbase = (const char*)a.v + row0 * ROWB;
  const float* ksbase = a.k_scale + row0;
  const float* vsbase = a.v_scale + row0;
  // direct copies: LDS row RPI*i + lane/CPR holds that key row, its 16-byte chunks
  // XOR-permuted by the K and V swizzles
  uint32_t kcoff[NCP], vcoff[NCP];
#pragma unroll
  for (int i = 0; i < NCP; i++) {
    const uint32_t row = RPI * i + lane / CPR;
    kcoff[i] = row * rstride + (((lane % CPR) ^ gqa_swz_k8<D>(row)) << 4);
    vcoff[i] = row * rstride + (((lane % CPR) ^ gqa_swz_v8<D>(row)) << 4);
  }
  // K fragments: key row 16kb + l16, bytes (D/4)g + 16hh .. +15 (chunk KCH*g + hh)
  uint32_t ka[2 * KCH];
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int hh = 0; hh < KCH; hh++) {
      const uint32_t row = 16 * kb + l16;
      ka[KCH * kb + hh] = row * ROWB + (((KCH * g + hh) ^ gqa_swz_k8<D>(row)) << 4);
    }
  // transposing V reads: lane 2e + h of group g reads key row R = 16(e/4) + 4g + e%4 at
  // byte 8h of column chunk db, so output byte e of lane l is column 16db + l%16 of key R --
  // the key order in which P^T is packed below
  uint32_t va[NB];
  {
    const uint32_t e = (lane & 15) >> 1, h = lane & 1;
    const uint32_t row = 16 * (e >> 2) + 4 * g + (e & 3);
#pragma unroll
    for (int db = 0; db < NB; db++) va[db] = TILE + row * ROWB + 8 * h + ((db ^ gqa_swz_v8<D>(row)) << 4);
  }
  // scales of the tile's keys: register v of block kb holds key 16kb + 4g + v
  const uint32_t g16 = 16u * g;
  const uint32_t sa[4] = {2 * TILE + g16, 2 * TILE + 64 + g16, 2 * TILE + SCB + g16, 2 * TILE + SCB + 64 + g16};

  auto issue = [&](int t) {
    const int key0 = start + t * TK, valid = min(TK, end - key0);
    FA_LDS char* dst = ring + (t % GQA_NS) * STAGE;
    const uint32_t bytes = (uint32_t)(valid - 1) * rstride + ROWB;
    const auto rk = make_rsrc(kbase + (size_t)key0 * rstride, bytes);
    const auto rv = make_rsrc(vbase + (size_t)key0 * rstride, bytes);
    if (valid == TK) {
#pragma unroll
      for (int i = 0; i < NCP; i++) dma16_buf<kStream>(rk, dst + i * 1024, kcoff[i]);
#pragma unroll
      for (int i = 0; i < NCP; i++) dma16_buf<kStream>(rv, dst + TILE + i * 1024, vcoff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NCP; i++) {
        const uint32_t row = RPI * i + lane / CPR, rc = min(row, (uint32_t)(valid - 1));
        dma16_buf<kStream>(rk, dst + i * 1024, rc * rstride + (((lane % CPR) ^ gqa_swz_k8<D>(row)) << 4));
        dma16_buf<kStream>(rv, dst + TILE + i * 1024, rc * rstride + (((lane % CPR) ^ gqa_swz_v8<D>(row)) << 4));
      }
    }
    // scales of keys key0 + lane (lanes past the tile repeat its last key); 4 bytes of each
    // key's Hkv scales, the rest read by the other kv heads' waves through L2, so these keep
    // the default cache policy (1.7 % faster than streaming them)
    const uint32_t so = (uint32_t)min(lane, valid - 1) * sstride;
    const uint32_t sbytes = (uint32_t)(valid - 1) * sstride + 4;
    dma4_buf(make_rsrc(ksbase + (size_t)key0 * a.Hkv, sbytes), dst + 2 * TILE, so);
    dma4_buf(make_rsrc(vsbase + (size_t)key0 * a.Hkv, sbytes), dst + 2 * TILE + SCB, so);
  };

  float m_ref = -INFINITY, neg = 0.f, l = 0.f;
  f32x4_t o[NB];
#pragma unroll
  for (int d = 0; d < NB; d++) o[d] = f32x4_t{};

  // same ring discipline as the bf16 kernel: up to GQA_NS - 1 tiles of copies in flight
#pragma unroll
  for (int p = 0; p < GQA_NS - 1; p++)
    if (p < n_tiles) issue(p);
  for (int t = 0; t < n_tiles; t++) {
    if (t + GQA_NS - 1 < n_tiles) {
      issue(t + GQA_NS - 1);
      wait_vmcnt<(GQA_NS - 1) * OPS>();
    } else {
      wait_tile<OPS>(n_tiles - 1 - t);
    }
    asm volatile("" ::: "memory");
    const uint32_t st = lds_addr(ring) + (t % GQA_NS) * STAGE;

    i32x4_t kf[2 * KCH], sc[4];
    {
      constexpr int NR = 2 * KCH + 4;
      uint32_t ad[NR];
#pragma unroll
      for (int i = 0; i < 2 * KCH; i++) ad[i] = st + ka[i];
#pragma unroll
      for (int i = 0; i < 4; i++) ad[2 * KCH + i] = st + sa[i];
      i32x4_t r[NR];
      if constexpr (NR == 8) lds_b128_x8(r, ad);
      else lds_b128_x6(r, ad);
#pragma unroll
      for (int i = 0; i < 2 * KCH; i++) kf[i] = r[i];
#pragma unroll
      for (int i = 0; i < 4; i++) sc[i] = r[2 * KCH + i];
    }
    f32x4_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      s[kb] = f32x4_t{};
#pragma unroll
      for (int hh = 0; hh < KCH; hh++) {
        const i32x4_t w = kf[KCH * kb + hh];
        s[kb] = mfma16x16x32_bf16(e4m3x8_to_bf16(i32x2_t{w.x, w.y}), qf[2 * hh], s[kb]);
        s[kb] = mfma16x16x32_bf16(e4m3x8_to_bf16(i32x2_t{w.z, w.w}), qf[2 * hh + 1], s[kb]);
      }
    }
    const f32x4_t ks0 = __builtin_bit_cast(f32x4_t, sc[0]), ks1 = __builtin_bit_cast(f32x4_t, sc[1]);
    const f32x4_t vs0 = __builtin_bit_cast(f32x4_t, sc[2]), vs1 = __builtin_bit_cast(f32x4_t, sc[3]);
#pragma unroll
    for (int v = 0; v < 4; v++) {
      s[0][v] *= ks0[v];
      s[1][v] *= ks1[v];
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
    if (__builtin_amdgcn_ballot_w64(mx * c > m_ref * c + 8.f)) {  // lazy rescale (P <= 2^8)
      const float m_new = fmaxf(m_ref, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast((m_ref - m_use) * c);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < NB; d++) o[d] *= alpha;
      m_ref = m_new;
      neg = -m_use * c;
    }
    float e[8];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        e[4 * kb + v] = exp2_fast(fmaf(s[kb][v], c, neg));
        l += e[4 * kb + v];
      }
    const i32x4_t pb = {pack_bf16(e[0] * vs0[0], e[1] * vs0[1]), pack_bf16(e[2] * vs0[2], e[3] * vs0[3]),
                        pack_bf16(e[4] * vs1[0], e[5] * vs1[1]), pack_bf16(e[6] * vs1[2], e[7] * vs1[3])};
    i32x2_t vr[NB];
    {
      uint32_t ad[NB];
#pragma unroll
      for (int db = 0; db < NB; db++) ad[db] = st + va[db];
      if constexpr (NB == 8) lds_tr8_x8(vr, ad);
      else lds_tr8_x4(vr, ad);
    }
#pragma unroll
    for (int db = 0; db < NB; db++) o[db] = mfma16x16x32_bf16(e4m3x8_to_bf16(vr[db]), pb, o[db]);
  }

  const float l_tot = xor32_sum(xor16_sum(l));
  if (l16 < G) {
    const int hq = kvh * G + l16;
    const size_t pidx = ((size_t)b * a.Hq + hq) * a.n_split + split;
    float* po = a.part_o + pidx * D;
#pragma unroll
    for (int db = 0; db < NB; db++) *(f32x4_t*)(po + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      a.part_ml[2 * pidx] = m_ref;
      a.part_ml[2 * pidx + 1] = l_tot;
    }
  }
}

}  // namespace

template <int D>
hipError_t launch_gqa_split(const DecodeArgs& a, bool fp8, int grid, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
#define FA_G(n)                                                     \
  case n:                                                           \
    if (fp8) gqa_decode_split_fp8<D, n><<<grid, 64, 0, s>>>(a);     \
    else gqa_decode_split<D, n><<<grid, 64, 0, s>>>(a);             \
    break;
    FA_G(1) FA_G(2) FA_G(3) FA_G(4) FA_G(5) FA_G(6) FA_G(7) FA_G(8)
    FA_G(9) FA_G(10) FA_G(11) FA_G(12) FA_G(13) FA_G(14) FA_G(15) FA_G(16)
#undef FA_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gqa_split_kernels(const DecodeArgs& a, int D, bool fp8, hipStream_t s) {
  const int grid = a.n_split * ((a.B + 7) / 8 * 8) * a.Hkv;  // see gqa_item
  return D == 128 ? launch_gqa_split<128>(a, fp8, grid, s)
       : D == 64  ? launch_gqa_split<64>(a, fp8, grid, s)
                  : hipErrorInvalidValue;
}

}  // namespace fa
