// Prefill forward kernels on bf16 matrix cores: MHA / GQA (bf16 q/k/v) and MLA with
// per-token scales (e4m3 or bf16 nope part, bf16 rope part, bf16 V or e4m3 V with per-row
// scales).
//
// Method: the flash-attention forward that Modular's "KVPipelineGeneric" page describes
// (S = Q.K' and O += P.V per K/V tile over a pipeline of K/V stages), with the online
// softmax whose per-row correction the "MLASmemStorage" page keeps in a correction
// buffer; here the correction stays in the lane that owns the row.  The AMD "buffers"
// page's roles map as follows: QRegisterBuffer -> Q fragments in VGPRs for the whole
// block; KBufferLDS / KVBufferLDS (direct DRAM->LDS, no register staging) ->
// buffer_load ... lds into a swizzled two-stage LDS ring; VBufferTransposeLoads ->
// ds_read_b64_tr_b16; PRegisterBuffer -> P packed to bf16 in VGPRs straight from the S^T
// accumulators; OutputRegisterBuffer -> O^T accumulators.
//
// Workgroup: NW waves, query blocks of 32 * NW rows (32 per wave), K/V tiles of BN = 64
// keys; NW = 4 (two workgroups per CU), or 8 (one workgroup per CU, sharing each K/V tile
// between twice the rows) for long causal bf16 prefills of head dim 128.  Causal
// workgroups take a pair of query blocks (i, n-1-i), so every workgroup has the same
// number of key tiles; workgroups are ordered head-major within each XCD (the
// dispatcher deals workgroups to the 8 XCDs round-robin), so the workgroups of one
// (batch, head) run together and share its K/V through that XCD's L2.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int BN = 64;
// Lazy rescaling: the running reference max only moves when a row max exceeds it by more
// than 8 (log2 units), so P values stay <= 2^8; O and l share the reference, so O / l is
// unchanged and most tiles skip the rescale.
constexpr float kRescaleLog2 = 8.f;

template <int ROWB>
__device__ __forceinline__ uint32_t swz_rows(uint32_t row) {
  static_assert(ROWB == 256 || ROWB == 128, "row size");
  return ROWB == 256 ? swz256(row) : swz_half(row);
}

// A tile of BN rows of ROWB bytes copied global -> LDS by the NW waves of the workgroup with
// 16-byte direct loads.  LDS row r holds tile row r with its chunks XOR-permuted by
// swz_rows(r): each lane fetches the global chunk that belongs at its LDS slot.  Per-lane
// source offsets are computed once; a tile costs one instruction per wave per KiB.
// 16-byte chunk swizzle of an e4m3 V tile (128-byte rows): the transposing byte reads of a
// half-wave cover the rows {r, r+1, r+2, r+3, r+8, .., r+11} (r = 0 or 4, the key order of
// P^T) at two adjacent chunks; rows alternate bank halves by parity, and XOR-ing the chunk
// with 2 * (bit 1 of the row | bit 3 of the row << 1) puts the 4 rows of each parity at the
// two chunks on 8 distinct 16-byte slots of their half, so the half-wave reads all 64 banks
// once.
__device__ __forceinline__ uint32_t swz_v8(uint32_t row) { return (((row >> 1) & 1u) | ((row >> 2) & 2u)) << 1; }

template <int ROWB>
struct DefaultSwz {
  __device__ __forceinline__ static uint32_t f(uint32_t row) { return swz_rows<ROWB>(row); }
};
struct SwzV8 {
  __device__ __forceinline__ static uint32_t f(uint32_t row) { return swz_v8(row); }
};

template <int ROWB, class SWZ = DefaultSwz<ROWB>, int NW = 4>
struct RowDma {
  static constexpr int RPI = 1024 / ROWB;           // rows per wave instruction
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int NI = BN * ROWB / 1024 / NW;  // instructions per wave per tile
  static_assert(NI >= 1, "tile too small");
  uint32_t voff[NI];

  __device__ __forceinline__ void init(int wave, int lane, uint32_t stride) {
#pragma unroll
    for (int i = 0; i < NI; i++) {
      const uint32_t row = (i * NW + wave) * RPI + lane / CPR;
      voff[i] = row * stride + ((((uint32_t)lane % CPR) ^ SWZ::f(row)) << 4);
    }
  }
  // Rows [0, valid) of the tile start at `base`, `stride` bytes apart; LDS rows at or past
  // `valid` receive a copy of row valid - 1 (never read as keys: they are masked).
  __device__ __forceinline__ void issue(const char* base, uint32_t stride, int valid, FA_LDS char* dst, int wave,
                                        int lane) const {
    const auto r = make_rsrc(base, (uint32_t)(valid - 1) * stride + ROWB);
    if (valid >= BN) {
#pragma unroll
      for (int i = 0; i < NI; i++) dma16_buf(r, dst + (i * NW + wave) * 1024, voff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NI; i++) {
        const uint32_t row = (i * NW + wave) * RPI + lane / CPR;
        const uint32_t rc = min(row, (uint32_t)(valid - 1));
        dma16_buf(r, dst + (i * NW + wave) * 1024, rc * stride + ((((uint32_t)lane % CPR) ^ SWZ::f(row)) << 4));
      }
    }
  }
};

// ------------------------------------------------------------------------------------
// Q.K^T policies: Q in registers, the K part of an LDS stage, one 32-key block of S^T.

// MHA / GQA: bf16 q/k of head dim D.
template <int D, int NW_ = 4>
struct QkBf16 {
  static constexpr int NW = NW_;  // waves of the workgroup that share the copies
  static constexpr bool REV_SECOND = false;  // key order of a causal pair's second block
  static constexpr bool STAGE_O = false;     // O rows staged through LDS for whole-row stores
  static constexpr int ROWB = D * 2;
  static constexpr int KBYTES = BN * ROWB;
  struct QFrag {
    i32x4_t c[D / 16];
  };
  struct Lane {
    RowDma<ROWB, DefaultSwz<ROWB>, NW> dma;
    uint32_t ka[D / 16];  // LDS offset of this lane's K chunk for MFMA step c (block 0)
  };

  __device__ static void init(const PrefillArgs& p, int wave, int lane, Lane& s) {
    s.dma.init(wave, lane, p.Hkv * ROWB);
    const uint32_t l32 = lane & 31, hl = lane >> 5, sw = swz_rows<ROWB>(l32);
#pragma unroll
    for (int c = 0; c < D / 16; c++) s.ka[c] = l32 * ROWB + (((2 * c + hl) ^ sw) << 4);
  }
  __device__ static void load_q(const PrefillArgs& p, int b, int h, int qrow, int hl, QFrag& q) {
    const char* base = (const char*)p.q + (((size_t)b * p.Sq + qrow) * p.Hq + h) * (size_t)ROWB;
#pragma unroll
    for (int c = 0; c < D / 16; c++) q.c[c] = *(const i32x4_t*)(base + c * 32 + hl * 16);
  }
  __device__ static void issue(const PrefillArgs& p, const Lane& s, int b, int h, int kvh, int key0, FA_LDS char* dst,
                               int wave, int lane) {
    (void)h;
    const char* base = (const char*)p.k + (((size_t)b * p.Skv + key0) * p.Hkv + kvh) * (size_t)ROWB;
    s.dma.issue(base, p.Hkv * ROWB, min(BN, p.Skv - key0), dst, wave, lane);
  }
  __device__ static void scores(const QFrag& q, const Lane& s, const FA_LDS char* stage, int kb, int hl,
                                f32x16_t& acc, bool /*has_kscale*/) {
    (void)hl;
    acc = f32x16_t{};
#pragma unroll
    for (int c = 0; c < D / 16; c++) acc = mfma32x32x16_bf16(lds_b128(stage + s.ka[c] + kb * 32 * ROWB), q.c[c], acc);
  }
};

// MLA prefill with per-token scales: nope (Dn = 128) in e4m3 or bf16, rope (Dr = 64) bf16
// with Hr rope heads, fp32 q_scale per query row and k_scale per key.
// K part of a stage: k_nope [BN][Dn] | k_rope [BN][64] bf16 | k_scale [BN] fp32.
template <bool FP8, int NW_ = 4>
struct QkMla {
  static constexpr int NW = NW_;  // waves of the workgroup that share the copies
  static constexpr bool REV_SECOND = true;  // key order of a causal pair's second block
  static constexpr bool STAGE_O = FP8;      // O rows staged through LDS for whole-row stores
  static constexpr int NROWB = FP8 ? 128 : 256;
  static constexpr int KN = 0;
  static constexpr int KR = BN * NROWB;
  static constexpr int KS = KR + BN * 128;
  static constexpr int KBYTES = KS + BN * 4;
  static constexpr int NNA = FP8 ? 4 : 8;
  struct QFrag {
    i32x8_t n8[FP8 ? 2 : 1];  // e4m3: 2 MFMA steps of 32 bytes per lane
    i32x4_t n16[FP8 ? 1 : 8];
    i32x4_t r[4];
    float qs;
  };
  struct Lane {
    RowDma<NROWB, DefaultSwz<NROWB>, NW> ndma;
    RowDma<128, DefaultSwz<128>, NW> rdma;
    uint32_t na[NNA];  // nope chunk offsets
    uint32_t ra[4];    // rope chunk offsets
    uint32_t sa;       // k_scale offset of this lane's first key
    uint32_t sf;       // k_scale offset of key l32 of a 32-key block
  };

  __device__ static void init(const PrefillArgs& p, int wave, int lane, Lane& s) {
    s.ndma.init(wave, lane, p.Hq * NROWB);
    s.rdma.init(wave, lane, p.Hr * 128);
    const uint32_t l32 = lane & 31, hl = lane >> 5;
    if constexpr (FP8) {
      const uint32_t sw = swz_half(l32);
#pragma unroll
      for (int c = 0; c < 2; c++)
#pragma unroll
        for (int e = 0; e < 2; e++) s.na[2 * c + e] = KN + l32 * 128 + (((4 * c + 2 * hl + e) ^ sw) << 4);
    } else {
      const uint32_t sw = swz256(l32);
#pragma unroll
      for (int c = 0; c < 8; c++) s.na[c] = KN + l32 * 256 + (((2 * c + hl) ^ sw) << 4);
    }
    const uint32_t swr = swz_half(l32);
#pragma unroll
    for (int c = 0; c < 4; c++) s.ra[c] = KR + l32 * 128 + (((2 * c + hl) ^ swr) << 4);
    s.sa = KS + 16 * hl;
    s.sf = KS + 4 * l32;
  }
  __device__ static void load_q(const PrefillArgs& p, int b, int h, int qrow, int hl, QFrag& q) {
    const size_t tok = ((size_t)b * p.Sq + qrow) * p.Hq + h;
    const char* n = (const char*)p.q + tok * NROWB;
    if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < 2; c++) {
        const i32x4_t lo = *(const i32x4_t*)(n + c * 64 + hl * 32);
        const i32x4_t hi = *(const i32x4_t*)(n + c * 64 + hl * 32 + 16);
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
  __device__ static void issue(const PrefillArgs& p, const Lane& s, int b, int h, int kvh, int key0, FA_LDS char* dst,
                               int wave, int lane) {
    (void)kvh;
    const int valid = min(BN, p.Skv - key0);
    s.ndma.issue((const char*)p.k + (((size_t)b * p.Skv + key0) * p.Hq + h) * (size_t)NROWB, p.Hq * NROWB, valid,
                 dst + KN, wave, lane);
    const int hr = p.Hr == 1 ? 0 : h;
    s.rdma.issue((const char*)p.k_rope + (((size_t)b * p.Skv + key0) * p.Hr + hr) * 128, p.Hr * 128, valid, dst + KR,
                 wave, lane);
    if (p.k_scale && wave == 0) {
      const float* base = p.k_scale + ((size_t)b * p.Skv + key0) * p.Hq + h;
      const auto r = make_rsrc(base, (uint32_t)((valid - 1) * p.Hq + 1) * 4);
      dma4_buf(r, dst + KS, (uint32_t)min(lane, valid - 1) * p.Hq * 4);
    }
  }
  __device__ static void scores(const QFrag& q, const Lane& s, const FA_LDS char* stage, int kb, int hl,
                                f32x16_t& acc, bool has_kscale) {
    // F = k_scale (x) q_scale over the block's 32 keys and 32 rows, in the S^T accumulator
    // layout, by one fp32 outer-product MFMA (the lanes of half 0 give the key scales and the
    // row scale, those of half 1 zeros): one rounding per product, as q_scale * k_scale on the
    // vector ALU, without its 16 multiplies and four scale reads
    const float kv = has_kscale ? *(const FA_LDS float*)(stage + s.sf + kb * 128) : 1.f;
    const f32x16_t f = mfma32x32x2_f32(hl ? 0.f : kv, hl ? 0.f : q.qs, f32x16_t{});
    f32x16_t sn{};
    if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < 2; c++) {
        const i32x4_t lo = lds_b128(stage + s.na[2 * c] + kb * 32 * NROWB);
        const i32x4_t hi = lds_b128(stage + s.na[2 * c + 1] + kb * 32 * NROWB);
        sn = mfma32x32x64_e4m3(i32x8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, q.n8[c], sn);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; c++) sn = mfma32x32x16_bf16(lds_b128(stage + s.na[c] + kb * 32 * NROWB), q.n16[c], sn);
    }
    // the nope product scaled in place, then the rope products accumulate onto it
#pragma unroll
    for (int v = 0; v < 16; v++) sn[v] *= f[v];
#pragma unroll
    for (int c = 0; c < 4; c++) sn = mfma32x32x16_bf16(lds_b128(stage + s.ra[c] + kb * 32 * 128), q.r[c], sn);
    acc = sn;
  }
};

// ------------------------------------------------------------------------------------
// Per-row running state and the per-tile step.

template <int DV>
struct RowAcc {
  f32x16_t o[DV / 32];  // O^T: register v of block db holds d = 32db + 8(v/4) + 4hl + v%4
  float m_ref;          // reference max of the raw scores (-inf before the first visible key)
  float neg;            // -max(m_ref, 0 if -inf) * c
  float l;              // lane-partial sum of the bf16-rounded P of this lane's keys
};

// S^T of one K tile (all BN/32 key blocks).
template <class QK>
__device__ __forceinline__ void tile_scores(f32x16_t (&s)[BN / 32], const typename QK::QFrag& q,
                                            const typename QK::Lane& ks, const FA_LDS char* kst, int hl, bool has_ks) {
#pragma unroll
  for (int kb = 0; kb < BN / 32; kb++) QK::scores(q, ks, kst, kb, hl, s[kb], has_ks);
}

// ------------------------------------------------------------------------------------
// V policies: the V part of an LDS stage, its copy, the per-key factor folded into P, and
// O^T += V^T . P^T over one tile.

// bf16 V (rows of DV bf16), read transposed two bytes wide.
template <int DV_, int NW_ = 4>
struct VBf16 {
  static constexpr int NW = NW_;
  static constexpr int DV = DV_;
  static constexpr int ROWB = DV * 2;
  static constexpr int BYTES = BN * ROWB;
  static constexpr bool SCALED = false;
  struct Lane {
    RowDma<ROWB, DefaultSwz<ROWB>, NW> dma;
    uint32_t va[2][DV / 32];
  };
  __device__ static void init(const PrefillArgs& p, int wave, int lane, Lane& s) {
    s.dma.init(wave, lane, p.Hkv * ROWB);
    const uint32_t g = lane >> 4, i16 = lane & 15;
    const uint32_t row0 = 4 * (g >> 1) + (i16 >> 2), col0 = 16 * (g & 1) + 4 * (i16 & 3);
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int db = 0; db < DV / 32; db++) {
        const uint32_t row = row0 + 8 * u, col = col0 + 32 * db;
        s.va[u][db] = row * ROWB + ((((col >> 3)) ^ swz_rows<ROWB>(row)) << 4) + (((col >> 2) & 1) << 3);
      }
  }
  __device__ static void issue(const PrefillArgs& p, const Lane& s, int b, int h, int kvh, int key0, FA_LDS char* dst,
                               int wave, int lane) {
    (void)h;
    s.dma.issue((const char*)p.v + (((size_t)b * p.Skv + key0) * p.Hkv + kvh) * (size_t)ROWB, p.Hkv * ROWB,
                min(BN, p.Skv - key0), dst, wave, lane);
  }
  __device__ static f32x4_t scale4(const FA_LDS char*, int, int) { return f32x4_t{1.f, 1.f, 1.f, 1.f}; }
  // P^T block (kb, tp) -> O^T
  __device__ static void pv(RowAcc<DV>& st, const i32x4_t& pb, const Lane& s, const FA_LDS char* vst, int kb, int tp) {
#pragma unroll
    for (int db = 0; db < DV / 32; db++) {
      const int rows = (32 * kb + 16 * tp) * ROWB;
      const i32x2_t lo = lds_tr16(vst + s.va[0][db] + rows);
      const i32x2_t hi = lds_tr16(vst + s.va[1][db] + rows);
      st.o[db] = mfma32x32x16_bf16(cat(lo, hi), pb, st.o[db]);
    }
  }
};

// e4m3 V (rows of DV codes) with one fp32 scale per key row: V = code * v_scale.  The codes
// are read transposed one byte wide (ds_read_b64_tr_b8: 8 keys of one column per lane, one
// read per product) and converted to bf16 exactly; the scale is folded into P, so
// O^T += V_code^T . (P . v_scale)^T runs on the bf16 matrix cores.
// V part of a stage: codes [BN][DV] | v_scale [BN] fp32.
template <int DV_, int NW_ = 4>
struct VE4m3 {
  static constexpr int NW = NW_;
  static constexpr int DV = DV_;
  static constexpr int ROWB = DV;
  static constexpr int VS = BN * ROWB;
  static constexpr int BYTES = VS + BN * 4;
  static constexpr bool SCALED = true;
  struct Lane {
    RowDma<ROWB, SwzV8, NW_> dma;
    uint32_t va[DV / 32];
    uint32_t sa;
  };
  __device__ static void init(const PrefillArgs& p, int wave, int lane, Lane& s) {
    s.dma.init(wave, lane, p.Hkv * ROWB);
    // 16-lane group gq: lane 2e + h reads key row 8(e/4) + 4(gq/2) + e%4 at byte
    // 32db + 16(gq%2) + 8h, so lane L receives column 32db + L%32 of the keys
    // 8(e/4) + 4(L/32) + e%4, e = 0..7 -- the key order of P^T (the S^T accumulator layout)
    const uint32_t gq = lane >> 4, i = lane & 15, e = i >> 1, hb = i & 1;
    const uint32_t row0 = 8 * (e >> 2) + 4 * (gq >> 1) + (e & 3);
#pragma unroll
    for (int db = 0; db < DV / 32; db++)
      s.va[db] = row0 * ROWB + (((2 * db + (gq & 1)) ^ swz_v8(row0)) << 4) + 8 * hb;
    s.sa = VS + 16 * (lane >> 5);
  }
  __device__ static void issue(const PrefillArgs& p, const Lane& s, int b, int h, int kvh, int key0, FA_LDS char* dst,
                               int wave, int lane) {
    (void)h;
    const int valid = min(BN, p.Skv - key0);
    const size_t row = ((size_t)b * p.Skv + key0) * p.Hkv + kvh;
    s.dma.issue((const char*)p.v + row * ROWB, p.Hkv * ROWB, valid, dst, wave, lane);
    if (wave == 0) {
      const auto r = make_rsrc(p.v_scale + row, (uint32_t)((valid - 1) * p.Hkv + 1) * 4);
      dma4_buf(r, dst + VS, (uint32_t)min(lane, valid - 1) * p.Hkv * 4);
    }
  }
  // v_scale of keys 32kb + 16tp + 8j + 4hl .. +3 (the keys of P^T register 4j .. 4j+3)
  __device__ static f32x4_t scale4(const FA_LDS char* vst, int kb, int tp_j) {
    (void)kb;
    return lds_f32x4(vst + tp_j);
  }
  __device__ static void pv(RowAcc<DV>& st, const i32x4_t& pb, const Lane& s, const FA_LDS char* vst, int kb, int tp) {
#pragma unroll
    for (int db = 0; db < DV / 32; db++) {
      const i32x2_t w = lds_tr8(vst + s.va[db] + (32 * kb + 16 * tp) * ROWB);
      st.o[db] = mfma32x32x16_bf16(e4m3x8_to_bf16(w), pb, st.o[db]);
    }
  }
};

// Mask, row max, lazy rescale of O and l, then P^T = exp2(S^T c - m c) (times the V
// policy's per-key factor) packed to bf16, and the row sums of P.
template <class VP, bool CAUSAL>
__device__ __forceinline__ void tile_softmax(RowAcc<VP::DV>& st, f32x16_t (&s)[BN / 32], i32x4_t (&pb)[BN / 32][2],
                                             const typename VP::Lane& vl, const FA_LDS char* vst, int key0,
                                             bool masked, int qrow, int off, int Skv, float c, int hl) {
  constexpr int DV = VP::DV;
  if (masked) {
    // register v of block kb holds key key0 + 4hl + (32kb + 8(v/4) + v%4): visible iff
    // that constant offset is below lim
    const int lim = (CAUSAL ? min(Skv, qrow + off + 1) : Skv) - key0 - 4 * hl;
#pragma unroll
    for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
      for (int v = 0; v < 16; v++) s[kb][v] = (32 * kb + 8 * (v >> 2) + (v & 3)) < lim ? s[kb][v] : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
    for (int v = 0; v < 16; v++) mx = fmaxf(mx, s[kb][v]);
  mx = xor32_max(mx);
  if (__builtin_amdgcn_ballot_w64(mx * c > st.m_ref * c + kRescaleLog2)) {
    const float m_new = fmaxf(st.m_ref, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast((st.m_ref - m_use) * c);
    st.l *= alpha;
#pragma unroll
    for (int d = 0; d < DV / 32; d++) st.o[d] *= alpha;
    st.m_ref = m_new;
    st.neg = -m_use * c;
  }
#pragma unroll
  for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
    for (int tp = 0; tp < 2; tp++) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; i++) e[i] = exp2_fast(fmaf(s[kb][8 * tp + i], c, st.neg));
      if constexpr (VP::SCALED) {
        // register 8tp + i holds key 32kb + 16tp + 8(i/4) + 4hl + i%4
        const f32x4_t f0 = VP::scale4(vst, kb, vl.sa + (32 * kb + 16 * tp) * 4);
        const f32x4_t f1 = VP::scale4(vst, kb, vl.sa + (32 * kb + 16 * tp + 8) * 4);
#pragma unroll
        for (int i = 0; i < 8; i++) st.l += e[i];
        pb[kb][tp] = i32x4_t{pack_bf16(e[0] * f0[0], e[1] * f0[1]), pack_bf16(e[2] * f0[2], e[3] * f0[3]),
                             pack_bf16(e[4] * f1[0], e[5] * f1[1]), pack_bf16(e[6] * f1[2], e[7] * f1[3])};
      } else {
        pb[kb][tp] = i32x4_t{pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]), pack_bf16(e[4], e[5]), pack_bf16(e[6], e[7])};
#pragma unroll
        for (int i = 0; i < 4; i++) st.l = dot2_bf16(pb[kb][tp][i], kBf16PairOne, st.l);
      }
    }
}

template <class QK, class VP, bool CAUSAL, int KPART>
__device__ __forceinline__ void tile_step(RowAcc<VP::DV>& st, const typename QK::QFrag& q, const typename QK::Lane& ks,
                                          const typename VP::Lane& vl, const FA_LDS char* stage, int key0,
                                          bool masked, int qrow, int off, int Skv, float c, int hl, bool has_ks) {
  f32x16_t s[BN / 32];
  tile_scores<QK>(s, q, ks, stage, hl, has_ks);
  i32x4_t pb[BN / 32][2];
  tile_softmax<VP, CAUSAL>(st, s, pb, vl, stage + KPART, key0, masked, qrow, off, Skv, c, hl);
#pragma unroll
  for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
    for (int tp = 0; tp < 2; tp++) VP::pv(st, pb[kb][tp], vl, stage + KPART, kb, tp);
}

// ------------------------------------------------------------------------------------

// VARLEN: a ragged batch of packed sequences; sequence b owns query rows cu_q[b] ..
// cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1.  The grid covers the longest sequence
// (n_qblocks query blocks); a work item past its own sequence's blocks exits at once.
template <class QK, class VP, bool CAUSAL, bool VARLEN = false>
__global__ __launch_bounds__(64 * QK::NW, 2) void prefill_kernel(PrefillArgs pa, int n_qblocks) {
  static_assert(QK::NW == VP::NW, "K and V copies split over the same waves");
  constexpr int BM = 32 * QK::NW;
  constexpr int DV = VP::DV;
  constexpr int KPART = (QK::KBYTES + 1023) / 1024 * 1024;
  constexpr int OROWB = DV * 2;  // bf16 output row
  constexpr int STAGE = KPART + VP::BYTES;
  // One LDS object per stage: the compiler then sees that reads of one stage cannot alias
  // the direct copies into the other and does not wait for those copies before reading.
  __shared__ __attribute__((aligned(1024))) char stage0_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1_raw[STAGE];
  FA_LDS char* stage0 = (FA_LDS char*)stage0_raw;
  FA_LDS char* stage1 = (FA_LDS char*)stage1_raw;

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;

  // work item (workgroup i runs on XCD i % 8); the items of one (batch, head) stay on one
  // XCD, in order, so they share its K/V in that XCD's L2
  const int G = gridDim.x, x = blockIdx.x % 8, jx = blockIdx.x / 8;
  const int per_head = CAUSAL ? (n_qblocks + 1) / 2 : n_qblocks;
  int bh, it;
  if constexpr (VARLEN) {
    // sequences differ in length: (sequence, head) pairs are dealt round-robin to the XCDs
    // (pair bh on XCD bh % 8), so every XCD gets the same share of every sequence; the grid is
    // padded to whole rounds of 8 pairs
    bh = x + 8 * (jx / per_head);
    it = jx % per_head;
    if (bh >= pa.B * pa.Hq) return;
  } else {
    // equal (batch, head) pairs: each XCD takes a contiguous range of work items
    const int w = x * (G / 8) + min(x, G % 8) + jx;
    bh = w / per_head;
    it = w % per_head;
  }
  int b = bh / pa.Hq;
  const int h = bh % pa.Hq;
  const int kvh = h / (pa.Hq / pa.Hkv);
  PrefillArgs p = pa;
  // LSE of row (b, h, qrow) at lse_off + h * lse_hs + qrow
  size_t lse_off = (size_t)b * p.Hq * p.Sq;
  size_t lse_hs = (size_t)p.Sq;
  if constexpr (VARLEN) {
    // offsets are clamped into the packed tensors, so any array contents stay in bounds
    const int q0 = min(max(p.cu_q[b], 0), p.total_q), q1 = min(max(p.cu_q[b + 1], q0), p.total_q);
    const int k0 = min(max(p.cu_k[b], 0), p.total_k), k1 = min(max(p.cu_k[b + 1], k0), p.total_k);
    p.Sq = min(q1 - q0, pa.Sq);
    p.Skv = k1 - k0;
    n_qblocks = (p.Sq + BM - 1) / BM;
    if (it >= (CAUSAL ? (n_qblocks + 1) / 2 : n_qblocks)) return;
    p.q = (const char*)p.q + (size_t)q0 * p.Hq * QK::ROWB;
    p.o = (char*)p.o + (size_t)q0 * p.Hq * OROWB;
    p.k = (const char*)p.k + (size_t)k0 * p.Hkv * QK::ROWB;
    p.v = (const char*)p.v + (size_t)k0 * p.Hkv * VP::ROWB;
    lse_off = (size_t)q0;
    lse_hs = (size_t)p.total_q;
    b = 0;  // the pointers now start at the sequence
  }
  int blk[2] = {it, it};
  int nblk = 1;
  if (CAUSAL) {
    blk[0] = n_qblocks - 1 - it;
    blk[1] = it;
    nblk = blk[0] == blk[1] ? 1 : 2;
  }

  typename QK::Lane kl;
  QK::init(p, wave, lane, kl);
  typename VP::Lane vl;
  VP::init(p, wave, lane, vl);
  const float c = p.scale * kLog2e;
  const int off = p.Skv - p.Sq;
  const bool has_ks = p.k_scale != nullptr;

  auto issue = [&](int t, FA_LDS char* dst) {
    const int key0 = t * BN;
    QK::issue(p, kl, b, h, kvh, key0, dst, wave, lane);
    VP::issue(p, vl, b, h, kvh, key0, dst + KPART, wave, lane);
  };

  for (int bi = 0; bi < nblk; bi++) {
    const int q0 = blk[bi] * BM;
    int kv_end = p.Skv;
    if (CAUSAL) kv_end = max(0, min(p.Skv, min(q0 + BM, p.Sq) - 1 + off + 1));
    const int n_tiles = (kv_end + BN - 1) / BN;
    const int wrow0 = q0 + 32 * wave;
    int wave_end = kv_end, mask_from = p.Skv / BN;
    if (CAUSAL) {
      wave_end = max(0, min(kv_end, wrow0 + 31 + off + 1));
      const int lim = wrow0 + off + 1;
      mask_from = min(mask_from, lim > 0 ? lim / BN : 0);
    }
    const int wave_tiles = (wave_end + BN - 1) / BN;
    const int qrow = wrow0 + l32;

    typename QK::QFrag qf;
    QK::load_q(p, b, h, min(qrow, p.Sq - 1), hl, qf);
    RowAcc<DV> st;
#pragma unroll
    for (int d = 0; d < DV / 32; d++) st.o[d] = f32x16_t{};
    st.m_ref = -INFINITY;
    st.neg = 0.f;
    st.l = 0.f;

    // MLA: the second block of a causal pair takes its key tiles in descending order.  The
    // first blocks of a head's pairs then read K/V along one ascending front and the second
    // blocks along one descending front, instead of each second block starting over from key
    // 0 at its own time, so that the workgroups of a head find more of its tiles in L2 (a
    // head's K/V, 3-4 MB, is about one XCD's L2: 4 % faster on B1 H128 S8192; on the bf16
    // MHA workloads, 2 MB per head, 1-2 % slower, so they keep ascending order).
    const bool rev = CAUSAL && QK::REV_SECOND && bi == 1;
    auto tix = [&](int t) { return rev ? n_tiles - 1 - t : t; };
    if (bi > 0) barrier();  // every wave is done reading the previous block's last stage
    if (n_tiles > 0) issue(tix(0), stage0);
    for (int t = 0; t < n_tiles; t += 2) {
      wait_vmcnt<0>();
      barrier();
      if (t + 1 < n_tiles) issue(tix(t + 1), stage1);
      const int j0 = tix(t);
      if (j0 < wave_tiles)
        tile_step<QK, VP, CAUSAL, KPART>(st, qf, kl, vl, stage0, j0 * BN, j0 >= mask_from, qrow, off, p.Skv, c, hl, has_ks);
      if (t + 1 >= n_tiles) break;
      wait_vmcnt<0>();
      barrier();
      if (t + 2 < n_tiles) issue(tix(t + 2), stage0);
      const int j1 = tix(t + 1);
      if (j1 < wave_tiles)
        tile_step<QK, VP, CAUSAL, KPART>(st, qf, kl, vl, stage1, j1 * BN, j1 >= mask_from, qrow, off, p.Skv, c, hl,
                                         has_ks);
    }

    // epilogue: O = O^T / l, LSE = m_ref * scale + ln l
    const float l_tot = xor32_sum(st.l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    constexpr bool STAGE_O = QK::STAGE_O && DV == 128 && 4 * 32 * OROWB <= STAGE;
    if constexpr (STAGE_O) {
      // MLA with e4m3 nope and bf16 V: O goes through LDS so that each store instruction writes
      // four whole 256-byte rows.  Stored straight from the O^T layout, each store writes 16
      // bytes of each of 32 rows, and lines that left L2 partly written were written back more
      // than once (1.7x the output bytes on B1 H128 S8192, where K/V fill L2; 1 % faster
      // staged).  This wave's 32 rows: 16-byte chunk c of row r at chunk c ^ (r & 15) (the
      // writes of 16 rows then cover all banks).  The e4m3-V stage is too small for four
      // waves' rows, and the bf16 MHA kernels' output lines are written once as they are.
      barrier();  // every wave is done with both stages, and no copy is in flight
      FA_LDS char* ow = (wave < 4 ? stage0 : stage1) + (wave & 3) * (32 * OROWB);
#pragma unroll
      for (int db = 0; db < DV / 32; db++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int ch = 4 * db + j;
          *(FA_LDS i32x2_t*)(ow + l32 * OROWB + ((ch ^ (l32 & 15)) << 4) + 8 * hl) =
              i32x2_t{pack_bf16(st.o[db][4 * j] * inv, st.o[db][4 * j + 1] * inv),
                      pack_bf16(st.o[db][4 * j + 2] * inv, st.o[db][4 * j + 3] * inv)};
        }
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int r = 4 * k + (lane >> 4), ch = lane & 15;
        const i32x4_t x = *(const FA_LDS i32x4_t*)(ow + r * OROWB + ((ch ^ (r & 15)) << 4));
        if (wrow0 + r < p.Sq)
          *(i32x4_t*)((char*)p.o + (((size_t)b * p.Sq + wrow0 + r) * p.Hq + h) * (size_t)OROWB + ch * 16) = x;
      }
      if (p.lse && hl == 0 && qrow < p.Sq)
        p.lse[lse_off + h * lse_hs + qrow] = l_tot > 0.f ? st.m_ref * p.scale + logf(l_tot) : -INFINITY;
    } else if (qrow < p.Sq) {
      char* ob = (char*)p.o + (((size_t)b * p.Sq + qrow) * p.Hq + h) * (size_t)OROWB;
#pragma unroll
      for (int db = 0; db < DV / 32; db++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int d = 32 * db + 8 * j + 4 * hl;
          const i32x2_t wv = {pack_bf16(st.o[db][4 * j] * inv, st.o[db][4 * j + 1] * inv),
                              pack_bf16(st.o[db][4 * j + 2] * inv, st.o[db][4 * j + 3] * inv)};
          *(i32x2_t*)(ob + d * 2) = wv;
        }
      if (p.lse && hl == 0)
        p.lse[lse_off + h * lse_hs + qrow] = l_tot > 0.f ? st.m_ref * p.scale + logf(l_tot) : -INFINITY;
    }
  }
}


int items(const PrefillArgs& a, int bm, int& n_qblocks) {
  n_qblocks = (a.Sq + bm - 1) / bm;
  const int per_head = a.causal ? (n_qblocks + 1) / 2 : n_qblocks;
  return per_head * a.B * a.Hq;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int D, hipStream_t s) {
  // Head dim 128 without the causal mask, over at least 2048 keys and with at least one
  // 256-row block per CU: 64 query rows per wave, one wave per SIMD (5-6 % faster on B4 H32
  // S4096, also with 8 kv heads, and on B8 S256/2048; slower with shorter key ranges, where
  // each block's pipeline fill and drain weigh more, and with fewer blocks than CUs).  Also
  // needs a (batch, kv head)'s key rows plus the tiles the pipeline runs ahead to span less
  // than 2^31 bytes (32-bit lane offsets into one buffer range).
  if (D == 128 && !a.causal && a.Skv >= 2048 && (size_t)a.B * a.Hq * ((a.Sq + 255) / 256) >= 256 &&
      (size_t)(a.Skv + 256) * (size_t)a.Hkv * 256 < (size_t(1) << 31))
    return launch_prefill_w64(a, s);
  int nqb;
  // 8 waves per workgroup measured 2-3 % faster for causal head dim 128 from 2048 query rows
  // on (slower for head dim 64 and without the causal mask)
  const bool wide = D == 128 && a.causal && a.Sq >= 2048;
  const int grid = items(a, wide ? 256 : 128, nqb);
  if (grid == 0) return hipSuccess;
  if (wide) {
    prefill_kernel<QkBf16<128, 8>, VBf16<128, 8>, true><<<grid, 512, 0, s>>>(a, nqb);
  } else if (D == 128) {
    if (a.causal) prefill_kernel<QkBf16<128>, VBf16<128>, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_kernel<QkBf16<128>, VBf16<128>, false><<<grid, 256, 0, s>>>(a, nqb);
  } else {
    if (a.causal) prefill_kernel<QkBf16<64>, VBf16<64>, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_kernel<QkBf16<64>, VBf16<64>, false><<<grid, 256, 0, s>>>(a, nqb);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_varlen_bf16(const PrefillArgs& a, int D, hipStream_t s) {
  // a.Sq is the longest query sequence; (sequence, head) pairs padded to a multiple of 8
  const int nqb = (a.Sq + 127) / 128;
  const int per_head = a.causal ? (nqb + 1) / 2 : nqb;
  const int grid = (a.B * a.Hq + 7) / 8 * 8 * per_head;
  if (grid == 0) return hipSuccess;
  if (D == 128) {
    if (a.causal) prefill_kernel<QkBf16<128>, VBf16<128>, true, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_kernel<QkBf16<128>, VBf16<128>, false, true><<<grid, 256, 0, s>>>(a, nqb);
  } else {
    if (a.causal) prefill_kernel<QkBf16<64>, VBf16<64>, true, true><<<grid, 256, 0, s>>>(a, nqb);
    else prefill_kernel<QkBf16<64>, VBf16<64>, false, true><<<grid, 256, 0, s>>>(a, nqb);
  }
  return hipGetLastError();
}

template <class QK, class VP>
void launch_mla(const PrefillArgs& a, int grid, int nqb, hipStream_t s) {
  if (a.causal) prefill_kernel<QK, VP, true><<<grid, 64 * QK::NW, 0, s>>>(a, nqb);
  else prefill_kernel<QK, VP, false><<<grid, 64 * QK::NW, 0, s>>>(a, nqb);
}

hipError_t launch_mla_prefill(const PrefillArgs& a, bool nope_fp8, bool v_fp8, hipStream_t s) {
  int nqb;
  // e4m3 nope, causal, from 2048 query rows: 8 waves and 256 query rows per workgroup,
  // sharing each K/V tile copy between twice the rows (as the bf16 prefill)
  const bool wide = nope_fp8 && a.causal && a.Sq >= 2048;
  const int grid = items(a, wide ? 256 : 128, nqb);
  if (grid == 0) return hipSuccess;
  if (wide) {
    if (v_fp8) launch_mla<QkMla<true, 8>, VE4m3<128, 8>>(a, grid, nqb, s);
    else launch_mla<QkMla<true, 8>, VBf16<128, 8>>(a, grid, nqb, s);
  } else if (nope_fp8) {
    if (v_fp8) launch_mla<QkMla<true>, VE4m3<128>>(a, grid, nqb, s);
    else launch_mla<QkMla<true>, VBf16<128>>(a, grid, nqb, s);
  } else {
    if (v_fp8) launch_mla<QkMla<false>, VE4m3<128>>(a, grid, nqb, s);
    else launch_mla<QkMla<false>, VBf16<128>>(a, grid, nqb, s);
  }
  return hipGetLastError();
}

}  // namespace fa
