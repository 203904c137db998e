// Decode (token generation) kernels: split-KV partials and their combine.
//
// The AMD "buffers" page gives its K/V tile buffers a token_gen variant; Modular's
// "KVPipelineGeneric" page (MLA decode utilities) pipelines K/V tiles through S = Q.K'
// and O += P.V.  With one query token per sequence there is no query-row parallelism
// to fill the GPU, so the KV range of each sequence is cut into splits processed by
// independent waves; each writes (row max m, row sum l, unnormalised O) and a combine
// kernel merges them: M = max_s m_s, w_s = 2^((m_s - M) c), O = sum w_s O_s / sum w_s l_s.
//
// This file: the MLA split kernel, the combine, and the launchers (the GQA split kernels are
// in gqa_decode.hip, built with the matrix-core results in ordinary vector registers).
#include <mutex>
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int TK = kDecodeTileKeys;  // keys per tile

// ------------------------------------------------------------------------------------
// MLA decode split: one workgroup of 4 waves -- one per SIMD, 512 registers each -- per
// (split, batch).  The heads form four groups of 32, the N columns of
// v_mfma_f32_32x32x16_bf16.  Wave w computes S^T = K.Q^T for head group w over the whole
// 576-deep contraction (its Q^T in 144 VGPRs), runs that group's softmax and writes its bf16
// P^T to LDS; then it takes O^T += V^T.P^T for output columns 128w .. 128w+127 of all 128
// heads (O^T in the 256 AGPRs), so each V^T operand read from LDS feeds four products.  The
// 576-wide latent tile (32 keys) is copied once per workgroup into a three-stage LDS ring by
// direct loads; its first 512 columns are V, so the cache is read from HBM once.
//
// bf16 cache, LDS tile layout ("chunk-column major"): 16-byte chunk c (8 latent columns) of
// key row r sits at (c / 2) * 1024 + (c % 2) * 512 + ((r + 4 (c % 4)) % 32) * 16, i.e. each
// 1 KiB block holds two chunk columns of all 32 rows, each column rotated by 4 (c % 4) row
// slots.  Then a direct copy instruction moves one whole block (lane l: row slot l % 32 of
// column 2j + l / 32, a source offset of one of two per-lane patterns plus 32 j), the K read
// of a contraction step is one contiguous 1 KiB block, and the transposing V reads of a pass
// hit 16 distinct 16-byte slots (all 64 banks once): no padding, and a handful of address
// registers.
//
// e4m3 cache with one fp32 scale per cache row (kv_scale [B, max_len]; the row serves as K
// and, through its first 512 columns, as V, so K = code * scale and V = code[:512] * scale):
//  * LDS rows are the 576 code bytes, unpadded; 16-byte chunk q of row r sits at chunk
//    q ^ ((r >> 2) & 3) (within its aligned group of four), which keeps both read patterns
//    free of bank conflicts; the tile's 32 row scales follow the codes;
//  * S^T A operand: one 16-byte read gives a lane 16 consecutive latent columns, i.e. its
//    halves of two 32x32x16 steps (the contraction order is permuted: block p, lane half hl,
//    step u, element i is column 32p + 16hl + 8u + i, and Q^T uses the same order), so a
//    wave issues half the K reads of the bf16 cache;
//  * V^T A operand: one ds_read_b64_tr_b8 per product (8 keys of one column per lane);
//  * codes convert exactly to bf16; the row scale multiplies S and is folded into P.

constexpr int MLA_DK = 576, MLA_DV = 512, MLA_ROWB = 1152;
constexpr int MLA_CTILE = TK * MLA_ROWB;              // 36 KiB per stage (bf16 cache)
constexpr int MLA_CBLK = MLA_CTILE / 1024;            // 36 one-KiB copy blocks per tile
constexpr int MLA_BW = 4;                             // waves (one per SIMD)
constexpr int MLA_QS = MLA_DK / 16;                   // S contraction steps per wave (36)
constexpr int MLA_OB = MLA_DV / 32 / MLA_BW;          // 32-column output blocks per wave (4)
static_assert(MLA_CBLK % MLA_BW == 0 && MLA_BW % 2 == 0, "bf16 tile copy split");
constexpr int MLA_CPW = MLA_CBLK / MLA_BW;            // direct copies per wave per tile, bf16 (9)
static_assert(MLA_CPW == MLA_QS / 4, "one copy per group of four S steps");
constexpr float kMlaGrow = 64.f;                      // log2 bound of P against the fixed reference

constexpr int M8_ROWB = 576;                          // e4m3 latent row
constexpr int M8_TILE = TK * M8_ROWB;                 // 18 KiB of codes per tile
constexpr int M8_BLKS = M8_TILE / 1024;               // 18 one-KiB direct copies per tile
constexpr int M8_STAGE = M8_TILE + 256;               // codes | row scales
constexpr int M8_CPW = 5;                             // direct copies per wave per tile, e4m3

// Split partials of the MLA O as 16-bit integers with one power-of-two scale per 128-column
// segment (the columns one wave holds) of each (head, split) row: value = q * 2^(e - 14), with
// 2^e above the segment's largest magnitude, so |q| < 2^14 and the truncation error is below
// 2^-13 of that largest magnitude (against the 2^-9 relative rounding of the bf16 output; the
// bound is absolute within a segment, so a column far below the segment's largest keeps an
// error relative to that largest value, not to its own).  The
// int16 rows (MLA_DV * 2 bytes) are followed by the exponents, [B, H, n_split, MLA_BW] int32.
// In fp32 the partials are 64 MiB at B64 H128, written by the splits and read back by the
// combine; two bytes per value halve that.  They fit in the workspace sized for fp32 partials.
constexpr int MLA_PB = 2;                      // bytes per partial O value
constexpr int MLA_SEG = MLA_DV / MLA_BW;       // columns per exponent (one wave's share)
constexpr int kMlaMinExp = -100;               // smaller segment maxima share this exponent
static_assert(MLA_DV * MLA_PB + 4 * MLA_BW <= MLA_DV * 4, "int16 rows and exponents within the fp32 sizing");
__device__ __forceinline__ int* mla_part_exps(const DecodeArgs& a) {
  return (int*)((char*)a.part_o + (size_t)a.B * a.Hq * a.n_split * MLA_DV * MLA_PB);
}
static_assert(M8_BLKS + 1 <= M8_CPW * MLA_BW && 2 * M8_CPW - 1 <= MLA_QS / 4,
              "the copies cover codes and scales, one per second group of four S steps");

// physical 16-byte chunk of logical chunk q in e4m3 row `row` (an involution)
__device__ __forceinline__ uint32_t m8_chunk(uint32_t row, uint32_t q) { return q ^ ((row >> 2) & 3u); }

// Work item of an MLA split kernel (one workgroup = one split of one sequence).  The grid
// is 1-D; workgroup i runs on XCD i % 8.  Every split of sequence b runs on XCD b % 8, at
// consecutive positions there, so the sequence's query rows (147 KiB for 128 heads) come
// into one L2 once instead of once per split.  Batch entries are padded to a multiple of 8;
// items past B exit.
__device__ __forceinline__ bool mla_item(const DecodeArgs& a, int& split, int& b) {
  const int i = blockIdx.x, x = i & 7, j = i >> 3;
  split = j % a.n_split;
  b = x + 8 * (j / a.n_split);
  return b < a.B;
}

template <bool E8>
__global__ __launch_bounds__(64 * MLA_BW, 1) void mla_decode_split(DecodeArgs a) {
  constexpr int STAGE = E8 ? M8_STAGE : MLA_CTILE;  // bytes per ring stage
  __shared__ __attribute__((aligned(1024))) char ring_raw[3 * STAGE];
  __shared__ __attribute__((aligned(1024))) char pt_raw[2 * MLA_BW * 2 * 1024];  // P^T of two tiles
  // head group whose scores outgrew the reference, per tile parity; lanes other than 0 of a
  // wave write their copy of the flag into a slot of their own (no branch on the lane), so
  // that the flags of the four waves sit side by side in slot 0
  __shared__ __attribute__((aligned(16))) int grow_s[2][64][MLA_BW];
  FA_LDS char* const ring = (FA_LDS char*)ring_raw;
  FA_LDS char* const pt = (FA_LDS char*)pt_raw;

  int split, b;
  if (!mla_item(a, split, b)) return;  // uniform over the workgroup
  const int L = min(max(a.kv_lens[b], 0), a.max_len);
  const int start = split * a.chunk;
  if (start >= L) return;  // uniform over the workgroup
  const int end = min(start + a.chunk, L);
  const int n_tiles = (end - start + TK - 1) / TK;

  const int wave = wave_id(), lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
  const int h = 32 * wave + l32;  // head of this lane in the S^T / softmax role
  const bool hvalid = h < a.Hq;
  const float c = a.scale * kLog2e;

  // Q^T of head group `wave` over the whole latent depth, as the B operand: column l32 = head
  // h; step i covers latent columns 16i + 8hl .. +7 (e4m3 cache: step i = 2p + u covers
  // columns 32p + 16hl + 8u .. +7, the order in which one 16-byte read of a code row gives a
  // lane its K operands of two steps)
  i32x4_t qf[MLA_QS];
  {
    const char* qp = (const char*)a.q + ((size_t)b * a.Hq + (hvalid ? h : 0)) * MLA_ROWB + (E8 ? 32 : 16) * hl;
#pragma unroll
    for (int i = 0; i < MLA_QS; i++) qf[i] = *(const i32x4_t*)(qp + (E8 ? 64 * (i >> 1) + 16 * (i & 1) : 32 * i));
  }
  const char* kv = (const char*)a.k + (size_t)b * a.max_len * (E8 ? M8_ROWB : MLA_ROWB);
  // direct copy k (0 .. 8) of a tile: block j = 4k + wave; lane l fills row slot l % 32 of
  // chunk column 2j + l / 32, i.e. key row (l % 32 - 8 (j % 2) - 4 (l / 32)) mod 32.  Rows past
  // the sequence repeat its last row; past the last tile the copies fetch nothing (an offset
  // beyond the range).
  const uint32_t crow = (uint32_t)(l32 - 8 * (wave & 1) - 4 * hl) & 31u;
  const uint32_t ring_lds = lds_addr(ring) + wave * 1024;
  struct Copy { i32x4_t r, rs; uint32_t src, dst; int valid; bool live; };
  auto plan_copy = [&](int t, int stage) {
    const int tt = min(t, n_tiles - 1);
    const int key0 = start + tt * TK, valid = min(TK, end - key0);
    Copy cp;
    cp.valid = valid;
    cp.live = t < n_tiles;
    if constexpr (E8) {
      cp.r = rsrc_words(kv + (size_t)key0 * M8_ROWB, (uint32_t)valid * M8_ROWB);
      cp.rs = rsrc_words(a.k_scale + (size_t)b * a.max_len + key0, (uint32_t)valid * 4);
      cp.dst = lds_addr(ring) + stage * STAGE;
    } else {
      cp.r = rsrc_words(kv + (size_t)key0 * MLA_ROWB, (uint32_t)valid * MLA_ROWB);
      cp.src = t < n_tiles ? min(crow, (uint32_t)(valid - 1)) * MLA_ROWB + 16u * hl + 32u * wave : kOutOfRange;
      cp.dst = ring_lds + stage * MLA_CTILE;
    }
    return cp;
  };
  // e4m3 cache: copy k (0 .. M8_CPW-1) of a tile is block j = 4k + wave; block j < 18 holds LDS bytes
  // [1024 j, +1024) of the code rows (lane l: byte o = 1024 j + 16 l, row o / 576, physical
  // chunk (o % 576) / 16), block 18 the 32 row scales, block 19 nothing
  auto copy = [&](const Copy& cp, int k) {
    if constexpr (E8) {
      const int j = 4 * k + wave;  // wave-uniform
      if (j < M8_BLKS) {
        // the lane's source offset from a fresh lane index (an asm the compiler cannot hoist):
        // offsets precomputed for every copy would stay live across the tile loop
        uint32_t lane_c;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_c));
        const uint32_t o = 1024u * j + 16u * lane_c, row = o / M8_ROWB, pc = (o % M8_ROWB) >> 4;
        const uint32_t src = min(row, (uint32_t)(cp.valid - 1)) * M8_ROWB + m8_chunk(row, pc) * 16;
        dma16_asm(cp.r, cp.dst + 1024u * j, cp.live ? src : kOutOfRange);
      } else if (j == M8_BLKS) {
        dma4_asm(cp.rs, cp.dst + M8_TILE, cp.live ? (uint32_t)min(lane, cp.valid - 1) * 4 : kOutOfRange);
      }
    } else {
      dma16_asm(cp.r, cp.dst + k * MLA_BW * 1024, cp.src + 32u * MLA_BW * k);
    }
  };
  // S^T A operand of step i: key row l32, chunk 2i + hl, at koff[i % 2] + 1024 i.  e4m3: the
  // 16-byte read j of group gi is code row l32, logical chunk 4 gi + 2j + hl (steps 4gi + 2j
  // and + 1), at koff[j] + 64 gi
  const uint32_t koff0 = E8 ? l32 * M8_ROWB + ((hl ^ ((l32 >> 2) & 3)) << 4) : hl * 512 + ((l32 + 4 * hl) & 31) * 16;
  const uint32_t koff1 = E8 ? l32 * M8_ROWB + (((2 + hl) ^ ((l32 >> 2) & 3)) << 4)
                            : hl * 512 + ((l32 + 8 + 4 * hl) & 31) * 16;
  // V^T reads (A operand of O^T) of P^T block tp, half u, output block d of this wave: key
  // rows 16tp + 8u + 4(g/2) + i16/4, output columns 128 wave + 32d + 16(g%2) + 4(i16%4) .. +3
  // (chunk 16 wave + 4d + 2(g%2) + (i16%4)/2), at voff[tp][u] + 2048 d
  uint32_t voff[2][2];
  {
    const uint32_t g = lane >> 4, i16 = lane & 15;
    const uint32_t rr = 4 * (2 * (g & 1) + ((i16 & 3) >> 1));
#pragma unroll
    for (int tp = 0; tp < 2; tp++)
#pragma unroll
      for (int u = 0; u < 2; u++)
        voff[tp][u] = (8 * wave + (g & 1)) * 1024 + ((i16 & 3) >> 1) * 512 + 8 * (i16 & 1) +
                      ((16 * tp + 8 * u + 4 * (g >> 1) + (i16 >> 2) + rr) & 31) * 16;
    if constexpr (E8) {
      // e4m3: one ds_read_b64_tr_b8 per operand.  16-lane group g (hl = g / 2, column half
      // dh = g % 2); lane 2e + h of the group reads key row 16tp + 8(e/4) + 4hl + e%4 at byte
      // 8h of logical chunk 8 wave + 2d + dh, so output byte e of lane l is column
      // 128 wave + 32d + l%32 of that key -- the P^T key order.  The XOR touches the two low
      // chunk bits: voff[tp][d % 2] + 64 (d / 2).
      const uint32_t e = (lane & 15) >> 1, hb = lane & 1;
#pragma unroll
      for (int tp = 0; tp < 2; tp++) {
        const uint32_t row = 16 * tp + 8 * (e >> 2) + 4 * (g >> 1) + (e & 3);
        const uint32_t x = (g & 1) ^ ((row >> 2) & 3);
#pragma unroll
        for (int par = 0; par < 2; par++) voff[tp][par] = row * M8_ROWB + 8 * hb + ((8 * wave + (x ^ (2 * par))) << 4);
      }
    }
  }
  FA_LDS int* const grow_own = (FA_LDS int*)&grow_s[0][lane][wave];

  // Softmax reference of head h, fixed at the first tile of a pass: P = 2^((s - m_ref) c)
  // stays below 2^kMlaGrow (bf16 keeps its relative precision at any size, and the fp32 sums
  // stay far from overflow), so O is never rescaled.  A tile whose scores outgrow that bound
  // makes the workgroup pass over the split again with the reference raised to that tile's
  // maximum (each such pass raises it by more than kMlaGrow / c, at a later tile).
  float m_ref = -INFINITY, l = 0.f;
  // O^T of output columns 128 wave .. +127 for every head: o[d][g] is output block d (32
  // columns) of head group g
  f32x16_t o[MLA_OB][MLA_BW];
  for (;;) {  // passes over the split: one, unless a tile outgrows the reference
#pragma unroll
    for (int d = 0; d < MLA_OB; d++)
#pragma unroll
      for (int g = 0; g < MLA_BW; g++) o[d][g] = f32x16_t{};
    l = 0.f;
    bool grew = false;
    float mx = 0.f;
    // Tile t sits in stage t % 3.  Iteration t (0 .. n_tiles) computes the scores of tile t,
    // then the PV product of tile t-1 with the softmax of tile t woven into it, so that the
    // exponentials run under the matrix products.  The ends cost a little idle work instead
    // of code of their own: at t = 0 the product reads tile 0's V against a zero P^T slot
    // (it adds exactly zero), and at t = n_tiles the scores are all masked (P = 0, no growth).
    {
      const Copy c0 = plan_copy(0, 0);
#pragma unroll
      for (int k = 0; k < (E8 ? M8_CPW : MLA_CPW); k++) copy(c0, k);
      // the zeros from an asm the compiler cannot hoist: a zero vector kept in registers across
      // the passes was spilled
      int z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
      for (int tp = 0; tp < 2; tp++) *(FA_LDS i32x4_t*)(pt + (2 * MLA_BW + 2 * wave + tp) * 1024 + lane * 16) = i32x4_t{z, z, z, z};
      grow_own[64 * MLA_BW] = 0;  // tile "-1" (parity 1)
    }
    int stc = 0;
    for (int t = 0; t <= n_tiles; t++) {
      // tile t landed; every wave is done with tile t-2 (whose stage takes tile t+1), has
      // written the P^T and growth flag of tile t-1 and has read those of tile t-2
      wait_vmcnt<0>();
      wait_lgkmcnt0();
      barrier();
      const int stn = stc == 2 ? 0 : stc + 1;
      const int stp = t == 0 ? stc : (stn == 2 ? 0 : stn + 1);
      const Copy cn = plan_copy(t + 1, stn);
      // S^T of this wave's 32 heads over the whole depth, the K reads one group of four steps
      // ahead of their products; the copies of tile t+1 go out one per group, so that no
      // wave stalls on a burst of them
      const FA_LDS char* kt = ring + stc * STAGE;
      f32x16_t s{};
      if constexpr (E8) {
        auto kread = [&](int gi, int j) { return lds_b128(kt + (j ? koff1 : koff0) + 64 * gi); };
        i32x4_t kr[2][2];
#pragma unroll
        for (int j = 0; j < 2; j++) kr[0][j] = kread(0, j);
#pragma unroll
        for (int gi = 0; gi < MLA_QS / 4; gi++) {
          if (gi + 1 < MLA_QS / 4) {
#pragma unroll
            for (int j = 0; j < 2; j++) kr[(gi + 1) & 1][j] = kread(gi + 1, j);
          }
          if (gi % 2 == 0) copy(cn, gi / 2);
#pragma unroll
          for (int j = 0; j < 2; j++) {
            const i32x4_t w = kr[gi & 1][j];
            s = mfma32x32x16_bf16(e4m3x8_to_bf16(i32x2_t{w.x, w.y}), qf[4 * gi + 2 * j], s);
            s = mfma32x32x16_bf16(e4m3x8_to_bf16(i32x2_t{w.z, w.w}), qf[4 * gi + 2 * j + 1], s);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        auto kread = [&](int i) { return lds_b128(kt + ((i & 1) ? koff1 : koff0) + 1024 * i); };
        i32x4_t kr[2][4];
#pragma unroll
        for (int j = 0; j < 4; j++) kr[0][j] = kread(j);
#pragma unroll
        for (int gi = 0; gi < MLA_QS / 4; gi++) {
          if (gi + 1 < MLA_QS / 4) {
#pragma unroll
            for (int j = 0; j < 4; j++) kr[(gi + 1) & 1][j] = kread(4 * (gi + 1) + j);
          }
          copy(cn, gi);
#pragma unroll
          for (int j = 0; j < 4; j++) s = mfma32x32x16_bf16(kr[gi & 1][j], qf[4 * gi + j], s);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // register v holds key 8(v/4) + 4hl + v%4 of the tile.  e4m3: the row scales of tile t
      // multiply S (and fold into P below: V = code * scale), before the mask so that a
      // masked score stays -inf whatever the scale
      const FA_LDS char* const rscale = kt + M8_TILE + 16 * hl;  // keys 8j + 4hl .. +3 at 32 j
      if constexpr (E8) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const f32x4_t r = lds_f32x4(rscale + 32 * j);
#pragma unroll
          for (int v = 0; v < 4; v++) s[4 * j + v] *= r[v];
        }
      }
      // keys past the split are masked
      const int key0 = start + t * TK;
      if (key0 + TK > end) {  // the last tiles only: a branch, not selects on every tile
        asm volatile("" ::: "memory");
        // the lane half from a fresh lane index (an asm the compiler cannot hoist), so that no
        // per-lane limit stays live across the tile loop
        int lane_m;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_m));
        const int lim = end - key0 - 4 * (lane_m >> 5);
#pragma unroll
        for (int v = 0; v < 16; v++) s[v] = (8 * (v >> 2) + (v & 3)) < lim ? s[v] : -INFINITY;
      }
      // O^T += V^T P^T of tile t-1, the V^T operands two (tp, d) pairs ahead of their four
      // products; slice k of the softmax of tile t after pair k: row maximum, growth flag,
      // exponentials, bf16 P^T with its row sum, P^T into the slot of tile t
      const FA_LDS char* vt = ring + stp * STAGE;
      const int u = (t - 1) & 1;
      // the growth flags of tile t-1 first, so that the branch on them waits for that read
      // alone; the P^T operands and the first V^T operands are in flight meanwhile
      const i32x4_t gflag = *(const FA_LDS i32x4_t*)&grow_s[(t - 1) & 1][0][0];
      i32x4_t pb[2][MLA_BW];
#pragma unroll
      for (int tp = 0; tp < 2; tp++)
#pragma unroll
        for (int g = 0; g < MLA_BW; g++) pb[tp][g] = lds_b128(pt + (u * 2 * MLA_BW + 2 * g + tp) * 1024 + lane * 16);
      // V^T operands as read (e4m3: the eight codes, converted at their products)
      using VRaw = std::conditional_t<E8, i32x2_t, i32x4_t>;
      auto vread = [&](int pi) -> VRaw {
        const int tp = pi / MLA_OB, d = pi % MLA_OB;
        if constexpr (E8) return lds_tr8(vt + voff[tp][d & 1] + 64 * (d >> 1));
        else return cat(lds_tr16(vt + voff[tp][0] + 2048 * d), lds_tr16(vt + voff[tp][1] + 2048 * d));
      };
      VRaw va[3];
      va[0] = vread(0);
      va[1] = vread(1);
      // tile t-1 outgrew the reference: pass again (its product has not been taken)
      if (gflag[0] | gflag[1] | gflag[2] | gflag[3]) {  // uniform over the workgroup; rare
        grew = true;
        break;
      }

      float neg = 0.f;
      i32x4_t pw[2];
#pragma unroll
      for (int pi = 0; pi < 2 * MLA_OB; pi++) {
        if (pi + 2 < 2 * MLA_OB) va[(pi + 2) % 3] = vread(pi + 2);
        const int tp = pi / MLA_OB, d = pi % MLA_OB;
        i32x4_t vop;
        if constexpr (E8) vop = e4m3x8_to_bf16(va[pi % 3]);
        else vop = va[pi % 3];
#pragma unroll
        for (int g = 0; g < MLA_BW; g++) o[d][g] = mfma32x32x16_bf16(vop, pb[tp][g], o[d][g]);
        if (pi == 0) {
          mx = s[0];
#pragma unroll
          for (int v = 1; v < 16; v++) mx = fmaxf(mx, s[v]);
        } else if (pi == 1) {
          mx = xor32_max(mx);
          m_ref = t == 0 ? fmaxf(m_ref, mx) : m_ref;  // O and l are still zero at t = 0
          const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
          neg = -m_use * c;
          grow_own[(t & 1) * 64 * MLA_BW] = __builtin_amdgcn_ballot_w64(mx * c + neg > kMlaGrow) != 0;
        } else if (pi < 6) {
          f32x4_t r4{};
          if constexpr (E8) r4 = lds_f32x4(rscale + 32 * (pi - 2));  // read again: fewer live registers
#pragma unroll
          for (int v = 0; v < 4; v++) {
            const int r = 4 * (pi - 2) + v;
            s[r] = exp2_fast(fmaf(s[r], c, neg));
            if constexpr (E8) {  // the weight sums unscaled; P^T carries the value scale
              l += s[r];
              s[r] *= r4[v];
            }
          }
        } else if (pi == 6) {
#pragma unroll
          for (int tp2 = 0; tp2 < 2; tp2++) {
            pw[tp2] = i32x4_t{pack_bf16(s[8 * tp2], s[8 * tp2 + 1]), pack_bf16(s[8 * tp2 + 2], s[8 * tp2 + 3]),
                              pack_bf16(s[8 * tp2 + 4], s[8 * tp2 + 5]), pack_bf16(s[8 * tp2 + 6], s[8 * tp2 + 7])};
            if constexpr (!E8) {
#pragma unroll
              for (int i = 0; i < 4; i++) l = dot2_bf16(pw[tp2][i], kBf16PairOne, l);
            }
          }
        } else {
#pragma unroll
          for (int tp2 = 0; tp2 < 2; tp2++)
            *(FA_LDS i32x4_t*)(pt + ((t & 1) * 2 * MLA_BW + 2 * wave + tp2) * 1024 + lane * 16) = pw[tp2];
        }
        // each product followed by a share of the slice's vector work, which then runs under it
#pragma unroll
        for (int g = 0; g < MLA_BW; g++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // up to five VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      stc = stn;
    }
    wait_vmcnt<0>();  // no copy may land in LDS after the workgroup ends
    if (!grew) break;
    m_ref = fmaxf(m_ref, mx);  // mx: the maximum of the tile that outgrew the reference
    barrier();                 // every wave has read the flags and is done with every stage
  }

  const float l_tot = xor32_sum(l);
  // The output addresses are formed here from a fresh lane index (an asm the compiler cannot
  // hoist), so that nothing computed before the loop stays live across it.
  int lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int l32e = lane_e & 31, hle = lane_e >> 5;
  if (hle == 0 && 32 * wave + l32e < a.Hq) {
    const size_t pidx = ((size_t)b * a.Hq + 32 * wave + l32e) * a.n_split + split;
    a.part_ml[2 * pidx] = m_ref;
    a.part_ml[2 * pidx + 1] = l_tot;
  }
  // O^T register v of block (d, g) holds output column 128 wave + 32d + 8(v/4) + 4hl + v%4 of
  // head 32g + l32
#pragma unroll
  for (int g = 0; g < MLA_BW; g++) {
    // the segment (this wave's 128 columns of head 32g + l32) lies in lanes l32 and l32 + 32
    float mx = 0.f;
#pragma unroll
    for (int d = 0; d < MLA_OB; d++)
#pragma unroll
      for (int v = 0; v < 16; v++) mx = fmaxf(mx, fabsf(o[d][g][v]));
    mx = xor32_max(mx);
    const int e = mx > 0.f ? max(__builtin_amdgcn_frexp_expf(mx), kMlaMinExp) : kMlaMinExp;  // mx < 2^e
    const float sc = __builtin_amdgcn_ldexpf(1.f, 14 - e);
    const int hg = 32 * g + l32e;
    if (hg < a.Hq) {
      const size_t pidx = ((size_t)b * a.Hq + hg) * a.n_split + split;
      if (hle == 0) mla_part_exps(a)[pidx * MLA_BW + wave] = e;
      char* po = (char*)a.part_o + (pidx * MLA_DV + MLA_SEG * wave + 4 * hle) * MLA_PB;
#pragma unroll
      for (int d = 0; d < MLA_OB; d++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const auto lo = __builtin_amdgcn_cvt_pk_i16((int)(o[d][g][4 * j] * sc), (int)(o[d][g][4 * j + 1] * sc));
          const auto hi = __builtin_amdgcn_cvt_pk_i16((int)(o[d][g][4 * j + 2] * sc), (int)(o[d][g][4 * j + 3] * sc));
          *(i32x2_t*)(po + (32 * d + 8 * j) * MLA_PB) = i32x2_t{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
        }
    }
  }

}

// ------------------------------------------------------------------------------------
// Combine: merges, for every (batch, head) row, the splits that cover [0, L_b) in split
// order (deterministic, no atomics): O = sum_s w_s O_s / sum_s w_s l_s with
// w_s = exp2((m_s - M) c), M = max_s m_s.  A thread owns 8 consecutive output columns of
// one row, so its loads of the partials are independent reads, non-temporal (read once).
// PB: bytes per partial O value (4: fp32, the GQA splits; MLA_PB: the MLA splits).

constexpr int CMB_COLS = 8;

template <int PB>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a, int Dv) {
  const int tpr = Dv / CMB_COLS;  // threads per row
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int bh = gid / tpr, d0 = (gid % tpr) * CMB_COLS;
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq;
  const int L = min(max(a.kv_lens[b], 0), a.max_len);
  const int ns = (L + a.chunk - 1) / a.chunk;
  const float c = a.scale * kLog2e;
  const float* ml = a.part_ml + (size_t)bh * a.n_split * 2;
  const char* po = (const char*)a.part_o + ((size_t)bh * a.n_split * Dv + d0) * PB;
  float M = -INFINITY;
  for (int s = 0; s < ns; s++) M = fmaxf(M, ml[2 * s]);
  float den = 0.f;
  f32x4_t x0{}, x1{};
#pragma unroll 4
  for (int s = 0; s < ns; s++) {
    const float w = exp2_fast((ml[2 * s] - M) * c);
    den = fmaf(w, ml[2 * s + 1], den);
    const char* ps = po + (size_t)s * Dv * PB;
    f32x4_t u0, u1;
    if constexpr (PB == 4) {
      u0 = __builtin_nontemporal_load((const f32x4_t*)ps);
      u1 = __builtin_nontemporal_load((const f32x4_t*)ps + 1);
    } else {
      static_assert(PB == MLA_PB, "partial format");
      const i32x4_t w = __builtin_nontemporal_load((const i32x4_t*)ps);
      const int e = mla_part_exps(a)[((size_t)bh * a.n_split + s) * MLA_BW + d0 / MLA_SEG] - 14;
#pragma unroll
      for (int i = 0; i < 2; i++) {
        // low and high 16-bit halves, sign-extended
        u0[2 * i] = __builtin_amdgcn_ldexpf((float)(short)w[i], e);
        u0[2 * i + 1] = __builtin_amdgcn_ldexpf((float)(w[i] >> 16), e);
        u1[2 * i] = __builtin_amdgcn_ldexpf((float)(short)w[2 + i], e);
        u1[2 * i + 1] = __builtin_amdgcn_ldexpf((float)(w[2 + i] >> 16), e);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x0[i] = fmaf(w, u0[i], x0[i]);
      x1[i] = fmaf(w, u1[i], x1[i]);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  __bf16* out = (__bf16*)a.o + (size_t)bh * Dv + d0;
  *(i32x4_t*)out = i32x4_t{pack_bf16(x0[0] * inv, x0[1] * inv), pack_bf16(x0[2] * inv, x0[3] * inv),
                           pack_bf16(x1[0] * inv, x1[1] * inv), pack_bf16(x1[2] * inv, x1[3] * inv)};
  if (a.lse && d0 == 0) a.lse[bh] = den > 0.f ? M * a.scale + logf(den) : -INFINITY;
}

}  // namespace

hipError_t launch_gqa_decode(const DecodeArgs& a, int D, bool fp8, hipStream_t s) {
  const hipError_t e = launch_gqa_split_kernels(a, D, fp8, s);
  if (e != hipSuccess) return e;
  combine_kernel<4><<<(a.B * a.Hq * (D / CMB_COLS) + 255) / 256, 256, 0, s>>>(a, D);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// The split partials of attn_decode_fwd_static, for callers that cannot allocate device memory:
// a buffer of fixed size in the code object, one copy per GPU, held until the process ends.
// Every call on a GPU shares its copy, and nothing in it needs clearing between calls: the
// combine reads only the partials of splits that start before their sequence's length, and
// each of those splits writes its partial first.  Host code never passes `scratch` itself to a
// kernel (in host code the name is a stand-in, not a device address): it passes the address
// hipGetSymbolAddress returns for the device the stream runs on.
static __device__ __align__(256) unsigned char scratch[kDecodeStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each device, once resolved
}  // namespace

// Device address of the static partials buffer on the device that stream s runs on (the
// current device for the null stream), resolved once per device with that device current.
static hipError_t static_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_gqa_decode_static(DecodeArgs a, int D, bool fp8, hipStream_t s) {
  void* p = nullptr;
  const hipError_t e = static_scratch(s, &p);
  if (e != hipSuccess) return e;
  a.part_o = (float*)p;
  a.part_ml = (float*)((char*)p + ((size_t)a.B * a.Hq * a.n_split * D * 4 + 255) / 256 * 256);
  return launch_gqa_decode(a, D, fp8, s);
}

hipError_t launch_mla_decode(const DecodeArgs& a, bool fp8, hipStream_t s) {
  const int grid = a.n_split * ((a.B + 7) / 8 * 8);  // see mla_item
  if (fp8) mla_decode_split<true><<<grid, 64 * MLA_BW, 0, s>>>(a);
  else mla_decode_split<false><<<grid, 64 * MLA_BW, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_kernel<MLA_PB><<<(a.B * a.Hq * (MLA_DV / CMB_COLS) + 255) / 256, 256, 0, s>>>(a, MLA_DV);
  return hipGetLastError();
}

}  // namespace fa
