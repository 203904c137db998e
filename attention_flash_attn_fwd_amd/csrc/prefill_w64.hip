// Prefill forward for bf16 MHA / GQA of head dim 128 without the causal mask, with 64 query
// rows per wave: one wave per SIMD (a workgroup of 4 waves, 256 query rows, one workgroup per
// CU, 512 registers per lane), a software pipeline inside each wave instead of the overlap of
// two waves per SIMD.  (With the causal mask the four waves of a block end at different key
// tiles but stay in step through the shared ring, so the diagonal tiles leave SIMDs idle: the
// 32-row kernels serve that case.)
//
// Method: the flash-attention forward of Modular's "KVPipelineGeneric" page (S = Q.K' and
// O += P.V per K/V tile over a pipeline of K/V stages; its sub-MMAs of one tile run beside
// the softmax of another).  Here a step of 32 keys issues, in one instruction stream,
//   S^T(j+1) = K(j+1).Q^T      16 products (each 16-byte K read feeds both 32-row halves)
//   O^T     += V^T(j-1).P^T(j-1) 16 products (each transposed V fragment feeds both halves)
//   P(j)     = exp2(S(j) c - m c) packed to bf16, with the row sums
// so the exponentials of one tile run under the products of two others, with no dependency
// between them inside the step.
//
// Softmax reference: fixed per block at each row's maximum over its first key tile, so the
// steps need no row maximum and never rescale O^T (the accumulators stay in AGPRs, written by
// the matrix cores only).  P may then exceed 1; bf16 P and the fp32 sums keep their relative
// precision at any size.  A row whose final sum exceeds kW64Limit (a later score outgrew the
// reference by about 40 / c, or did not stay finite) makes the workgroup sweep the block's
// scores once for the exact row maxima and run the block again with them (P <= 1).
//
// K/V tiles go HBM -> LDS by direct buffer loads into an eight-stage ring (separate K and V
// rings, 64 KiB each, rows XOR-swizzled as in the other prefill kernels); every step issues
// the copies of the tile five steps ahead and every second step waits for the tiles two
// steps ahead and synchronises the workgroup.  Copies past the key range read nothing and
// write zeros (buffer range check).
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kW64Keys = 32;                 // keys per step
constexpr int kW64Stages = 8;                // ring depth
constexpr int kW64Stage = kW64Keys * 256;    // bytes per K (or V) stage: 32 rows of 128 bf16
constexpr int kW64Lead = 5;                  // a step issues the tile this many steps ahead
constexpr float kW64Limit = 0x1p40f;

// 16-byte direct copy (as dma16_asm) without a compiler memory fence: the copies write ring
// stages that no read of the current step touches, and the workgroup barriers (which are
// fences) order them against the reads of later steps, so LDS reads may be scheduled across.
__device__ __forceinline__ void w64_dma(const i32x4_t& rsrc, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(rsrc)
               : "m0");
}

struct W64Acc {
  f32x16_t o[4][2];  // O^T block (d block db, row half rb): register v holds d = 32db + 8(v/4) + 4hl + v%4
  float l[2];        // lane-partial row sums of the bf16-rounded P
  float neg[2];      // -m_ref * c (0 when the row has no visible key)
  float m_ref[2];
};

struct W64Lane {
  uint32_t ka[8];      // LDS byte address (K ring, stage 0) of this lane's chunk of MFMA step c
  uint32_t va[2][4];   // LDS byte address (V ring, stage 0) of the transposed reads (row half u, d block db)
  uint32_t coff[2];    // global byte offset (within a tile) of this lane's two 16-byte copy chunks
  uint32_t cdst[2];    // LDS byte offset (within a stage) of the 1 KiB block of each copy
};

// S^T of the 32 keys of one K stage for both row halves.
__device__ __forceinline__ void w64_scores(f32x16_t (&s)[2], const i32x4_t (&q)[2][8], const W64Lane& L,
                                           uint32_t koff) {
  s[0] = f32x16_t{};
  s[1] = f32x16_t{};
#pragma unroll
  for (int c = 0; c < 8; c++) {
    const i32x4_t k = lds_b128((const FA_LDS char*)(uintptr_t)(L.ka[c] + koff));
    s[0] = mfma32x32x16_bf16(k, q[0][c], s[0]);
    s[1] = mfma32x32x16_bf16(k, q[1][c], s[1]);
  }
}

// O^T += V^T . P^T over the 32 keys of one V stage.
__device__ __forceinline__ void w64_pv(W64Acc& a, const i32x4_t (&p)[2][2], const W64Lane& L, uint32_t voff) {
#pragma unroll
  for (int tp = 0; tp < 2; tp++)
#pragma unroll
    for (int db = 0; db < 4; db++) {
      const i32x2_t lo = lds_tr16((const FA_LDS char*)(uintptr_t)(L.va[0][db] + voff + 16 * tp * 256));
      const i32x2_t hi = lds_tr16((const FA_LDS char*)(uintptr_t)(L.va[1][db] + voff + 16 * tp * 256));
      const i32x4_t v = cat(lo, hi);
      a.o[db][0] = mfma32x32x16_bf16(v, p[0][tp], a.o[db][0]);
      a.o[db][1] = mfma32x32x16_bf16(v, p[1][tp], a.o[db][1]);
    }
}

// Keys of the step at or past lim[rb] (per lane: row limit - first key - 4 hl) get -inf.
// Register v of half rb holds key 8(v/4) + 4hl + v%4 of the step.
__device__ __forceinline__ void w64_mask(f32x16_t (&s)[2], const int (&lim)[2]) {
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int v = 0; v < 16; v++) s[rb][v] = (8 * (v >> 2) + (v & 3)) < lim[rb] ? s[rb][v] : -INFINITY;
}

// P = exp2(S c - m c) packed to bf16 (the P^T operand layout is the S^T accumulator layout),
// row sums from the rounded P.
__device__ __forceinline__ void w64_exps(W64Acc& a, const f32x16_t (&s)[2], i32x4_t (&p)[2][2], float c) {
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int tp = 0; tp < 2; tp++) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; i++) e[i] = exp2_fast(fmaf(s[rb][8 * tp + i], c, a.neg[rb]));
      p[rb][tp] = i32x4_t{pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]), pack_bf16(e[4], e[5]), pack_bf16(e[6], e[7])};
#pragma unroll
      for (int i = 0; i < 4; i++) a.l[rb] = dot2_bf16(p[rb][tp][i], kBf16PairOne, a.l[rb]);
    }
}

// Row maxima of S over the lane pair (l, l ^ 32), per half.
__device__ __forceinline__ void w64_rowmax(const f32x16_t (&s)[2], float (&mx)[2]) {
#pragma unroll
  for (int rb = 0; rb < 2; rb++) {
    float m = s[rb][0];
#pragma unroll
    for (int v = 1; v < 16; v++) m = fmaxf(m, s[rb][v]);
    mx[rb] = xor32_max(m);
  }
}

// Issue order of a step's instructions: a few reads ahead, then each product followed by one
// LDS read and four vector operations (the exponentials of the step run under the products).
__device__ __forceinline__ void w64_schedule() {
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
  for (int i = 0; i < 32; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
}

__global__ __launch_bounds__(256, 1) void prefill_w64_kernel(PrefillArgs p, int n_qblocks) {
  constexpr int BM = 256;
  __shared__ __attribute__((aligned(1024))) char kring_raw[kW64Stages * kW64Stage];
  __shared__ __attribute__((aligned(1024))) char vring_raw[kW64Stages * kW64Stage];
  __shared__ int redo_s[4];

  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;

  // work item: query block `it` of (batch, head) bh; the items of one (batch, head) stay on
  // one XCD (workgroup i runs on XCD i % 8), in order, so they share its K/V in that XCD's L2
  const int G = gridDim.x, x = blockIdx.x % 8, jx = blockIdx.x / 8;
  const int w_item = x * (G / 8) + min(x, G % 8) + jx;
  const int bh = w_item / n_qblocks, it = w_item % n_qblocks;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int kvh = h / (p.Hq / p.Hkv);

  const uint32_t kring = lds_addr((FA_LDS char*)kring_raw), vring = lds_addr((FA_LDS char*)vring_raw);
  const uint32_t stride = (uint32_t)p.Hkv * 256u;  // bytes between consecutive keys
  W64Lane L;
  {
    const uint32_t sw = swz256(l32);
#pragma unroll
    for (int c = 0; c < 8; c++) L.ka[c] = kring + l32 * 256 + (((2 * c + hl) ^ sw) << 4);
    const uint32_t g = lane >> 4, i16 = lane & 15;
    const uint32_t row0 = 4 * (g >> 1) + (i16 >> 2), col0 = 16 * (g & 1) + 4 * (i16 & 3);
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int db = 0; db < 4; db++) {
        const uint32_t row = row0 + 8 * u, col = col0 + 32 * db;
        L.va[u][db] = vring + row * 256 + (((col >> 3) ^ swz256(row)) << 4) + (((col >> 2) & 1) << 3);
      }
    // copy i of this wave: rows 4(4i + wave) .. +3 of the tile; lane -> row + lane / 16, LDS slot lane % 16
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint32_t grp = 4 * i + wave, row = 4 * grp + (lane >> 4);
      L.coff[i] = row * stride + ((((uint32_t)lane & 15) ^ swz256(row)) << 4);
      L.cdst[i] = grp * 1024;
    }
  }
  const float c = p.scale * kLog2e;

  // copies of tile t (keys 32t ..) into ring stage t % 8.  One buffer range per (batch, kv
  // head) covers its Skv keys; a tile's offset goes into the lane offsets, so keys past Skv are
  // out of range and read nothing (zeros).  The host keeps (Skv + 256) * stride below 2^31.
  const size_t kv0 = ((size_t)b * p.Skv * p.Hkv + kvh) * 256;
  const uint32_t range = p.Skv > 0 ? (uint32_t)(p.Skv - 1) * stride + 256u : 0u;
  const i32x4_t rk = rsrc_words((const char*)p.k + kv0, range);
  const i32x4_t rv = rsrc_words((const char*)p.v + kv0, range);
  auto issue = [&](int t) {
    const uint32_t toff = (uint32_t)(t * kW64Keys) * stride;
    const uint32_t st = (uint32_t)(t & (kW64Stages - 1)) * kW64Stage;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      w64_dma(rk, kring + st + L.cdst[i], L.coff[i] + toff);
      w64_dma(rv, vring + st + L.cdst[i], L.coff[i] + toff);
    }
  };

  // query rows of block bi for this wave: Q fragments (rows past Sq read row Sq - 1)
  i32x4_t q[2][8];
  auto load_q = [&](int q0) {
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
      const int qrow = min(q0 + 64 * wave + 32 * rb + l32, p.Sq - 1);
      const char* base = (const char*)p.q + (((size_t)b * p.Sq + qrow) * p.Hq + h) * (size_t)256;
#pragma unroll
      for (int cc = 0; cc < 8; cc++) q[rb][cc] = *(const i32x4_t*)(base + cc * 32 + hl * 16);
    }
  };

  W64Acc a;
  const int q0 = it * BM;
  load_q(q0);
#pragma unroll
  for (int t = 0; t < kW64Lead; t++) issue(t);  // the first tiles

  {
    const int n_wg = (p.Skv + kW64Keys - 1) / kW64Keys;  // tiles of the workgroup (and of each wave)
    const int wrow0 = q0 + 64 * wave;
    const int wave_n = n_wg;
    const int main_end = p.Skv / kW64Keys;  // steps below need no mask (whole tiles)
    const int rowlim[2] = {p.Skv, p.Skv};   // per half: keys below rowlim are visible

    // One pass over the block; tiles 0 .. kW64Lead-1 are already issued.  GIVEN: the
    // reference is in a.m_ref / a.neg (else it is taken from the first tile).
    auto pass = [&](auto given_ref) {
#pragma unroll
      for (int db = 0; db < 4; db++) a.o[db][0] = a.o[db][1] = f32x16_t{};
      a.l[0] = a.l[1] = 0.f;
      f32x16_t s[2][2];     // S^T of tiles j and j + 1: s[j % 2]
      i32x4_t pb[2][2][2];  // packed P of tiles j - 1 and j: pb[j % 2]
      // B(0): tiles 0..2 landed (3 and 4 may be in flight)
      wait_vmcnt<8>();
      barrier();
      issue(kW64Lead);
      // step 0 (every wave, also one whose rows see no key: its scores are all masked)
      w64_scores(s[0], q, L, 0);
      {
        const int lim[2] = {rowlim[0] - 4 * hl, rowlim[1] - 4 * hl};
        w64_mask(s[0], lim);
      }
      if constexpr (!decltype(given_ref)::value) {
        float mx[2];
        w64_rowmax(s[0], mx);
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
          a.m_ref[rb] = mx[rb];
          a.neg[rb] = -(mx[rb] == -INFINITY ? 0.f : mx[rb]) * c;
        }
      }
      w64_scores(s[1], q, L, 1 * kW64Stage);
      w64_exps(a, s[0], pb[0], c);

      // step j, U = j % 8 at compile time: [wait + barrier when j is even] S(j+1) from K stage
      // U+1, P.V of tile j-1 from V stage U-1, P(j) (keys masked when MASK), copies of tile
      // j+5 into stage U+5.  Past a wave's last tile its rows see no key, so its products
      // only add zeros.
      auto step = [&](int j, auto u_tag, auto mask_tag) {
        constexpr int U = decltype(u_tag)::value, cu = U & 1, nx = cu ^ 1;
        if constexpr ((U & 1) == 0) {
          wait_vmcnt<8>();
          barrier();
        }
        w64_scores(s[nx], q, L, (uint32_t)((U + 1) & 7) * kW64Stage);
        w64_pv(a, pb[nx], L, (uint32_t)((U + 7) & 7) * kW64Stage);
        if constexpr (decltype(mask_tag)::value) {
          const int lim[2] = {rowlim[0] - j * kW64Keys - 4 * hl, rowlim[1] - j * kW64Keys - 4 * hl};
          w64_mask(s[cu], lim);
        }
        w64_exps(a, s[cu], pb[cu], c);
        w64_schedule();
        issue(j + kW64Lead);
      };
      using F = std::false_type;
      using T = std::true_type;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      using I4 = std::integral_constant<int, 4>;
      using I5 = std::integral_constant<int, 5>;
      using I6 = std::integral_constant<int, 6>;
      using I7 = std::integral_constant<int, 7>;
      using I0 = std::integral_constant<int, 0>;

      int j = 1;
      // this wave's unmasked steps, eight at a time (j = 1 mod 8 at the top)
      while (j + 8 <= main_end) {
        step(j, I1{}, F{});
        step(j + 1, I2{}, F{});
        step(j + 2, I3{}, F{});
        step(j + 3, I4{}, F{});
        step(j + 4, I5{}, F{});
        step(j + 5, I6{}, F{});
        step(j + 6, I7{}, F{});
        step(j + 7, I0{}, F{});
        j += 8;
      }
      // the rest of this wave's steps, keys masked (step wave_n adds the P.V of its last tile)
      if (j <= wave_n) {
        for (;;) {
          step(j, I1{}, T{});
          if (++j > wave_n) break;
          step(j, I2{}, T{});
          if (++j > wave_n) break;
          step(j, I3{}, T{});
          if (++j > wave_n) break;
          step(j, I4{}, T{});
          if (++j > wave_n) break;
          step(j, I5{}, T{});
          if (++j > wave_n) break;
          step(j, I6{}, T{});
          if (++j > wave_n) break;
          step(j, I7{}, T{});
          if (++j > wave_n) break;
          step(j, I0{}, T{});
          if (++j > wave_n) break;
        }
      }
      // the workgroup's remaining steps: this wave only keeps the ring going
      for (; j <= n_wg; j++) {
        if ((j & 1) == 0) {
          wait_vmcnt<8>();
          barrier();
        }
        issue(j + kW64Lead);
      }
      // every copy has landed and every wave is done with the ring
      wait_vmcnt<0>();
      barrier();
    };

    pass(std::false_type{});
    // a row whose sum outgrew the limit: exact row maxima, then the block again
    {
      const bool big = !(xor32_sum(a.l[0]) <= kW64Limit) || !(xor32_sum(a.l[1]) <= kW64Limit);
      if (lane == 0) redo_s[wave] = __builtin_amdgcn_ballot_w64(big) != 0;
      barrier();
      const int redo = redo_s[0] | redo_s[1] | redo_s[2] | redo_s[3];
      if (redo) {
        float mx[2] = {-INFINITY, -INFINITY};
        for (int t = 0; t < n_wg; t++) {
          barrier();  // every wave is done with the stage this copy overwrites
          const int key0 = t * kW64Keys;
#pragma unroll
          for (int i = 0; i < 2; i++) w64_dma(rk, kring + L.cdst[i], L.coff[i] + (uint32_t)key0 * stride);
          wait_vmcnt<0>();
          barrier();
          f32x16_t sc[2];
          w64_scores(sc, q, L, 0);
          const int lim[2] = {rowlim[0] - key0 - 4 * hl, rowlim[1] - key0 - 4 * hl};
          w64_mask(sc, lim);
          float m[2];
          w64_rowmax(sc, m);
          mx[0] = fmaxf(mx[0], m[0]);
          mx[1] = fmaxf(mx[1], m[1]);
        }
        barrier();
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
          a.m_ref[rb] = mx[rb];
          a.neg[rb] = -(mx[rb] == -INFINITY ? 0.f : mx[rb]) * c;
        }
#pragma unroll
        for (int t = 0; t < kW64Lead; t++) issue(t);
        pass(std::true_type{});
      }
    }
    // epilogue: O = O^T / l, LSE = m_ref * scale + ln l
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
      const int qrow = wrow0 + 32 * rb + l32;
      const float l_tot = xor32_sum(a.l[rb]);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (qrow < p.Sq) {
        char* ob = (char*)p.o + (((size_t)b * p.Sq + qrow) * p.Hq + h) * (size_t)256;
#pragma unroll
        for (int db = 0; db < 4; db++)
#pragma unroll
          for (int jq = 0; jq < 4; jq++) {
            const int d = 32 * db + 8 * jq + 4 * hl;
            const i32x2_t wv = {pack_bf16(a.o[db][rb][4 * jq] * inv, a.o[db][rb][4 * jq + 1] * inv),
                                pack_bf16(a.o[db][rb][4 * jq + 2] * inv, a.o[db][rb][4 * jq + 3] * inv)};
            *(i32x2_t*)(ob + d * 2) = wv;
          }
        if (p.lse && hl == 0)
          p.lse[(size_t)b * p.Hq * p.Sq + (size_t)h * p.Sq + qrow] =
              l_tot > 0.f ? a.m_ref[rb] * p.scale + logf(l_tot) : -INFINITY;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_w64(const PrefillArgs& a, hipStream_t s) {
  if (a.causal) return hipErrorInvalidValue;
  const int nqb = (a.Sq + 255) / 256;
  const int grid = nqb * a.B * a.Hq;
  if (grid == 0) return hipSuccess;
  prefill_w64_kernel<<<grid, 256, 0, s>>>(a, nqb);
  return hipGetLastError();
}

}  // namespace fa
