// Device building blocks of the gfx950 attention kernels.
//
// Operand layouts (CDNA4 MFMA, as measured on gfx950 with single-wave probes):
//   v_mfma_f32_32x32x16_bf16: A[m][k] lane l holds m = l%32, k = 8*(l/32)+i (i < 8);
//     B[k][n] lane l holds n = l%32, the same k; C lane l, register v holds
//     row 8*(v/4) + 4*(l/32) + v%4, column l%32.
//   v_mfma_f32_16x16x32_bf16: A lane l holds m = l%16, k = 8*(l/16)+i; C lane l, register v
//     holds row 4*(l/16) + v, column l%16.
//   v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, unit scales): m/n and C as the 32x32 bf16
//     form; each lane holds 32 k values.
//   ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i%4) of the
//     8-byte word read by lane 4*e + i/4, for e = 0..3 -- i.e. when lanes 4r..4r+3
//     address row r (4 consecutive 16-bit columns each), lane i receives column i of
//     rows 0..3.
//   global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l (base = M0).
//
// Both attention products run transposed: S^T = K.Q^T (K from LDS as A, Q^T from
// registers as B) and O^T = V^T.P^T (V^T from LDS through transposing reads as A,
// P^T from registers as B).  Then a lane owns one query column of S^T, P^T and O^T at
// once, so the softmax row state (max, sum, rescale factor) stays in that lane and only
// meets the other half-wave holding the same query.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

#define FA_LDS __attribute__((address_space(3)))

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;

constexpr float kLog2e = 1.44269504088896340736f;

// ------------------------------------------------------------------ matrix cores

__device__ __forceinline__ f32x16_t mfma32x32x16_bf16(i32x4_t a, i32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32_bf16(i32x4_t a, i32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// e4m3 x e4m3 -> fp32, K = 64, block scales fixed at 2^0 (E8M0 code 127).
__device__ __forceinline__ f32x16_t mfma32x32x64_e4m3(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x16_t mfma32x32x2_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ LDS access

__device__ __forceinline__ i32x4_t lds_b128(const FA_LDS char* p) {
  return *(const FA_LDS i32x4_t*)p;
}
__device__ __forceinline__ f32x4_t lds_f32x4(const FA_LDS char* p) {
  return *(const FA_LDS f32x4_t*)p;
}
__device__ __forceinline__ i32x2_t lds_tr16(const FA_LDS char* p) {
  i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4_t*)p);
  return __builtin_bit_cast(i32x2_t, v);
}
// ds_read_b64_tr_b8: within each 16-lane group, lane 8h + b receives byte b of the 8-byte
// words read by lanes h, h + 2, ..., h + 14 -- i.e. when lanes 2e + h address row e
// (8 consecutive bytes at column 8h), lane i receives column i of rows 0..7 (measured on
// gfx950 with a single-wave probe).
__device__ __forceinline__ i32x2_t lds_tr8(const FA_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2_t*)p);
}
// Eight ds_read_b64_tr_b16 at LDS byte addresses a[i], issued back to back and waited for
// once, in one asm statement: the reads overlap, and the compiler, which sees no LDS read here,
// adds no wait of its own for direct-to-LDS copies still in flight into other buffers -- the
// caller must already have waited (s_waitcnt vmcnt) for the copies of the data read here.
// Outputs are early-clobber: a read may land before a later read of the block issues.
__device__ __forceinline__ void lds_tr16_x8(i32x2_t (&r)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}
// Eight ds_read_b64_tr_b8, issued and waited for as one block (see lds_tr16_x8).
__device__ __forceinline__ void lds_tr8_x8(i32x2_t (&r)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %8\n\t"
      "ds_read_b64_tr_b8 %1, %9\n\t"
      "ds_read_b64_tr_b8 %2, %10\n\t"
      "ds_read_b64_tr_b8 %3, %11\n\t"
      "ds_read_b64_tr_b8 %4, %12\n\t"
      "ds_read_b64_tr_b8 %5, %13\n\t"
      "ds_read_b64_tr_b8 %6, %14\n\t"
      "ds_read_b64_tr_b8 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}
// Eight 16-byte LDS reads, issued and waited for as one block (see lds_tr16_x8).
__device__ __forceinline__ void lds_b128_x8(i32x4_t (&r)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}
// Four and six 16-byte LDS reads as one self-waiting block (see lds_tr16_x8).
__device__ __forceinline__ void lds_b128_x4(i32x4_t (&r)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}
__device__ __forceinline__ void lds_b128_x6(i32x4_t (&r)[6], const uint32_t (&a)[6]) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b128 %4, %10\n\t"
      "ds_read_b128 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
      : "memory");
}
// Four ds_read_b64_tr_b8 as one self-waiting block.
__device__ __forceinline__ void lds_tr8_x4(i32x2_t (&r)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %4\n\t"
      "ds_read_b64_tr_b8 %1, %5\n\t"
      "ds_read_b64_tr_b8 %2, %6\n\t"
      "ds_read_b64_tr_b8 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const FA_LDS char* p) { return (uint32_t)(uintptr_t)p; }

__device__ __forceinline__ i32x4_t cat(i32x2_t a, i32x2_t b) {
  i32x4_t r;
  r.x = a.x; r.y = a.y; r.z = b.x; r.w = b.y;
  return r;
}

// Direct global -> LDS copy of 16 (or 4) bytes per lane; `lds` must be wave-uniform.
__device__ __forceinline__ void dma16(const void* g, FA_LDS char* lds) {
  __builtin_amdgcn_global_load_lds(g, (FA_LDS void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, FA_LDS char* lds) {
  __builtin_amdgcn_global_load_lds(g, (FA_LDS void*)lds, 4, 0, 0);
}

// Buffer resource over `bytes` bytes at `base` (raw addressing, stride 0) for the
// buffer_load ... lds form of the direct copy: the source address is an SGPR base plus a
// per-lane 32-bit offset, so no per-lane 64-bit address arithmetic is needed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// A buffer offset past any range make_rsrc describes: the load fetches nothing from memory
// (raw buffer loads range-check the offset against the record count).
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache policy of a copy (the instruction's cache-policy bits): kCacheDefault for data that is
// read again (prefill K/V tiles, shared by workgroups through L2; cache lines that several copy
// instructions read in parts, as the MLA decode's column-block copies do), kStream ("nt",
// non-temporal) for lines that one copy instruction reads whole and nothing reads again (the
// GQA decode's cache rows: 7-11 % faster there; 2.5 % slower on the prefill, and 30 % slower
// on the MLA decode's partial-line copies, whose other parts then miss L2).
constexpr int kCacheDefault = 0, kStream = 2;
template <int CPOL = kCacheDefault>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, FA_LDS char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)lds, 16, voff, 0, 0, CPOL);
}
template <int CPOL = kCacheDefault>
__device__ __forceinline__ void dma4_buf(__amdgpu_buffer_rsrc_t r, FA_LDS char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)lds, 4, voff, 0, 0, CPOL);
}
// The same 16-byte copy issued from inline asm, with the descriptor as four scalar words.
// The compiler does not track it: it adds no wait of its own before later LDS reads (it
// cannot tell which stage of a ring a copy writes), so the caller waits with wait_vmcnt
// and synchronises before reading the destination.  One wait state between the M0 write
// and the copy that reads it.
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4_t{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}
__device__ __forceinline__ void dma16_asm(const i32x4_t& rsrc, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_asm(const i32x4_t& rsrc, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that also keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value: branches on
// it then stay scalar branches instead of exec-mask regions.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// ------------------------------------------------------------------ LDS swizzles
//
// K/V tiles live in LDS as rows of keys, 16-byte chunks XOR-permuted per row.  Readers:
//  * the S^T A operand: 16 consecutive lanes read 16 consecutive rows at one logical
//    chunk, so the XOR must be one-to-one over those rows' bank phases;
//  * the transposing V reads: a 16-lane group reads 4 consecutive rows (row % 4 == 0
//    first) at one 32-byte slab (an aligned chunk pair), so those rows must land on
//    distinct chunk pairs.
// With 64 banks x 4 bytes, a 256-byte row starts every row at the same bank: swz256
// uses a 4-bit XOR, one-to-one over row % 16, with (xor >> 1) distinct over any 4
// aligned rows.  128-byte (and 1152-byte) rows alternate between two bank halves by
// parity: swz_half uses a 3-bit XOR of t = (row >> 1) % 8, one-to-one over t, with
// (xor >> 1) different for t and t + 1 when t is even (rows r and r + 2).

__device__ __forceinline__ uint32_t swz256(uint32_t row) {
  return ((row & 3u) << 2) | ((row >> 2) & 3u);
}
// The decode kernels' 16x16x32 layout reads V^T with 32 lanes covering 8 consecutive rows
// of one 32-byte column slab (and K with 16 consecutive rows of one chunk): swz16 makes the
// chunk-pair index (xor >> 1) equal row % 8 and stays one-to-one over row % 16.
__device__ __forceinline__ uint32_t swz16(uint32_t row) {
  return ((row & 7u) << 1) | ((row >> 3) & 1u);
}
// fp8 V tiles (128-byte rows, two rows per 256-byte bank row): the transposing reads of the
// decode layout gather 16 rows of one 16-byte column chunk per half-wave; this XOR of the
// chunk index is one-to-one over each parity class of those rows.
__device__ __forceinline__ uint32_t swz_fp8v(uint32_t row) {
  return ((row >> 1) & 3u) | ((row >> 2) & 4u);
}
__device__ __forceinline__ uint32_t swz_half(uint32_t row) {
  uint32_t t = (row >> 1) & 7u;
  return ((t & 1u) << 1) | ((t >> 1) & 1u) | (t & 4u);
}

// ------------------------------------------------------------------ lane exchange

__device__ __forceinline__ float bits_f(uint32_t u) { return __uint_as_float(u); }

// max / sum of x over lanes l and l ^ 32
__device__ __forceinline__ float xor32_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  uint32_t a = p[0], b = p[1];
  return fmaxf(bits_f(a), bits_f(b));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  uint32_t a = p[0], b = p[1];
  return bits_f(a) + bits_f(b);
}
// max / sum of x over lanes l and l ^ 16
__device__ __forceinline__ float xor16_max(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  uint32_t a = p[0], b = p[1];
  return fmaxf(bits_f(a), bits_f(b));
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  uint32_t a = p[0], b = p[1];
  return bits_f(a) + bits_f(b);
}

// ------------------------------------------------------------------ numerics

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + a.lo * b.lo + a.hi * b.hi over packed bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(int a, int b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc, false);
}
constexpr int kBf16PairOne = 0x3F803F80;  // packed bf16 {1.0, 1.0}

// eight e4m3fn codes (bytes of w, low byte first) -> eight bf16, exactly (every e4m3fn value
// is a bf16 value; v_cvt_scalef32_pk_bf16_fp8 with scale 1, OCP e4m3fn on gfx950)
__device__ __forceinline__ i32x4_t e4m3x8_to_bf16(i32x2_t w) {
  i32x4_t r;
  r.x = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w.x, 1.f, false));
  r.y = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w.x, 1.f, true));
  r.z = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w.y, 1.f, false));
  r.w = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w.y, 1.f, true));
  return r;
}

// two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ int pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(int, v);
}

// Online-softmax step for one query row held by a lane pair (l, l ^ 32).
// Given the tile's row max `mx` (already reduced over the pair) updates the running
// max m and returns the factor alpha = exp2((m_old - m_new) * c) that rescales the
// running sum and the O accumulator, and `neg` = -m_new * c to form exp2(s*c + neg).
// A row that has seen no visible key keeps m = -inf; its exponent base is then 0 so
// that no inf - inf appears, and alpha = 0.
struct RowState {
  float m;   // running max of the raw scores (-inf before the first visible key)
  float l;   // running sum of exp2((s - m) * c) over this lane's keys
};
__device__ __forceinline__ float softmax_rescale(RowState& st, float mx, float c, float& neg) {
  float m_new = fmaxf(st.m, mx);
  float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  float alpha = exp2_fast((st.m - m_use) * c);
  neg = -m_use * c;
  st.m = m_new;
  return alpha;
}

}  // namespace fa
