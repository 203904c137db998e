// Per-token e4m3 quantisation: the step that produces the e4m3 nope operands and their
// fp32 per-row scales consumed by the per-token-scale MLA prefill (Modular's
// "MLASmemStorage" page keeps one fp32 scale per Q-tile row and per K-tile row next to
// the fp8 nope tiles).  For every row x of fp32 values:
//   scale = fl32(amax |x| / 448)   (1 for an all-zero row; 448 = the largest e4m3fn value)
//   code_j = e4m3fn(fl32(x_j / scale)), round to nearest even (gfx950's fp8 conversion
//            produces the OCP e4m3fn format)
// The kernel is a streaming pass (5 bytes moved per element): a row is handled by Lr
// lanes of one wave (Lr = the smallest power of two with 4 Lr >= cols, at most 64), each
// lane loading 16-byte groups of four values.  Loads and stores carry the non-temporal
// cache policy (each byte is touched once): 15 % faster than the default.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int QZ_SLOTS = 16;  // 16-byte groups a lane holds at once (cols <= 64 * 4 * 16 = 4096)

// max over the Lr lanes (a power of two) that share a row, by exchanges within the wave:
// quad permutations for lanes 1 and 2 apart, the half-row and row mirrors to cover 8 and
// 16 lanes (max is idempotent, so any pairing that joins the groups will do), then the
// 16- and 32-lane swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_max(float v, int Lr) {
  if (Lr >= 2) v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  if (Lr >= 4) v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  if (Lr >= 8) v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  if (Lr >= 16) v = fmaxf(v, dpp_f<0x140>(v)); // row_mirror
  if (Lr >= 32) v = xor16_max(v);
  if (Lr >= 64) v = xor32_max(v);
  return v;
}

// NK: 16-byte groups per lane per row (a power of two); a wave takes QZ_SLOTS / NK row
// groups of 64 / Lr rows and issues every load before converting, so each wave keeps up
// to 16 KiB of reads in flight.
template <int NK>
__global__ __launch_bounds__(256) void quantize_rows_kernel(QuantArgs a) {
  constexpr int NG = QZ_SLOTS / NK;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int Lr = a.lanes_per_row;
  const int rpg = 64 / Lr;  // rows per group
  const int li = lane & (Lr - 1), rw = lane / Lr;
  const long long row0 = ((long long)blockIdx.x * 4 + wave) * NG * rpg + rw;
  const int cols = a.cols;

  f32x4_t v[NG][NK];
#pragma unroll
  for (int g = 0; g < NG; g++) {
    const long long row = row0 + (long long)g * rpg;
#pragma unroll
    for (int k = 0; k < NK; k++) {
      const int j = 4 * li + 4 * Lr * k;
      v[g][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (row < a.n_rows && j < cols) v[g][k] = __builtin_nontemporal_load((const f32x4_t*)(a.x + row * cols + j));
    }
  }
#pragma unroll
  for (int g = 0; g < NG; g++) {
    const long long row = row0 + (long long)g * rpg;
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < NK; k++)
#pragma unroll
      for (int i = 0; i < 4; i++) mx = fmaxf(mx, fabsf(v[g][k][i]));
    mx = row_max(mx, Lr);
    const float sc = mx > 0.f ? mx / 448.f : 1.f;
    if (row < a.n_rows) {
      uint8_t* cr = a.codes + row * cols;
#pragma unroll
      for (int k = 0; k < NK; k++) {
        const int j = 4 * li + 4 * Lr * k;
        if (j < cols) {
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[g][k][0] / sc, v[g][k][1] / sc, 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(v[g][k][2] / sc, v[g][k][3] / sc, w, true);
          __builtin_nontemporal_store(w, (int*)(cr + j));
        }
      }
      if (li == 0) a.scale[row] = sc;
    }
  }
}

}  // namespace

hipError_t launch_quantize_rows(const QuantArgs& a, hipStream_t s) {
  const int Lr = a.lanes_per_row;
  int nk = (a.cols + 4 * Lr - 1) / (4 * Lr);
  int NK = 1;
  while (NK < nk) NK <<= 1;
  const long long rows_per_block = 4LL * (QZ_SLOTS / NK) * (64 / Lr);
  const long long grid = (a.n_rows + rows_per_block - 1) / rows_per_block;
  if (grid == 0) return hipSuccess;
  switch (NK) {
    case 1: quantize_rows_kernel<1><<<(unsigned)grid, 256, 0, s>>>(a); break;
    case 2: quantize_rows_kernel<2><<<(unsigned)grid, 256, 0, s>>>(a); break;
    case 4: quantize_rows_kernel<4><<<(unsigned)grid, 256, 0, s>>>(a); break;
    case 8: quantize_rows_kernel<8><<<(unsigned)grid, 256, 0, s>>>(a); break;
    case 16: quantize_rows_kernel<16><<<(unsigned)grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fa
