// Host-only planning arithmetic shared by the C ABI (api.cpp: validation and workspace
// sizes) and the kernel launchers: the split-KV plans of the decode kernels and the row
// layout of the quantiser.  No HIP calls; built into libattn.so and, for the CPU sanitizer
// tests, into a host-only library with api.cpp.
#include <algorithm>

#include "launch.h"

namespace fa {

using std::max;
using std::min;

SplitPlan gqa_decode_plan(int B, int Hkv, int max_len) {
  int chunk = 1024;
  // one wave per (split, batch, kv head): keep at least ~2048 of them for small batches or
  // few kv heads
  while (chunk > kDecodeTileKeys && (long)B * Hkv * ((max_len + chunk - 1) / chunk) < 2048) chunk /= 2;
  SplitPlan p;
  p.chunk = chunk;
  p.n_split = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
  return p;
}

SplitPlan mla_decode_plan(int B, int H, int max_len) {
  (void)H;
  // one workgroup per CU: aim for >= 256 workgroups in total
  int want = B > 0 ? (256 + B - 1) / B : 1;
  int n_tiles = max_len > 0 ? (max_len + kDecodeTileKeys - 1) / kDecodeTileKeys : 1;
  want = max(1, min(want, n_tiles));
  int chunk = ((n_tiles + want - 1) / want) * kDecodeTileKeys;
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

int quantize_lanes_per_row(int cols) {
  int lr = 1;
  while (lr < 64 && 4 * lr < cols) lr <<= 1;
  return lr;
}

}  // namespace fa
