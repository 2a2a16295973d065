// Host-side launch shape choices of the GEMM sites: which tile a launch
// runs with and how far a launch that cannot fill the CUs is split over K.
// Plain host logic, kept out of the device sources so that it can be built
// and checked without a GPU compiler.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qi21_internal.h"

namespace qi21 {

// 256 x 256 tiles unless their rounds over the CUs are so much emptier
// than those of 128 x 128 tiles that the smaller kernel wins: a full round
// of 256 x 256 tiles runs about 1.4x the rate of the 128 x 128 kernel
// (measured 1.3-1.5x), so the larger tile is taken while its fill times
// 1.4 is at least the smaller tile's fill.  At 1024 rows that picks 256 x
// 256 for qkv and gate/up (192 and 384 tiles: 1.33x and 1.30x faster than
// 128 x 128) and 128 x 128 for O and down (64 tiles: 1.45x faster).  Of
// the two 256 x 256 forms the 4-wave one is taken: on the 1024^2 step it
// measured 1.7% faster than the 8-wave one (58.66 against 59.69 ms,
// interleaved), its gain coming from the long gate/up and down GEMMs.
int gemm_pick_tile(int M, int N, int K) {
  (void)K;
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
  }
  if (N % 256 != 0) return 1;
  const long t256 = (long)((M + 255) / 256) * (N / 256), t128 = (long)((M + 127) / 128) * (N / 128);
  const long r256 = (t256 + cus - 1) / cus, r128 = (t128 + cus - 1) / cus;
  // fill256 * 1.4 >= fill128, with fill = tiles / (rounds * cus)
  return t256 * 140 * r128 >= t128 * 100 * r256 ? 0 : 1;
}

// Split over K where the whole tiles of a 256 x 256 launch fill less than
// half the CUs and the 128 x 128 kernel would be picked: at 1024 rows the
// down GEMM (64 tiles of 256 x 256) runs as 256 work units of a quarter of
// K each, at the 256 x 256 kernel's rate, and the row pass that follows
// adds the partial products.  Needs at least 512 rows (two 256-row tiles).
int gemm_split_count(int M, int N, int K, int maxs) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
  }
  if (M < 512 || N % 256 != 0 || K % 64 != 0 || gemm_pick_tile(M, N, K) != 1) return 1;
  const long t = (long)((M + 255) / 256) * (N / 256);
  if (2 * t > cus) return 1;
  int sp = (int)std::min<long>(cus / t, maxs);
  while (sp > 1 && (K / 64) % sp != 0) --sp;
  return std::max(sp, 1);
}

}  // namespace qi21
