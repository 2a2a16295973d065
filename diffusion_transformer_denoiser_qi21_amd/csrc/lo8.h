// Device helpers of the lo8 operand form: a float operand v kept as
// hi = f16(v) plus its residual v - hi in OCP e4m3 (fp8) scaled by a power
// of two per block, for the scaled fp8 MFMA of gfx950.
//
// Row layout: columns are grouped by 128; group g of a row takes 384
// bytes, the 128 halves f16(v) and then the 128 e4m3 bytes of the scaled
// residuals, so a GEMM walks a row in 128-byte k-tiles of two f16 k-tiles
// and one fp8 k-tile per group.  Scales are E8M0 bytes (e + 127 for 2^e).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qi21 {

// halves offset of column c's f16 value, byte offset of its fp8 residual
__device__ __forceinline__ int lo8_hi_at(int c) { return (c >> 7) * 192 + (c & 127); }
__device__ __forceinline__ int lo8_lo_at(int c) { return (c >> 7) * 384 + 256 + (c & 127); }

// Scale exponent of a block whose largest magnitude is mx: e with mx 2^-e in
// [128, 256), so every element fits e4m3 (largest finite 448) with a
// binade of headroom; clamped to E8M0's range (byte e + 127 in [0, 254]).
__device__ __forceinline__ int lo8_exp(float mx) {
  const int be = (int)((__float_as_uint(mx) >> 23) & 0xff);  // biased exponent (0: zero or subnormal)
  return max(-127, min(127, be - 127 - 7));
}

// four f32 values -> four e4m3 bytes (round to nearest even), first value
// in the lowest byte
__device__ __forceinline__ unsigned pack_e4m3(float a, float b, float c, float d) {
  const unsigned w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
}

}  // namespace qi21
