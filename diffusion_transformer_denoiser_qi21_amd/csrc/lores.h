// Device helpers of the two residual operand forms: a float operand v kept
// as hi = f16(v) plus its residual v - hi in a narrow float scaled by a
// power of two per block, for the scaled MFMAs of gfx950.  Scales are E8M0
// bytes (e + 127 for the factor 2^e).
//
// lo8: columns grouped by 128; group g of a row takes 384 bytes, the 128
// halves f16(v) and then the 128 OCP e4m3 (fp8) bytes of the scaled
// residuals, so a GEMM walks a row in 128-byte k-tiles of two f16 k-tiles
// and one fp8 k-tile per group.  Activations: one scale per 64 columns,
// two per group.
//
// lo4: columns grouped by 256; group g takes 640 bytes, the 256 halves
// and then 128 bytes of e2m1 (fp4) residuals, two per byte (the even
// column in the low nibble): four f16 k-tiles and one fp4 k-tile per
// group.  One scale per 32 columns (the MX block), eight per group: byte
// 4 h + s of the group for the block 2 s + h.  That is the order in which
// the lanes of a 32 x 32 x 64 fp4 MFMA take them (k-step s of the fp4
// k-tile, lane half h): a lane reads its four k-steps' scales as one
// dword.  The 16 x 16 x 128 fp4 MFMA's lane group g (of four) takes
// block g in k-step 0 and block 4 + g in k-step 1: bytes g / 2 and
// g / 2 + 2 of the dword at 4 (g % 2).
//
// Scale arrays are blocked by 256 rows and, inside a block, ordered group
// by group: the bytes of rows r .. r + 31 for one group sit next to each
// other, so the 32 rows a GEMM lane group reads at once come from a few
// cache lines.  With q scale bytes per group and G groups per row, the
// byte of row r, group g, position b is
//   (r / 256) * 256 G q + g * 256 q + (r % 256) * q + b
// (an array holds whole blocks: round_up(rows, 256) rows).
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

// lo4 positions: halves offset of column c's f16 value, byte of the pair
// (c, c + 1) (c even)
__device__ __forceinline__ int lo4_hi_at(int c) { return (c >> 8) * 320 + (c & 255); }
__device__ __forceinline__ int lo4_lo_at(int c) { return (c >> 8) * 640 + 512 + ((c & 255) >> 1); }

// scale byte of row r, column c in a blocked scale array of rows of w
// columns (see above): lo8 (q = 2 per 128-column group), lo4 (q = 8 per
// 256-column group, the block 2 s + h of the group at 4 h + s)
__device__ __forceinline__ size_t lo8_sc_at(int r, int c, int w) {
  return (size_t)(r >> 8) * 256 * (w >> 6) + (size_t)(c >> 7) * 512 + (r & 255) * 2 + ((c >> 6) & 1);
}
__device__ __forceinline__ size_t lo4_sc_at(int r, int c, int w) {
  const int b = (c & 255) >> 5;
  return (size_t)(r >> 8) * 256 * (w >> 5) + (size_t)(c >> 8) * 2048 + (r & 255) * 8 + 4 * (b & 1) + (b >> 1);
}

// Scale exponent of an fp4 block whose largest magnitude is mx: the
// smallest e with mx 2^-e <= 6 (e2m1's largest value), so nothing
// saturates: mx 2^-e lands in [4, 6] or (3, 4); clamped to E8M0's range.
__device__ __forceinline__ int lo4_exp(float mx) {
  const unsigned b = __float_as_uint(mx);
  const int be = (int)((b >> 23) & 0xff);
  const int e = be - 127 - ((b & 0x7fffff) <= 0x400000 ? 2 : 1);
  return max(-127, min(127, e));
}

// four f32 values (within +-6) -> four e2m1 nibbles in 16 bits, the first
// value in the lowest nibble
__device__ __forceinline__ unsigned pack_e2m1(float a, float b, float c, float d) {
  const unsigned w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c, d, 1.0f, 1) & 0xffffu;
}

}  // namespace qi21
