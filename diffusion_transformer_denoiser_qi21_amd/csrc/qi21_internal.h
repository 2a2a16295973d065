// Internal launch interface of the qi21 kernels (gfx950 / CDNA4).
//
// Every launcher takes device pointers and a HIP stream and assumes its
// shape arguments were validated by the caller (qi21_api.cpp checks them
// on the host before any launch); the comment on each one states what it
// assumes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qi21 {

typedef _Float16 f16;

// s_waitcnt immediate (gfx9 encoding): vmcnt 6 bits at [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; the maximum of a field means "no wait".
constexpr int wait_imm(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | ((lgkm & 0xF) << 8);
}

enum Epi { EPI_F16 = 0, EPI_F32 = 1, EPI_SWIGLU = 2, EPI_QKV = 3, EPI_SWIGLU2 = 4, EPI_QKROPE = 5, EPI_VT = 6,
           EPI_RESID = 7, EPI_GELU = 8, EPI_SWIGLU8 = 9, EPI_SWIGLU4 = 10 };

// C = A * W^T over f16 operands with f32 accumulation.
//   A: [M][lda] f16 (K contiguous), W: [N][kw] f16 (kw contiguous); column
//   k of A meets column k % kw of W, so with kw = K / 2 an A row holding
//   [hi | lo] halves of a float operand is multiplied by W twice.
//   EPI_F16:    out f16 [M][ldo] = acc * oscale
//   EPI_F32:    out f32 [M][ldo] = acc * oscale
//   EPI_SWIGLU: W is the interleaved gate/up plane (groups of 32 gate rows,
//               then the 32 matching up rows); out f16 [M][ldo] with N/2
//               columns = silu(g*inscale) * (u*inscale) * oscale
//   EPI_SWIGLU2: as EPI_SWIGLU, the value h written as the pair
//               out[r][c] = f16(h), out[r][N/2 + c] = f16(h - f16(h))
//   EPI_SWIGLU8 / EPI_SWIGLU4: as EPI_SWIGLU, h written in the lo8 / lo4
//               row form (lores.h): out row r (ldo halves) holds f16(h) and
//               the scaled residuals of its N/2 columns, with the scales in
//               the blocked array osc.  Large-M 4-wave kernel only.
//   EPI_QKROPE: N = 2H, W = the q then k projection rows; per row and
//               128-column head: RMSNorm of the accumulators (weights nq for
//               q heads, nk for k heads, eps in the accumulators' scale),
//               then interleaved-pair RoPE with the packed table rope
//               [M][128] (launch_rope_pack); q heads
//               to out f16 [M][ldo], k heads to kout f16 [M][ldk] (column
//               c - H).  Large-M kernels only (tile 0 / 2).
//   EPI_VT:     out f16 [M][ldo] = acc * oscale with output column c stored at
//               vt_pos(c) and only columns c < nvalid (V^T from Wv and the
//               rows as the W operand).  Large-M kernels only.
//   EPI_GELU:   out f16 [M][ldo] = gelu_tanh(acc * inscale) * oscale
//   EPI_RESID:  out f32 [M][ldo] += gate[c] * acc * oscale (the gated residual
//               of a block's branch, x += tanh(g) y, in place)
//   EPI_QKV:    columns [0, 2H) -> out f16 [M][ldo] (q|k), columns [2H, 3H)
//               -> out2 f16 transposed, out2[c - 2H][row] with leading
//               dimension ld2 (V^T), both * oscale; H = N/3.
// Residual operands (lo = 8 or 4; large-M 4-wave kernel, row-layout
// epilogues): A and W rows are in the lo8 / lo4 row form (lores.h), K
// counting the halves of the whole row (1.5 / 1.25 times the columns), so
// of every 3 / 5 k-tiles the last holds the residuals of the columns the
// others hold as halves, multiplied on the scaled fp8 / fp4 MFMA.  Scales
// (blocked by 256 rows, lores.h): lo8, A's per 64 columns in asc (lds =
// K / 64 bytes per row), W's one per row in wsc[n]; lo4, A's and W's per
// 32 columns in asc / wsc (lds = ldws = K / 32).  The arrays hold whole
// 256-row blocks.  osc (EPI_SWIGLU8 / 4): the hidden's, blocked likewise.
// kw = K (no wrap), ldw the W row stride.
// Assumes: N % 128 == 0, K % 64 == 0, kw % 64 == 0, K % kw == 0, M >= 1,
// 16-byte aligned rows (lda a multiple of 8), for EPI_QKV N/3 % 128 == 0
// and ld2 >= M.
struct GemmArgs {
  int M, N, K;
  const f16* A; int lda;
  const f16* W; int kw;
  int ldw = 0;  // W row stride in halves (0: kw)
  // residual operands (see above): 0 none, 8 lo8, 4 lo4
  int lo = 0;
  const uint8_t* asc = nullptr; int lds = 0;
  const uint8_t* wsc = nullptr; int ldws = 0;
  // EPI_SWIGLU8 / EPI_SWIGLU4 output scales
  uint8_t* osc = nullptr;
  void* out; int ldo;
  f16* out2; int ld2;
  float oscale, inscale;
  // EPI_QKROPE
  const float* nq = nullptr; const float* nk = nullptr;
  const float* rope = nullptr;  // [M][128]: per two pairs (2m, 2m+1): cos 2m, cos 2m+1, sin 2m, sin 2m+1
  float eps = 0.0f;
  f16* kout = nullptr; int ldk = 0;
  // EPI_VT
  int nvalid = 0;
  // EPI_RESID
  const float* gate = nullptr;
  // split over K (256 x 256 kernels, EPI_F32 only): work unit u covers tile
  // u % tiles over k-tiles [(u / tiles) KT / ksplit, ...) and writes its
  // partial product to out + (u / tiles) * pstride (floats)
  int ksplit = 1;
  size_t pstride = 0;
};
hipError_t launch_gemm(int epi, const GemmArgs& a, int tile, hipStream_t s);
// the tile a launch would pick (0: 256x256, 1: 128x128, ...)
int gemm_pick_tile(int M, int N, int K);

// Flash attention, head_dim 128, over up to two key sources.  Keys
// [0, n1) come from source 1 (K rows k1 + j*ldk1 + h*128, V^T rows
// vt1 + (h*128 + d)*ldvt1 + j), keys [n1, n1+n2) from source 2 likewise.
// Query i sees keys j < vis[i] when vis != nullptr (vis non-decreasing,
// 1 <= vis[i] <= n1 + n2), else all keys.  out f16 [nq][ldo] at column
// h*128 = softmax(q k^T / sqrt(128)) V * oscale.
// Assumes: V^T leading dimensions are multiples of 8 and at least
// round_up(n, 64) with finite (zeroed) padding; K rows 16-byte aligned.
struct FlashArgs {
  const f16* q; int ldq; int nq; int heads;
  const f16* k1; int ldk1; const f16* vt1; int ldvt1; int n1;
  const f16* k2; int ldk2; const f16* vt2; int ldvt2; int n2;
  const uint32_t* vis;
  f16* out; int ldo;
  float oscale;
};
hipError_t launch_flash(const FlashArgs& a, hipStream_t s);
// The segments' blocks in launches of two segments each (the rows of two
// programs, each attending to its own keys; combined grids fill the CUs
// where one program's rows would not).
hipError_t launch_flash(const FlashArgs* segs, int nseg, hipStream_t s);

// rowop over `rows` rows of width h (h % 4 == 0, h <= 8192):
//   mode & 1: x += gate (.) y            (gate = mods + g_off, already tanh-ed;
//             y = the sum of nparts planes [rows][h] pstride floats apart)
//   mode & 2: xn = f16(LN(x) * (1 + mods[s_off + c]) * oscale)
//   mode & 4: (with & 2) xn is [rows][2h]: the value v as the pair
//             xn[r][c] = f16(v), xn[r][h + c] = f16(v - f16(v))
//   mode & 8: (with & 2, not with & 4) xn rows of 3h bytes in the lo8 row
//             form (lores.h): f16(v) and e4m3((v - f16(v)) 2^-e), e per 64
//             columns in the blocked scale array xsc; h % 128 == 0
//   mode & 16: (with & 2 only) the lo4 row form, rows of 2.5h bytes, e per
//             32 columns in the blocked array xsc; h % 256 == 0
// ldxn: xn's row stride in halves (0: h, 2h, 1.5h or 1.25h as the mode implies;
// otherwise at least that, and a multiple of 4)
hipError_t launch_rowop(int rows, int h, int mode, float* x, const float* y, f16* xn,
                        const float* mods, int g_off, int s_off, float eps, float oscale,
                        hipStream_t s, int nparts = 1, size_t pstride = 0, uint8_t* xsc = nullptr, int ldxn = 0);
// How many K splits a 256 x 256 GEMM of this shape should run with so its
// work units fill the CUs where whole tiles would not (1: no split); at
// most maxs, and K / 64 divisible by it.
int gemm_split_count(int M, int N, int K, int maxs);

// txt_in norm over rows of width c (c % 4 == 0, c <= 8192): xn f16 =
// f32(v / sqrt(mean(v^2) + eps)) * (w + 1), float64 sum of squares
hipError_t launch_txtnorm(int rows, int c, const float* feats, const float* w, float eps, f16* xn, hipStream_t s);

// Per-head RMSNorm(w) + interleaved RoPE on the q and k columns of the
// panel (q at column 0, k at column heads*128, row stride ldp), in place.
// If kdst != nullptr the normalised k goes to kdst[row][ldk] instead.
// cos/sin: [rows][64] f32.  eps is the norm's eps (already scaled for the
// panel's range guard).
hipError_t launch_qkrope(int rows, int heads, f16* panel, int ldp, const float* norm_q,
                         const float* norm_k, const float* cosb, const float* sinb, float eps,
                         f16* kdst, int ldk, hipStream_t s);

// x[r][c] = sum_k tok[r][k] * img_in[c][k], k < 64, f32.  h % 64 == 0.
hipError_t launch_embed(int rows, int h, const float* tok, const float* img_in, float* x,
                        hipStream_t s);

// out[r][o] = sum_c (LN(x[r])[c] * fs[c]) * proj_out[o][c], o < 64, f32;
// sets *flag |= 1 when any output is not finite.  h % 256 == 0.
hipError_t launch_final(int rows, int h, const float* x, const float* fs, const float* proj_out,
                        float eps, float* out, int* flag, hipStream_t s);

// dst[i] = flag == 0 ? src[i] : dst[i], i < count (count % 4 == 0).
hipError_t launch_commit(int count, const float* src, float* dst, const int* flag, hipStream_t s);

// mods_dev = [s1 | tanh g1 | s2 | tanh g2] from the raw [4h] modulation.
hipError_t launch_mods(int h, const float* mods, float* mods_dev, hipStream_t s);

// Weight conversion to f16: dst row (r / group) * gstride + goff + r % group
// (ld = cols) receives source row r.  src_dtype 0 f32, 1 bf16, 2 f16.
// ldd: dst row stride in halves (0: cols); lo = 8 / 4: dst rows in the
// lo8 / lo4 row form (f16 values at their lores.h positions; cols % 128 /
// 256 == 0).
hipError_t launch_plane(int src_dtype, const void* src, int rows, int cols, f16* dst, int group,
                        int gstride, int goff, hipStream_t s, int ldd = 0, int lo = 0);
// The fp4 part of a lo4 weight plane whose f16 values are set: per row and
// 32-column block, e with the block's largest |w| 2^-e <= 6 (the smallest
// such), the residual nibbles e2m1(w 2^-e) and the scale byte e + 127 in
// the blocked array sc (whole 256-row blocks).  cols % 256 == 0.
hipError_t launch_plane4(int rows, int cols, f16* plane, int ld, uint8_t* sc, hipStream_t s);
// The fp8 part of a lo8 weight plane (rows of ld halves in the lo8 row
// form whose f16 values are set): each row's residual bytes become
// e4m3(w 2^-e), w the f16 value, e per row such that the row's largest
// |w| 2^-e lies in [128, 256), and sc[r] = e + 127 (E8M0).  cols % 128 == 0.
hipError_t launch_plane8(int rows, int cols, f16* plane, int ld, uint8_t* sc, hipStream_t s);

// The time path ([QI] Qi21Dit::temb / mods): mods [4h] (raw [s1|g1|s2|g2])
// and fs [h] = 1 + final_scale of model time t, from f32 weights t_lin1
// [h][256], t_lin2 [h][h], modulation [4h][h], norm_out [h][h]; work holds
// 256 + 2h floats.  h % 4 == 0.
hipError_t launch_time_mods(int h, float t, const float* t_lin1, const float* t_lin2, const float* modulation,
                            const float* norm_out, float* work, float* mods, float* fs, hipStream_t s);

// x[i] += dt v[i], i < n (product and sum rounded separately)
hipError_t launch_axpy(int n, float dt, const float* v, float* x, hipStream_t s);

// dst f32 [n] = src (src_dtype 0 f32, 1 bf16, 2 f16)
hipError_t launch_to_f32(int src_dtype, const void* src, size_t n, float* dst, hipStream_t s);

// fill count 32-bit words with value (a kernel, so it is safe to capture)
hipError_t launch_fill32(void* p, uint32_t value, size_t count, hipStream_t s);
// dst[i] = src[i] * f, i < n (device pointers; in place allowed)
hipError_t launch_scale(int n, const float* src, float f, float* dst, hipStream_t s);
// RoPE tables cos / sin [n][64] packed into out [n][128] for the q|k GEMM
// epilogue: out[r][4m + (0, 1, 2, 3)] = cos[r][2m], cos[r][2m + 1],
// sin[r][2m], sin[r][2m + 1]
hipError_t launch_rope_pack(int n, const float* cos, const float* sin, float* out, hipStream_t s);

}  // namespace qi21
