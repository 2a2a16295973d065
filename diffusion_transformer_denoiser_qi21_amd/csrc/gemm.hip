// MFMA GEMM of the denoiser's four projection sites (qkv, O, gate/up, down).
//
// C[M][N] = A[M][K] * W[N][K]^T with f16 operands and f32 accumulation.
// Both operands are K-contiguous in HBM (activations row-major, weight
// planes [out][in]), which is exactly the layout the MFMA A and B
// fragments want, so no operand is ever transposed.
//
// Three kernels share the tile walk, the LDS layout and the loads:
//
// * gemm16_kernel, the large-M kernel of the step: block tile 256 x 256 x
//   64, 4 waves of 128 x 128 on v_mfma_f32_16x16x32_f16 (lo4: plus the
//   scaled fp4 MFMA), 2 LDS stages filled by buffer loads that write
//   straight into LDS (no register staging).  Each load reads 8 whole
//   128-byte rows, which the L2 -> CU path serves about 1.4x faster than
//   16 half rows.  A-rows past M come back as zeros from the buffer
//   resource's range check.  The main loop is branch-free and its
//   schedule is pinned; one barrier per k-tile, after which all loads of
//   the k-tile two ahead go out.
// * gemm_dma_kernel, the same tile on v_mfma_f32_32x32x16_f16: the lo8 form,
//   the 8-wave form (128 x 64 per wave) and work units with an odd number
//   of k-tiles.
// * gemm_rs_kernel, the small-M / narrow-N kernel: block tile BM x BN x 64,
//   global -> registers -> LDS, double-buffered.
//
// LDS rows hold the k-slice of one A or W row in 16-byte chunks, XOR-
// swizzled so the 16-byte fragment reads of 16 consecutive rows fall on 16
// different bank groups.  Blocks are dealt to the 8 XCDs round-robin; the
// launch remaps them so each XCD works on a compact 4-row group of tiles
// (A and W slices shared in that XCD's L2).
//
// Epilogues (fused, from the accumulators): f16 store, f32 store, the
// SwiGLU of the interleaved gate/up plane, and the qkv split that writes
// the v columns transposed (V^T, the layout the attention kernel streams).
// Range-guard factors are powers of two folded into oscale / inscale.
#include "qi21_internal.h"
#include "lores.h"

#include <algorithm>

namespace qi21 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

// silu through the hardware reciprocal (~1 ulp; the result is stored as f16)
__device__ __forceinline__ float silu_f(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// the tanh approximation of GELU (stored as f16)
__device__ __forceinline__ float gelu_f(float v) {
  return 0.5f * v * (1.0f + tanhf(0.7978845608028654f * (v + 0.044715f * v * v * v)));
}

// Block -> (tile row, tile column).  Hardware deals block b to XCD b % 8;
// blocks of one XCD get a contiguous run of tiles, enumerated in groups of
// 4 tile rows so that the ~32 tiles an XCD runs at once span 4 A panels and
// 8 W panels instead of 1 and 32.
__device__ __forceinline__ void tile_of(int M, int N, int BM, int BN, int& tm, int& tn) {
  const int tiles_n = N / BN, tiles_m = (M + BM - 1) / BM;
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int G = 4;
  if (tiles_m % G == 0) {
    const int per = G * tiles_n;
    const int g = bid / per, w = bid - g * per;
    tm = g * G + w % G;
    tn = w / G;
  } else {
    tm = bid / tiles_n;
    tn = bid - tm * tiles_n;
  }
}

// Position of key (row) r in a V^T row: bits 2 and 3 of r swapped, which
// keeps runs of 4 keys contiguous and gathers keys {4h..4h+3, 8+4h..8+4h+3}
// of every 16 into one 16-byte chunk (the attention kernel's P V operand).
__device__ __forceinline__ int vt_pos(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// The 32 columns of a row that a 32 x 32 accumulator tile gives two lanes:
// lane l (hsel 0) holds the 4-column chunks 0, 2, 4, 6 (in its g = 0..3
// parts) and lane l + 32 the chunks 1, 3, 5, 7.  One lane-half swap per
// register makes the runs contiguous.  pair_halves: chunks of 4 halves; the
// lower lane returns columns 0..7 and 16..23, the upper 8..15 and 24..31
// (vector k goes to column 16 k + 8 hsel).  pair_words: chunks of 4 bytes;
// the lower lane returns the bytes of columns 0..15, the upper those of
// 16..31 (at byte 16 hsel).  Every lane must take part.
__device__ __forceinline__ void pair_halves(const half4 (&h)[4], u32x4 (&out)[2]) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const u32x2 x = __builtin_bit_cast(u32x2, h[2 * k]), y = __builtin_bit_cast(u32x2, h[2 * k + 1]);
    const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false);
    out[k] = u32x4{s0[0], s1[0], s0[1], s1[1]};
  }
}
__device__ __forceinline__ u32x4 pair_words(const unsigned (&q)[4]) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(q[0], q[2], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(q[1], q[3], false, false);
  return u32x4{s0[0], s0[1], s1[0], s1[1]};
}

// Epilogue of a wave whose output rows [r0, r0 + 32 TM) and columns
// [c0, c0 + 32 TN) were accumulated with the W fragment as the MFMA's A
// operand (C^T = W A^T): the 32x32 accumulator layout (lane l holds
// column l % 32, rows 8g + 4(l / 32) + e in register 4g + e) then gives
// lane l output row r0 + 32i + l % 32 and the 4 consecutive output columns
// c0 + 32j + 8g + 4(l / 32) + (0..3) in registers 4g..4g+3, written as one
// 16-byte (f32) or 8-byte (f16) store.  Requires ldo % 4 == 0.
template <int EPI, int TM, int TN>
__device__ __forceinline__ void epilogue_rows(const GemmArgs& a, floatx16 (&acc)[TM][TN], int r0, int c0, int lane,
                                              size_t obase = 0) {
  const int hsel = lane >> 5, l32 = lane & 31;
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + i * 32 + l32;
      if (row < a.M) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = c0 + j * 32 + 8 * g + 4 * hsel;
            floatx4* xp = reinterpret_cast<floatx4*>(reinterpret_cast<float*>(a.out) + (size_t)row * a.ldo + c);
            const floatx4 gt = *reinterpret_cast<const floatx4*>(a.gate + c);
            floatx4 x = *xp;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(gt[e], acc[i][j][4 * g + e] * a.oscale, x[e]);
            *xp = x;
          }
      }
    }
  } else if constexpr (EPI == EPI_F16 || EPI == EPI_GELU) {
    // f16 rows: 16-byte stores through the lane-half swap
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + i * 32 + l32;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        half4 h[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          floatx4 v = floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          if constexpr (EPI == EPI_GELU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu_f(v[e] * a.inscale);
          }
          v = v * a.oscale;
          h[g] = half4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
        }
        u32x4 hv[2];
        pair_halves(h, hv);
        if (row < a.M) {
#pragma unroll
          for (int k = 0; k < 2; ++k)
            *reinterpret_cast<u32x4*>(reinterpret_cast<f16*>(a.out) + obase + (size_t)row * a.ldo + c0 + j * 32 +
                                      16 * k + 8 * hsel) = hv[k];
        }
      }
    }
  } else if constexpr (EPI == EPI_F32) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + i * 32 + l32;
      if (row < a.M) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const size_t o = obase + (size_t)row * a.ldo + c0 + j * 32 + 8 * g + 4 * hsel;
            const floatx4 v =
                floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]} * a.oscale;
            *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(a.out) + o) = v;
          }
      }
    }
  } else if constexpr (EPI == EPI_QKROPE) {
    // the wave's TN = 4 column tiles are one 128-column head (c0 % 128 == 0);
    // lanes l and l ^ 32 hold the two halves of a row
    static_assert(TN == 4, "a wave spans one head");
    const int H = a.N / 2;
    const bool isk = c0 >= H;
    const float* nw = isk ? a.nk : a.nq;
    f16* dst = isk ? a.kout + (c0 - H) : reinterpret_cast<f16*>(a.out) + c0;
    const int ld = isk ? a.ldk : a.ldo;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + i * 32 + l32;
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) ss = __builtin_fmaf(acc[i][j][e], acc[i][j][e], ss);
      {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
      const float inv = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
      // the row's packed table: cos and sin of the lane's two pairs in one
      // 16-byte load (rows past M read the last row; their results are not
      // stored, but every lane takes part in the swaps)
      const float* tr = a.rope + (size_t)min(row, a.M - 1) * 128;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        half4 h[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = j * 32 + 8 * g + 4 * hsel;  // dims d .. d+3: pairs d/2, d/2 + 1
          const floatx4 w = *reinterpret_cast<const floatx4*>(nw + d);
          const floatx4 t = *reinterpret_cast<const floatx4*>(tr + d);  // cos d/2, d/2+1, sin d/2, d/2+1
          const floatx2 cs = floatx2{t[0], t[1]}, sn = floatx2{t[2], t[3]};
          const float a0 = (acc[i][j][4 * g] * inv) * w[0], b0 = (acc[i][j][4 * g + 1] * inv) * w[1];
          const float a1 = (acc[i][j][4 * g + 2] * inv) * w[2], b1 = (acc[i][j][4 * g + 3] * inv) * w[3];
          h[g] = half4{(f16)(a0 * cs[0] - b0 * sn[0]), (f16)(a0 * sn[0] + b0 * cs[0]), (f16)(a1 * cs[1] - b1 * sn[1]),
                       (f16)(a1 * sn[1] + b1 * cs[1])};
        }
        u32x4 hv[2];
        pair_halves(h, hv);
        if (row < a.M) {
#pragma unroll
          for (int k = 0; k < 2; ++k)
            *reinterpret_cast<u32x4*>(dst + (size_t)row * ld + j * 32 + 16 * k + 8 * hsel) = hv[k];
        }
      }
    }
  } else if constexpr (EPI == EPI_VT) {
    // output rows are V dims, columns are keys: key c goes to vt_pos(c),
    // which keeps aligned runs of 4 together.  Columns from nvalid up to
    // the leading dimension (whole groups of 16, within which vt_pos
    // permutes) get zeros: the attention kernel reads whole 64-key tiles
    // and multiplies the columns past the keys by P = 0, which must not
    // meet a stale non-finite value.
    const int cz = a.ldo & ~15;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + i * 32 + l32;
      if (row < a.M) {
        f16* orow = reinterpret_cast<f16*>(a.out) + (size_t)row * a.ldo;
        // keys base + 4 hsel .. + 3 (chunk 2m) and base + 8 + 4 hsel .. + 3
        // (chunk 2m + 1) land at positions base + 8 hsel .. + 7: one 16-byte
        // store.  A group of 16 keys is below cz whole or not at all, and the
        // host guarantees nvalid <= cz.
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const int base = c0 + j * 32 + 16 * m;
            if (base < cz) {
              half8 v;
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int c = base + 8 * h + 4 * hsel;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  v[4 * h + e] = c + e < a.nvalid ? (f16)(acc[i][j][4 * (2 * m + h) + e] * a.oscale) : (f16)0.0f;
              }
              *reinterpret_cast<half8*>(orow + base + 8 * hsel) = v;
            }
          }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU8) {
    // the wave's 4 column tiles are 64 hidden columns, one scale block per
    // row: lanes l and l ^ 32 hold its two halves
    static_assert(TN == 4, "a wave spans one 64-column scale block");
    const int hc = c0 / 2;  // first hidden column of the wave
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + i * 32 + l32;
      half4 hi[2][4];
      floatx4 lo[2][4];
      float mx = 0.0f;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float h = silu_f(acc[i][2 * p][4 * g + e] * a.inscale) * (acc[i][2 * p + 1][4 * g + e] * a.inscale) *
                            a.oscale;
            hi[p][g][e] = (f16)h;
            lo[p][g][e] = h - (float)hi[p][g][e];  // exact in f32
            mx = fmaxf(mx, fabsf(lo[p][g][e]));
          }
      {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      const int ex = lo8_exp(mx);
      const float inv = __builtin_ldexpf(1.0f, -ex);
      // contiguous runs through the lane-half swap (every lane takes part;
      // rows past M skip the stores)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        unsigned q[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const floatx4 v = lo[p][g] * inv;
          q[g] = pack_e4m3(v[0], v[1], v[2], v[3]);
        }
        const u32x4 codes = pair_words(q);
        u32x4 hv[2];
        pair_halves(hi[p], hv);
        if (row < a.M) {
          f16* orow = reinterpret_cast<f16*>(a.out) + (size_t)row * a.ldo;
          uint8_t* brow = reinterpret_cast<uint8_t*>(orow);
#pragma unroll
          for (int k = 0; k < 2; ++k)
            *reinterpret_cast<u32x4*>(orow + lo8_hi_at(hc + p * 32 + 16 * k + 8 * hsel)) = hv[k];
          *reinterpret_cast<u32x4*>(brow + lo8_lo_at(hc + p * 32) + 16 * hsel) = codes;
        }
      }
      if (row < a.M && hsel == 0) a.osc[lo8_sc_at(row, hc, a.N / 2)] = (uint8_t)(ex + 127);
    }
  } else if constexpr (EPI == EPI_SWIGLU4) {
    // the wave's 4 column tiles are 64 hidden columns, two 32-column scale
    // blocks p per row: lanes l and l ^ 32 hold the two halves of each
    static_assert(TN == 4, "a wave spans two 32-column scale blocks");
    const int hc = c0 / 2;  // first hidden column of the wave
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + i * 32 + l32;
      half4 hi[2][4];
      floatx4 lo[2][4];
      float mx[2] = {0.0f, 0.0f};
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float h = silu_f(acc[i][2 * p][4 * g + e] * a.inscale) * (acc[i][2 * p + 1][4 * g + e] * a.inscale) *
                            a.oscale;
            hi[p][g][e] = (f16)h;
            lo[p][g][e] = h - (float)hi[p][g][e];  // exact in f32
            mx[p] = fmaxf(mx[p], fabsf(lo[p][g][e]));
          }
      int ex[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[p]), __float_as_uint(mx[p]), false, false);
        ex[p] = lo4_exp(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
      }
      // Lane l (hsel 0) holds columns 8g .. 8g + 3 of each 32-column block and
      // lane l + 32 columns 8g + 4 .. 8g + 7.  One lane-half swap per register
      // makes the runs contiguous: the lower lane then stores columns 16k ..
      // 16k + 7 and the upper 16k + 8 .. 16k + 15 of the f16 part (k = 0, 1;
      // 16 bytes each), and the lower lane the codes of columns 0 .. 15, the
      // upper those of 16 .. 31 (8 bytes each).  The permlane runs in every
      // lane; rows past M only skip the stores.
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float inv = __builtin_ldexpf(1.0f, -ex[p]);
        unsigned q[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const floatx4 v = lo[p][g] * inv;
          q[g] = pack_e2m1(v[0], v[1], v[2], v[3]) & 0xffffu;
        }
        const auto cs = __builtin_amdgcn_permlane32_swap(q[0] | (q[1] << 16), q[2] | (q[3] << 16), false, false);
        const u32x2 codes = {(cs[0] & 0xffffu) | (cs[1] << 16), (cs[0] >> 16) | (cs[1] & 0xffff0000u)};
        u32x4 hv[2];
        pair_halves(hi[p], hv);
        if (row < a.M) {
          f16* orow = reinterpret_cast<f16*>(a.out) + (size_t)row * a.ldo;
          uint8_t* brow = reinterpret_cast<uint8_t*>(orow);
#pragma unroll
          for (int k = 0; k < 2; ++k)
            *reinterpret_cast<u32x4*>(orow + lo4_hi_at(hc + p * 32 + 16 * k + 8 * hsel)) = hv[k];
          *reinterpret_cast<u32x2*>(brow + lo4_lo_at(hc + p * 32) + 8 * hsel) = codes;
          if (hsel == 0) a.osc[lo4_sc_at(row, hc + p * 32, a.N / 2)] = (uint8_t)(ex[p] + 127);
        }
      }
    }
  } else {  // EPI_SWIGLU, EPI_SWIGLU2: tiles (2p, 2p+1) hold matching gate / up columns
    static_assert(EPI == EPI_SWIGLU || EPI == EPI_SWIGLU2, "row-layout epilogue");
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = r0 + i * 32 + l32;
#pragma unroll
      for (int p = 0; p < TN / 2; ++p) {
        half4 hi[4], lo[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float h = silu_f(acc[i][2 * p][4 * g + e] * a.inscale) * (acc[i][2 * p + 1][4 * g + e] * a.inscale) *
                            a.oscale;
            hi[g][e] = (f16)h;
            lo[g][e] = (f16)(h - (float)hi[g][e]);  // exact in f32
          }
        // contiguous runs through the lane-half swap (every lane takes part)
        u32x4 hv[2], lv[2];
        pair_halves(hi, hv);
        if constexpr (EPI == EPI_SWIGLU2) pair_halves(lo, lv);
        if (row < a.M) {
          f16* op = reinterpret_cast<f16*>(a.out) + (size_t)row * a.ldo + c0 / 2 + p * 32 + 8 * hsel;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            *reinterpret_cast<u32x4*>(op + 16 * k) = hv[k];
            if constexpr (EPI == EPI_SWIGLU2) *reinterpret_cast<u32x4*>(op + a.N / 2 + 16 * k) = lv[k];
          }
        }
      }
    }
  }
}

// Epilogue of one wave's TM x TN grid of 32 x 32 accumulator tiles whose
// top-left output element is (r0, c0).  MFMA 32x32 accumulator layout: lane
// l holds column l % 32 and rows 8g + 4(l / 32) + e (g, e = 0..3) in
// register 4g + e.
template <int EPI, int TM, int TN>
__device__ __forceinline__ void epilogue(const GemmArgs& a, floatx16 (&acc)[TM][TN], int r0, int c0, int lane) {
  const int hsel = lane >> 5, l32 = lane & 31;
  const int rbase = r0 + 4 * hsel;
  const int cbase = c0 + l32;
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float gt = a.gate[cbase + j * 32];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
          if (row < a.M) {
            float* xp = reinterpret_cast<float*>(a.out) + (size_t)row * a.ldo + cbase + j * 32;
            *xp = __builtin_fmaf(gt, acc[i][j][e] * a.oscale, *xp);
          }
        }
    }
  } else if constexpr (EPI == EPI_F32 || EPI == EPI_F16 || EPI == EPI_GELU) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
          const int col = cbase + j * 32;
          if (row < a.M) {
            const float v = (EPI == EPI_GELU ? gelu_f(acc[i][j][e] * a.inscale) : acc[i][j][e]) * a.oscale;
            if constexpr (EPI == EPI_F32)
              reinterpret_cast<float*>(a.out)[(size_t)row * a.ldo + col] = v;
            else
              reinterpret_cast<f16*>(a.out)[(size_t)row * a.ldo + col] = (f16)v;
          }
        }
  } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU2) {
    // tiles (2p, 2p+1) of a wave hold matching gate / up columns
    const int hc0 = c0 / 2 + l32;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int p = 0; p < TN / 2; ++p)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
          if (row < a.M) {
            const float g = acc[i][2 * p][e] * a.inscale;
            const float u = acc[i][2 * p + 1][e] * a.inscale;
            const float h = silu_f(g) * u * a.oscale;
            f16* o = reinterpret_cast<f16*>(a.out) + (size_t)row * a.ldo + hc0 + p * 32;
            const f16 hi = (f16)h;
            o[0] = hi;
            // the rounding error of hi is exact in f32 (h has 24 significant bits)
            if constexpr (EPI == EPI_SWIGLU2) o[a.N / 2] = (f16)(h - (float)hi);
          }
        }
  } else {  // EPI_QKV: q | k to the panel, v transposed to out2
    const int two_h = (a.N / 3) * 2;
    if (c0 < two_h) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
            if (row < a.M)
              reinterpret_cast<f16*>(a.out)[(size_t)row * a.ldo + cbase + j * 32] = (f16)(acc[i][j][e] * a.oscale);
          }
    } else {
      // keys from M up to the leading dimension (whole groups of 16) get
      // zeros, as in the V^T epilogue above
      const int rz = a.ld2 & ~15;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          f16* dst = a.out2 + (size_t)(cbase + j * 32 - two_h) * a.ld2;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int row = rbase + i * 32 + 8 * g;  // a multiple of 4
            const int pos = vt_pos(row);
            half4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (f16)(acc[i][j][4 * g + e] * a.oscale);
            if (row + 3 < a.M) {
              *reinterpret_cast<half4*>(dst + pos) = v;
            } else if (row < rz) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (row + e >= a.M) v[e] = (f16)0.0f;
              *reinterpret_cast<half4*>(dst + pos) = v;
            }
          }
        }
    }
  }
}

// ───────────────────── large-M kernel: 256 x 256 x 64, LDS-direct loads ─────────────────────
constexpr int DBM = 256, DBN = 256, DBK = 64, DNS = 2;
constexpr int DSTAGE = (DBM + DBN) * DBK;  // halves per stage
// LDS rows of DBK = 64 halves: 8 chunks of 16 bytes; chunk c of row r sits
// at slot c ^ ((r >> 1) & 7), so the 16 rows a fragment read serves at once
// cover all 64 banks.
__device__ __forceinline__ int dswz(int r) { return (r >> 1) & 7; }

}  // namespace

// Persistent over work units (a tile, or with ksplit > 1 a tile's share of
// the k-tiles; units of one share come first): block b runs on XCD b % 8
// and walks that XCD's contiguous run of the grouped unit sequence, 32
// blocks abreast.  The next unit's first k-tiles are fetched while the
// current unit's epilogue stores drain.  NW = 4 waves of 128 x 128 (one per SIMD) or 8
// waves of 128 x 64 (two per SIMD, so one wave's issue stalls, barrier
// waits and epilogue are covered by the other's MFMAs).
//
// LO8 (the lo8 row form of GemmArgs): every third k-tile holds the fp8
// residuals of the 128 columns the two before it hold as halves.  The
// loads do not change (a k-tile is 128 bytes of each row either way); an
// fp8 k-tile is two k-steps of 64 columns, each a 32-byte fragment per
// lane and one scaled 32x32x64 MFMA per 32 x 32 tile, which takes as long
// as two f16 k-steps.  A unit runs whole groups of three k-tiles in one
// branch-free loop, so the accumulators stay in AGPRs.  Scales: the W
// rows' are fixed over a unit; the A rows' two bytes of a group are read
// at its first k-tile.
template <int EPI, int NW, int LO = 0>
__global__ __launch_bounds__(NW * 64, 1) void gemm_dma_kernel(GemmArgs a) {
  constexpr bool LO8 = LO == 8, LO4 = LO == 4;
  // 32 x 32 tiles per wave: 4 x 4 with 4 waves; 4 x 2 with 8, except the
  // q/k-norm epilogue, whose waves span whole 128-column heads (2 x 4)
  constexpr int TM = (NW == 8 && EPI == EPI_QKROPE) ? 2 : 4;
  constexpr int TN = (NW == 4 || EPI == EPI_QKROPE) ? 4 : 2;
  constexpr int WTM = TM * 32, WTN = TN * 32;  // wave tile
  constexpr int NCOL = DBN / WTN;              // waves across the block's columns
  constexpr int NL = 32 / NW;                  // 16-byte loads per lane per operand per k-tile
  static_assert(LO == 0 || (NW == 4 && EPI != EPI_QKV), "residual k-tiles: 4-wave row-layout kernels");
  extern __shared__ __attribute__((aligned(16))) f16 smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NCOL, wn = wave % NCOL;
  const int hsel = lane >> 5, l32 = lane & 31;
  const int K = a.K;
  const int KT = K / DBK / a.ksplit;  // k-tiles per work unit (LO8: a multiple of 3)
  const int ldw = a.ldw ? a.ldw : a.kw;
  const int tiles_n = a.N / DBN, tiles_m = (a.M + DBM - 1) / DBM;
  const int ntiles = tiles_n * tiles_m, nunits = ntiles * a.ksplit;
  // this block's run of the tile sequence
  int seq0, seq_end, seq_step;
  {
    const int nblk = gridDim.x, b = blockIdx.x;
    if (nblk < nunits && (nblk & 7) == 0) {
      const int per_xcd = nblk >> 3, x = b & 7, li = b >> 3;
      const int chunk = (nunits + 7) >> 3;
      seq0 = x * chunk + li;
      seq_end = min(nunits, (x + 1) * chunk);
      seq_step = per_xcd;
    } else {
      seq0 = b;
      seq_end = b + 1;
      seq_step = 1;
    }
  }
  // work unit sq -> tile (tm, tn) and its first k-tile kt0
  auto tile_rc = [&](int sq, int& tm, int& tn, int& kt0) {
    kt0 = (sq / ntiles) * KT;
    sq %= ntiles;
    constexpr int G = 4;
    if (tiles_m % G == 0) {
      const int per = G * tiles_n;
      const int g = sq / per, w = sq - g * per;
      tm = g * G + w % G;
      tn = w / G;
    } else {
      tm = sq / tiles_n;
      tn = sq - tm * tiles_n;
    }
  };
  // Load i (0..NL-1) of wave w fills LDS chunk positions p = (NL w + i) * 64
  // + lane of the A region and of the W region: row p / 8, slot p % 8, so
  // one load reads 8 whole 128-byte rows.
  // (fixed size: an array sized by a template-dependent constant and
  // captured by the lambdas below makes the host pass drop the kernel)
  int voa[8], vob[8];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int p = (wave * NL + i) * 64 + lane;
    const int r = p >> 3, c = (p & 7) ^ dswz(r);
    // the instruction offset (i % 4) KiB moves the LDS and the global
    // address alike; the global part is taken back here
    voa[i] = (r * a.lda + 8 * c) * 2 - (i & 3) * 1024;
    vob[i] = (r * ldw + 8 * c) * 2 - (i & 3) * 1024;
  }
  // Buffer resources over a tile's A rows and W rows; A rows at or past M
  // fall outside the resource's range and return zeros.
  auto rsrc_a = [&](int m0) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a.A + (size_t)m0 * a.lda), 0,
                                             (min(a.M - m0, DBM) - 1) * a.lda * 2 + K * 2, 0x00020000);
  };
  auto rsrc_b = [&](int n0) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a.W + (size_t)n0 * ldw), 0, DBN * ldw * 2, 0x00020000);
  };
  // W columns wrap every kw (K is kw or 2 kw)
  const int KTW = a.kw / DBK;
  int kt0 = 0;  // the current work unit's first k-tile
  // Load q (0 .. 2 NL - 1) of k-tile t into stage st: A-operand load q for
  // q < NL, W-operand load q - NL above.  Loads 4j .. 4j+3 of an operand
  // share one LDS base (M0) and differ in the instruction offset.
  auto load1 = [&](__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int st, int t, int q) {
    // (t is the global k-tile)
    const bool w = q >= NL;
    const int i = w ? q - NL : q;
    f16* base = smem + st * DSTAGE + (w ? DBM * DBK : 0) + (wave * NL + (i & ~3)) * 64 * 8;
    const __amdgpu_buffer_rsrc_t r = w ? rb : ra;
    const int vo = w ? vob[i] : voa[i];
    const int so = (w && t >= KTW ? t - KTW : t) * DBK * 2;
    switch (i & 3) {  // (the offset must be an immediate)
      case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, vo, so, 0, 0); break;
      case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, vo, so, 1024, 0); break;
      case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, vo, so, 2048, 0); break;
      default: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, vo, so, 3072, 0); break;
    }
  };
  floatx16 acc[TM][TN];
  half8 af[2][TM], bf[2][TN];
  // Fragment read r of k-step kk of k-tile t into buffer b, in the order the
  // MFMAs below consume them: A 0, W 0 .. TN-1, A 1 .. TM-1.
  auto read1 = [&](int t, int kk, int b, int r) {
    const f16* sa = smem + (t % DNS) * DSTAGE;
    const int c = kk * 2 + hsel;
    if (r == 0 || r > TN) {
      const int i = r == 0 ? 0 : r - TN;
      const int row = wm * WTM + i * 32 + l32;
      af[b][i] = *reinterpret_cast<const half8*>(sa + (row * 8 + (c ^ dswz(row))) * 8);
    } else {
      const int j = r - 1;
      const int row = wn * WTN + j * 32 + l32;
      bf[b][j] = *reinterpret_cast<const half8*>(sa + DBM * DBK + (row * 8 + (c ^ dswz(row))) * 8);
    }
  };
  // fp8 fragments: 32 bytes per lane (chunks 4 kk + 2 hsel and the next),
  // read in the same order, one fragment (two 16-byte reads) per call
  i32x8 af8[2][TM], bf8[2][TN];
  auto read8 = [&](int t, int kk, int b, int r) {
    const f16* sa = smem + (t % DNS) * DSTAGE;
    const int c = kk * 4 + 2 * hsel;
    const bool isa = r == 0 || r > TN;
    const int row = isa ? wm * WTM + (r == 0 ? 0 : r - TN) * 32 + l32 : wn * WTN + (r - 1) * 32 + l32;
    const f16* base = sa + (isa ? 0 : DBM * DBK) + row * 64;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + (c ^ dswz(row)) * 8);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + ((c + 1) ^ dswz(row)) * 8);
    const i32x8 v = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    if (isa)
      af8[b][r == 0 ? 0 : r - TN] = v;
    else
      bf8[b][r - 1] = v;
  };
  // every epilogue but the V^T one stores along output rows: C^T = W A^T
  constexpr bool ROWS = EPI != EPI_QKV;
  auto mfma1 = [&](int b, int k) {
    const int i = k / TN, j = k % TN;
    if constexpr (ROWS)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[b][j], af[b][i], acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[b][i], bf[b][j], acc[i][j], 0, 0, 0);
  };
  // scales of the residual k-tiles: lo8, the W rows' (per unit) and, per A
  // row, the two bytes of the current group's k-steps; lo4, per W row and
  // per A row the dword of the current group's four k-steps (lane half h)
  int wsc[TN], asc[TM];
  // an fp4 MFMA of k-step kk (the scale byte kk of each dword)
  auto mfma4 = [&](int b, int k, int kk) {
    const int i = k / TN, j = k % TN;
    const i32x8 wv = __builtin_bit_cast(i32x8, __builtin_shufflevector(__builtin_bit_cast(u32x4, bf[b][j]),
                                                                       u32x4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7));
    const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(__builtin_bit_cast(u32x4, af[b][i]),
                                                                       u32x4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7));
    switch (kk) {  // (the byte selects must be immediates)
      case 0: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc[i][j], 4, 4, 0, wsc[j], 0, asc[i]); break;
      case 1: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc[i][j], 4, 4, 1, wsc[j], 1, asc[i]); break;
      case 2: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc[i][j], 4, 4, 2, wsc[j], 2, asc[i]); break;
      default: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc[i][j], 4, 4, 3, wsc[j], 3, asc[i]); break;
    }
  };
  auto mfma8 = [&](int b, int k, int kk) {
    const int i = k / TN, j = k % TN;
    if (kk == 0)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf8[b][j], af8[b][i], acc[i][j], 0, 0, 0, wsc[j], 0,
                                                                  asc[i]);
    else
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf8[b][j], af8[b][i], acc[i][j], 0, 0, 0, wsc[j], 1,
                                                                  asc[i]);
  };
  constexpr int MM = TM * TN, NDS = TM + TN, NQ = 2 * NL;
  // A k-tile's NQ loads go out over three k-steps: [0, Q1) in the last
  // k-step of the k-tile two before, [Q1, Q2) and [Q2, NQ) in the first two
  // of the k-tile before.  (Before an fp8 k-tile's barrier there is one
  // k-step: [Q1, NQ) go out in it.)
  constexpr int Q1 = (NQ + 2) / 3, Q2 = Q1 + (NQ - Q1 + 1) / 2;
  // One k-step in a fixed order: MFMA k on fragment buffer b, then load
  // q0 + k of k-tile tl while below q1, then fragment read k of k-step kk
  // of k-tile t into buffer b ^ 1 when rd (with rd8: an fp8 fragment of
  // k-step kk of k-tile t into fp8 buffer 0 instead).
  auto step = [&](int b, bool rd, int t, int kk, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int tl,
                  int q0, int q1, bool rd8 = false) {
#pragma unroll
    for (int k = 0; k < MM; ++k) {
      mfma1(b, k);
      if (q0 + k < q1) load1(ra, rb, tl & 1, kt0 + tl, q0 + k);
      if (rd && !rd8 && k < NDS) read1(t, kk, b ^ 1, k);
      if constexpr (LO8)
        if (rd8 && k < NDS) read8(t, kk, 0, k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // lo4: a k-step of either kind (fp4 = the group's residual k-tile, whose
  // MFMAs take k-step mk's scale bytes), otherwise as step
  auto step4 = [&](bool fp4, int mk, int b, bool rd, int t, int kk, __amdgpu_buffer_rsrc_t ra,
                   __amdgpu_buffer_rsrc_t rb, int tl, int q0, int q1) {
#pragma unroll
    for (int k = 0; k < MM; ++k) {
      if (fp4)
        mfma4(b, k, mk);
      else
        mfma1(b, k);
      if (q0 + k < q1) load1(ra, rb, tl & 1, kt0 + tl, q0 + k);
      if (rd && k < NDS) read1(t, kk, b ^ 1, k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // An fp8 k-step: MFMA k (k-step kk8 of its k-tile) on fp8 buffer b8,
  // loads as above, then fragment read k of k-step kk of k-tile t: into
  // fp8 buffer 1 (rd8) or f16 buffer 0 (rd16).
  auto step8 = [&](int b8, int kk8, bool rd8, bool rd16, int t, int kk, __amdgpu_buffer_rsrc_t ra,
                   __amdgpu_buffer_rsrc_t rb, int tl, int q0, int q1) {
#pragma unroll
    for (int k = 0; k < MM; ++k) {
      mfma8(b8, k, kk8);
      if (q0 + k < q1) load1(ra, rb, tl & 1, kt0 + tl, q0 + k);
      if (rd8 && k < NDS) read8(t, kk, 1, k);
      if (rd16 && k < NDS) read1(t, kk, 0, k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // k-tile 0 and the first part of k-tile 1 of the unit at (tm, tn, kt0)
  auto prologue = [&](int tm, int tn, int kt0) {
    const __amdgpu_buffer_rsrc_t ra = rsrc_a(tm * DBM), rb = rsrc_b(tn * DBN);
#pragma unroll
    for (int q = 0; q < NQ; ++q) load1(ra, rb, 0, kt0, q);
#pragma unroll
    for (int q = 0; q < Q1; ++q) load1(ra, rb, 1, kt0 + min(1, KT - 1), q);
  };
  // the wait for, and the barrier after, a k-tile's reads and the next
  // k-tile's loads
  auto sync_tile = [&]() {
    __builtin_amdgcn_s_waitcnt(wait_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  int tm, tn;
  tile_rc(seq0, tm, tn, kt0);
  prologue(tm, tn, kt0);
  for (int sq = seq0; sq < seq_end; sq += seq_step) {
    const int m0 = tm * DBM, n0 = tn * DBN;
    const size_t obase = (size_t)(kt0 / KT) * a.pstride;  // partial plane of a split unit
    const __amdgpu_buffer_rsrc_t ra = rsrc_a(m0), rb = rsrc_b(n0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if constexpr (LO8) {
      // A scales: the tile's 256-row block of the blocked array (lds
      // bytes per row; rows past M read whatever the block holds there,
      // which only their unstored outputs see)
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.asc + (size_t)m0 * a.lds), 0, DBM * a.lds, 0x00020000);
      // the A scale bytes of the group at unit-local k-tile t (its k-steps
      // 2 g and 2 g + 1, g the global group): 32 rows' in 64 bytes
      auto load_asc = [&](int t) {
        const int g = (kt0 + t) / 3;
#pragma unroll
        for (int i = 0; i < TM; ++i)
          asc[i] = (int)__builtin_amdgcn_raw_buffer_load_b16(rs, g * 512 + (wm * WTM + i * 32 + l32) * 2, 0, 0);
      };
#pragma unroll
      for (int j = 0; j < TN; ++j) wsc[j] = a.wsc[n0 + wn * WTN + j * 32 + l32];
      load_asc(0);
      if (sq == seq0)
        __builtin_amdgcn_s_waitcnt(wait_imm(Q1, 15));
      else
        __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int r = 0; r < NDS; ++r) read1(0, 0, 0, r);
      __builtin_amdgcn_sched_barrier(0);
      // groups (f16, f16, fp8) of k-tiles t, t + 1, t + 2; the next group's
      // A scales are fetched after this group's fp8 MFMAs are issued
      for (int t = 0; t < KT - 3; t += 3) {
        step(0, true, t, 1, ra, rb, t + 1, Q1, Q2);
        step(1, true, t, 2, ra, rb, t + 1, Q2, NQ);
        step(0, true, t, 3, ra, rb, 0, 0, 0);
        sync_tile();
        step(1, true, t + 1, 0, ra, rb, t + 2, 0, Q1);
        step(0, true, t + 1, 1, ra, rb, t + 2, Q1, Q2);
        step(1, true, t + 1, 2, ra, rb, t + 2, Q2, NQ);
        step(0, true, t + 1, 3, ra, rb, 0, 0, 0);
        sync_tile();
        step(1, false, t + 2, 0, ra, rb, t + 3, 0, Q1, true);
        step8(0, 0, true, false, t + 2, 1, ra, rb, t + 3, Q1, NQ);
        sync_tile();
        step8(1, 1, false, true, t + 3, 0, ra, rb, t + 4, 0, Q1);
        load_asc(t + 3);
      }
      // the last group
      {
        const int t = KT - 3;
        step(0, true, t, 1, ra, rb, t + 1, Q1, Q2);
        step(1, true, t, 2, ra, rb, t + 1, Q2, NQ);
        step(0, true, t, 3, ra, rb, 0, 0, 0);
        sync_tile();
        step(1, true, t + 1, 0, ra, rb, t + 2, 0, Q1);
        step(0, true, t + 1, 1, ra, rb, t + 2, Q1, Q2);
        step(1, true, t + 1, 2, ra, rb, t + 2, Q2, NQ);
        step(0, true, t + 1, 3, ra, rb, 0, 0, 0);
        sync_tile();
        step(1, false, t + 2, 0, ra, rb, 0, 0, 0, true);
        step8(0, 0, true, false, t + 2, 1, ra, rb, 0, 0, 0);
        sync_tile();
        const int nsq = sq + seq_step;
        if (nsq < seq_end) {
          tile_rc(nsq, tm, tn, kt0);
          prologue(tm, tn, kt0);
        }
        step8(1, 1, false, false, 0, 0, ra, rb, 0, 0, 0);
      }
    } else if constexpr (LO4) {
      // the tile's 256-row blocks of the blocked scale arrays (lds / ldws
      // bytes per row)
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.asc + (size_t)m0 * a.lds), 0, DBM * a.lds, 0x00020000);
      const __amdgpu_buffer_rsrc_t rw =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.wsc + (size_t)n0 * a.ldws), 0, DBN * a.ldws, 0x00020000);
      // the scale dwords of the group at unit-local k-tile t: its fp4
      // k-tile's four k-steps for this lane half, per A row and per W row
      // (32 rows' dwords of one lane half in 256 bytes)
      auto load_sc = [&](int t) {
        const int o = ((kt0 + t) / 5) * 2048 + 4 * hsel;
#pragma unroll
        for (int i = 0; i < TM; ++i)
          asc[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, o + (wm * WTM + i * 32 + l32) * 8, 0, 0);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          wsc[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(rw, o + (wn * WTN + j * 32 + l32) * 8, 0, 0);
      };
      load_sc(0);
      if (sq == seq0)
        __builtin_amdgcn_s_waitcnt(wait_imm(Q1, 15));
      else
        __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int r = 0; r < NDS; ++r) read1(0, 0, 0, r);
      __builtin_amdgcn_sched_barrier(0);
      // one k-tile of either kind whose last k-step reads the next k-tile's
      // first fragments (loads of k-tiles t + 1 and t + 2 as in the plain loop)
      auto tile4 = [&](bool fp4, int t) {
        step4(fp4, 0, 0, true, t, 1, ra, rb, t + 1, Q1, Q2);
        step4(fp4, 1, 1, true, t, 2, ra, rb, t + 1, Q2, NQ);
        step4(fp4, 2, 0, true, t, 3, ra, rb, 0, 0, 0);
        sync_tile();
        step4(fp4, 3, 1, true, t + 1, 0, ra, rb, t + 2, 0, Q1);
      };
      // groups (f16 x 4, fp4) of k-tiles t .. t + 4; the next group's scales
      // are fetched once its fp4 MFMAs are issued
      for (int t = 0; t < KT - 5; t += 5) {
        tile4(false, t);
        tile4(false, t + 1);
        tile4(false, t + 2);
        tile4(false, t + 3);
        tile4(true, t + 4);
        load_sc(t + 5);
      }
      // the last group
      {
        const int t = KT - 5;
        tile4(false, t);
        tile4(false, t + 1);
        tile4(false, t + 2);
        step4(false, 0, 0, true, t + 3, 1, ra, rb, t + 4, Q1, Q2);
        step4(false, 1, 1, true, t + 3, 2, ra, rb, t + 4, Q2, NQ);
        step4(false, 2, 0, true, t + 3, 3, ra, rb, 0, 0, 0);
        sync_tile();
        step4(false, 3, 1, true, t + 4, 0, ra, rb, 0, 0, 0);
        step4(true, 0, 0, true, t + 4, 1, ra, rb, 0, 0, 0);
        step4(true, 1, 1, true, t + 4, 2, ra, rb, 0, 0, 0);
        step4(true, 2, 0, true, t + 4, 3, ra, rb, 0, 0, 0);
        sync_tile();
        const int nsq = sq + seq_step;
        if (nsq < seq_end) {
          tile_rc(nsq, tm, tn, kt0);
          prologue(tm, tn, kt0);
        }
        step4(true, 3, 1, false, 0, 0, ra, rb, 0, 0, 0);
      }
    } else {
      // k-tile 0 landed.  After an epilogue its stores share the vector
      // memory counter with these loads, so wait for all of them.
      if (sq == seq0)
        __builtin_amdgcn_s_waitcnt(wait_imm(Q1, 15));
      else
        __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int r = 0; r < NDS; ++r) read1(0, 0, 0, r);
      __builtin_amdgcn_sched_barrier(0);
      // (with KT = 1 the prologue's k-tile 1 is k-tile 0 again, in the stage
      // no one reads, and the loop below does not run)
      for (int t = 0; t < KT - 1; ++t) {
        step(0, true, t, 1, ra, rb, t + 1, Q1, Q2);
        step(1, true, t, 2, ra, rb, t + 1, Q2, NQ);
        step(0, true, t, 3, ra, rb, 0, 0, 0);
        // this wave's reads of stage t % 2 are done and k-tile t + 1 has
        // landed; after the barrier every wave is past both, so the stage
        // can take the first part of k-tile t + 2 (past the last k-tile:
        // k-tile 0 again, into a stage no one reads any more)
        sync_tile();
        step(1, true, t + 1, 0, ra, rb, t + 2 < KT ? t + 2 : t, 0, Q1);
      }
      // the last k-tile
      step(0, true, KT - 1, 1, ra, rb, 0, 0, 0);
      step(1, true, KT - 1, 2, ra, rb, 0, 0, 0);
      step(0, true, KT - 1, 3, ra, rb, 0, 0, 0);
      // every wave's reads of every stage are done and no load is in flight:
      // the next tile's first k-tiles can be fetched under the epilogue
      sync_tile();
      const int nsq = sq + seq_step;
      if (nsq < seq_end) {
        tile_rc(nsq, tm, tn, kt0);
        prologue(tm, tn, kt0);
      }
      step(1, false, 0, 0, ra, rb, 0, 0, 0);
    }
    if constexpr (ROWS)
      epilogue_rows<EPI, TM, TN>(a, acc, m0 + wm * WTM, n0 + wn * WTN, lane, obase);
    else
      epilogue<EPI, TM, TN>(a, acc, m0 + wm * WTM, n0 + wn * WTN, lane);
  }
  __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));  // no LDS-bound load outlives the block
}

// ───────────────────── large-M kernel, 16 x 16 x 32 MFMAs ─────────────────────
namespace {

// Row layout of a 16 x 16 accumulator tile of C^T = W A^T (the W fragment
// as the MFMA's A operand): lane l holds output row l % 16 of the tile and
// its 4 consecutive output columns 4 (l / 16) .. + 3 in registers 0..3.
// Two tiles j0 (even) and j0 + 1 merge through one v_permlane16_swap per
// register into runs of 8 columns: lane group g = l / 16 then holds
// columns m16_col(g) .. + 7 of the 32 the pair covers.  Every lane must
// take part.
__device__ __forceinline__ int m16_col(int g) { return 16 * (g & 1) + 8 * (g >> 1); }
__device__ __forceinline__ u32x4 merge16(const half4& x, const half4& y) {
  const u32x2 xv = __builtin_bit_cast(u32x2, x), yv = __builtin_bit_cast(u32x2, y);
  const auto s0 = __builtin_amdgcn_permlane16_swap(xv[0], yv[0], false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(xv[1], yv[1], false, false);
  return u32x4{s0[0], s1[0], s0[1], s1[1]};
}
__device__ __forceinline__ half4 to_half4(const floatx4& v) { return half4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]}; }
// sum / max of a value over the four lane groups that share an output row
__device__ __forceinline__ float row_sum16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float row_max16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 4 x 4 transpose of f16 values inside each quad of lanes: lane r (= lane
// % 4) of a quad holds x[r][0..3] packed two to a dword (the first in the
// low half) and gets x[0..3][r] back in the same packing.  Two exchanges:
// lanes r and r ^ 2 swap the column pair the other keeps, then lanes r and
// r ^ 1 the column the other keeps.  Every lane must take part.
__device__ __forceinline__ u32x2 quad_t16(u32x2 v, int r) {
  constexpr unsigned LO = 0x05040100u, HI = 0x07060302u;  // perm selectors: low / high halves of (src1, src0)
  const bool low2 = r < 2, odd = r & 1;
  // lanes 0, 1 keep columns 0, 1 and lanes 2, 3 columns 2, 3
  const unsigned got1 = (unsigned)__builtin_amdgcn_mov_dpp((int)(low2 ? v[1] : v[0]), 0x4e, 0xf, 0xf, false);
  const unsigned ra = low2 ? v[0] : got1;  // row r % 2 of the kept columns
  const unsigned rb = low2 ? got1 : v[1];  // row r % 2 + 2
  // even lanes keep the first of their two columns, odd lanes the second
  const unsigned keep = __builtin_amdgcn_perm(rb, ra, odd ? HI : LO);
  const unsigned got2 = (unsigned)__builtin_amdgcn_mov_dpp((int)__builtin_amdgcn_perm(rb, ra, odd ? LO : HI), 0xb1, 0xf,
                                                           0xf, false);
  const unsigned r02 = odd ? got2 : keep, r13 = odd ? keep : got2;  // rows 0, 2 and rows 1, 3 of column r
  return u32x2{__builtin_amdgcn_perm(r13, r02, LO), __builtin_amdgcn_perm(r13, r02, HI)};
}

// Epilogue of a wave whose output rows [r0, r0 + 128) and columns [c0, c0 +
// 128) sit in 8 x 8 tiles of 16 x 16 (tile (i, j): rows r0 + 16 i .., columns
// c0 + 16 j ..): lane l holds row r0 + 16 i + l % 16 and columns c0 + 16 j +
// 4 g .. + 3, g = l / 16.
template <int EPI>
__device__ __forceinline__ void epilogue16(const GemmArgs& a, floatx4 (&acc)[8][8], int r0, int c0, int lane,
                                           size_t obase) {
  // lane indices opaque here: address arithmetic derived from them stays in
  // the epilogue instead of being hoisted out of the tile loop, where its
  // registers would compete with the main loop's
  int l16 = lane & 15, g = lane >> 4;
  if constexpr (EPI == EPI_QKV) {
    // and taken afresh (the count of the lanes below this one, in an asm
    // statement that cannot move out of the tile loop), so that no lane
    // index computed before the loop has to live through it
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    l16 = ln & 15;
    g = ln >> 4;
  }
  asm volatile("" : "+v"(l16), "+v"(g));
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i + l16;
      if (row < a.M) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = c0 + 16 * j + 4 * g;
          floatx4* xp = reinterpret_cast<floatx4*>(reinterpret_cast<float*>(a.out) + (size_t)row * a.ldo + c);
          const floatx4 gt = *reinterpret_cast<const floatx4*>(a.gate + c);
          floatx4 x = *xp;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(gt[e], acc[i][j][e] * a.oscale, x[e]);
          *xp = x;
        }
      }
    }
  } else if constexpr (EPI == EPI_F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i + l16;
      if (row < a.M) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(a.out) + obase + (size_t)row * a.ldo + c0 + 16 * j +
                                      4 * g) = acc[i][j] * a.oscale;
      }
    }
  } else if constexpr (EPI == EPI_F16 || EPI == EPI_GELU) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i + l16;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        floatx4 v[2] = {acc[i][2 * p], acc[i][2 * p + 1]};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if constexpr (EPI == EPI_GELU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[u][e] = gelu_f(v[u][e] * a.inscale);
          }
          v[u] = v[u] * a.oscale;
        }
        const u32x4 o = merge16(to_half4(v[0]), to_half4(v[1]));
        if (row < a.M)
          *reinterpret_cast<u32x4*>(reinterpret_cast<f16*>(a.out) + obase + (size_t)row * a.ldo + c0 + 32 * p +
                                    m16_col(g)) = o;
      }
    }
  } else if constexpr (EPI == EPI_QKV) {
    // q | k columns (c0 < 2H) to out as f16; v columns transposed into out2
    // (V^T: one row per v column, key c at vt_pos(c)).  A lane holds one key
    // and 4 consecutive v columns of a tile; the 4 x 4 transpose inside each
    // quad (keys 4a .. 4a + 3 of the tile) gives lane 4a + r the 4 keys of
    // column 4g + r, which vt_pos keeps contiguous: one 8-byte store.  Keys
    // from M up to the leading dimension (whole groups of 16) get zeros.
    const int two_h = (a.N / 3) * 2;
    if (c0 < two_h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = r0 + 16 * i + l16;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const u32x4 o = merge16(to_half4(acc[i][2 * p] * a.oscale), to_half4(acc[i][2 * p + 1] * a.oscale));
          if (row < a.M)
            *reinterpret_cast<u32x4*>(reinterpret_cast<f16*>(a.out) + (size_t)row * a.ldo + c0 + 32 * p + m16_col(g)) = o;
        }
      }
    } else {
      const int r = l16 & 3, rz = a.ld2 & ~15;
      const bool tail = r0 + 128 > a.M;  // the wave holds rows past M
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = r0 + 16 * i + (l16 & ~3);  // the quad's first key
        const bool zero = tail && r0 + 16 * i + l16 >= a.M;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x2 v = __builtin_bit_cast(u32x2, to_half4(acc[i][j] * a.oscale));
          if (zero) v = u32x2{0u, 0u};
          v = quad_t16(v, r);
          if (key < rz)
            *reinterpret_cast<u32x2*>(a.out2 + (size_t)(c0 - two_h + 16 * j + 4 * g + r) * a.ld2 + vt_pos(key)) = v;
        }
        // one row slice at a time (as in the SwiGLU epilogue)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if constexpr (EPI == EPI_QKROPE) {
    // the wave's 128 columns are one head (c0 % 128 == 0); a row's 128
    // accumulators sit in its four lane groups
    const int H = a.N / 2;
    const bool isk = c0 >= H;
    const float* nw = isk ? a.nk : a.nq;
    f16* dst = isk ? a.kout + (c0 - H) : reinterpret_cast<f16*>(a.out) + c0;
    const int ld = isk ? a.ldk : a.ldo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i + l16;
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(acc[i][j][e], acc[i][j][e], ss);
      const float inv = rsqrtf(row_sum16(ss) * (1.0f / 128.0f) + a.eps);
      // the row's packed table: cos and sin of the lane's two pairs in one
      // 16-byte load (rows past M read the last row; their results are not
      // stored, but every lane takes part in the swaps)
      const float* tr = a.rope + (size_t)min(row, a.M - 1) * 128;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        half4 h[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = 2 * p + u;
          const int d = 16 * j + 4 * g;  // dims d .. d+3: pairs d/2, d/2 + 1
          const floatx4 w = *reinterpret_cast<const floatx4*>(nw + d);
          const floatx4 t = *reinterpret_cast<const floatx4*>(tr + d);  // cos d/2, d/2+1, sin d/2, d/2+1
          const float a0 = (acc[i][j][0] * inv) * w[0], b0 = (acc[i][j][1] * inv) * w[1];
          const float a1 = (acc[i][j][2] * inv) * w[2], b1 = (acc[i][j][3] * inv) * w[3];
          h[u] = half4{(f16)(a0 * t[0] - b0 * t[2]), (f16)(a0 * t[2] + b0 * t[0]), (f16)(a1 * t[1] - b1 * t[3]),
                       (f16)(a1 * t[3] + b1 * t[1])};
        }
        const u32x4 o = merge16(h[0], h[1]);
        if (row < a.M) *reinterpret_cast<u32x4*>(dst + (size_t)row * ld + 32 * p + m16_col(g)) = o;
      }
    }
  } else if constexpr (EPI == EPI_VT) {
    // output rows are V dims, columns are keys: key c goes to vt_pos(c),
    // which swaps bits 2 and 3, so the lane groups g = 0, 2 of a 16-key tile
    // fill positions 0..7 and g = 1, 3 positions 8..15.  Tiles 2p and 2p + 1
    // merge through v_permlane32_swap: lane group g then holds positions
    // 16 (g >> 1) + 8 (g & 1) .. + 7 of the pair's 32.  Columns from nvalid
    // up to the leading dimension (whole groups of 16) get zeros: the
    // attention kernel reads whole 64-key tiles and multiplies the columns
    // past the keys by P = 0, which must not meet a stale non-finite value.
    const int cz = a.ldo & ~15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i + l16;
      f16* orow = reinterpret_cast<f16*>(a.out) + (size_t)min(row, a.M - 1) * a.ldo;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        u32x2 x[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = c0 + 32 * p + 16 * u + 4 * g;
          half4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = c + e < a.nvalid ? (f16)(acc[i][2 * p + u][e] * a.oscale) : (f16)0.0f;
          x[u] = __builtin_bit_cast(u32x2, h);
        }
        const auto s0 = __builtin_amdgcn_permlane32_swap(x[0][0], x[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x[0][1], x[1][1], false, false);
        const int base = c0 + 32 * p + 16 * (g >> 1);  // this lane's 16-key group
        // a group of 16 keys is below cz whole or not at all, and the host
        // guarantees nvalid <= cz
        if (row < a.M && base < cz)
          *reinterpret_cast<u32x4*>(orow + base + 8 * (g & 1)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU4) {
    // the wave's 128 W rows are two groups p of 32 gate rows (tiles 4p,
    // 4p + 1) and the matching 32 up rows (4p + 2, 4p + 3): 64 hidden
    // columns, one 32-column scale block per group and row
    const int hc = c0 / 2;  // first hidden column of the wave
    // silu(g s) (u s) o = (g u) (s^2 o) / (1 + 2^(g (-s log2 e))): s and o
    // are powers of two, so both factors are exact scalings of the
    // constants and the exponent argument is that of exp(-g s)
    const float ke = a.inscale * -1.44269504088896341f, kp = a.inscale * a.inscale * a.oscale;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i + l16;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        half4 hi[2];
        floatx4 lo[2];
        float mx = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = acc[i][4 * p + u][e], uv = acc[i][4 * p + 2 + u][e];
            const float h = (gv * uv) * kp * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gv * ke));
            hi[u][e] = (f16)h;
            lo[u][e] = h - (float)hi[u][e];  // exact in f32
            mx = fmaxf(mx, fabsf(lo[u][e]));
          }
        const int ex = lo4_exp(row_max16(mx));
        const float inv = __builtin_ldexpf(1.0f, -ex);
        unsigned q[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const floatx4 v = lo[u] * inv;
          q[u] = pack_e2m1(v[0], v[1], v[2], v[3]);
        }
        // the codes of the lane's 8 columns, like the halves: one swap
        const auto cs = __builtin_amdgcn_permlane16_swap(q[0], q[1], false, false);
        const unsigned codes = (cs[0] & 0xffffu) | (cs[1] << 16);
        const u32x4 hv = merge16(hi[0], hi[1]);
        if (row < a.M) {
          f16* orow = reinterpret_cast<f16*>(a.out) + (size_t)row * a.ldo;
          uint8_t* brow = reinterpret_cast<uint8_t*>(orow);
          const int c = hc + 32 * p + m16_col(g);
          *reinterpret_cast<u32x4*>(orow + lo4_hi_at(c)) = hv;
          *reinterpret_cast<unsigned*>(brow + lo4_lo_at(c)) = codes;
          if (g == 0) a.osc[lo4_sc_at(row, hc + 32 * p, a.N / 2)] = (uint8_t)(ex + 127);
        }
      }
      // one row slice at a time: hoisting every slice's accumulator reads
      // would crowd the registers the main loop needs
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {  // EPI_SWIGLU, EPI_SWIGLU2: gate / up groups as for EPI_SWIGLU4
    static_assert(EPI == EPI_SWIGLU || EPI == EPI_SWIGLU2, "row-layout epilogue");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i + l16;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        half4 hi[2], lo[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float h = silu_f(acc[i][4 * p + u][e] * a.inscale) * (acc[i][4 * p + 2 + u][e] * a.inscale) * a.oscale;
            hi[u][e] = (f16)h;
            lo[u][e] = (f16)(h - (float)hi[u][e]);  // exact in f32
          }
        const u32x4 hv = merge16(hi[0], hi[1]);
        u32x4 lv = u32x4{0, 0, 0, 0};
        if constexpr (EPI == EPI_SWIGLU2) lv = merge16(lo[0], lo[1]);
        if (row < a.M) {
          f16* op = reinterpret_cast<f16*>(a.out) + (size_t)row * a.ldo + c0 / 2 + 32 * p + m16_col(g);
          *reinterpret_cast<u32x4*>(op) = hv;
          if constexpr (EPI == EPI_SWIGLU2) *reinterpret_cast<u32x4*>(op + a.N / 2) = lv;
        }
      }
    }
  }
}

}  // namespace

// The 4-wave 256 x 256 x 64 kernel on v_mfma_f32_16x16x32_f16: each wave
// computes 128 x 128 as 8 x 8 tiles of 16 x 16 (256 accumulators).  Loads,
// LDS layout, tile order and the persistent walk are those of
// gemm_dma_kernel; what differs:
//
// * A k-tile is two k-steps of 32.  A lane's fragment of k-step s is the
//   16-byte chunk 4 s + l / 16 of its row, rows l % 16 of each 16-row
//   slice.  B (W) fragments are double-buffered; an A fragment is
//   refilled in place once its 8 MFMAs are issued (96 registers).
// * All 16 loads of k-tile t + 2 go out in the k-step right after the
//   barrier of k-tile t, so each has a whole k-tile to land.
// * Stage indices are compile-time constants: k-tiles run in pairs (lo4:
//   groups of five in pairs), so a unit needs an even number of k-tiles
//   (lo4: of groups), and no fragment address is computed in the loop.
// * LO4: a group of four f16 k-tiles and one e2m1 k-tile per 256 columns.
//   An e2m1 k-tile's k-step s is one v_mfma_scale_f32_16x16x128_f8f6f4 per
//   tile (fp4 operands, same chunks as f16); lane group g takes scale
//   block g of the k-step (block 4 s + g of the group), which sits at byte
//   (g >> 1) + 2 s of the scale dword at 4 (g & 1).
//
// LSP / LOFF: a load after every LSP-th MFMA from the LOFF-th; BPOS: the
// MFMA of a row of 8 after which the next B fragment is read.  These fix
// the instruction order; the register allocator keeps the accumulators in
// AGPRs only for some of them (checked on the built code).
template <int EPI, int LO, int LSP, int LOFF, int BPOS>
__global__ __launch_bounds__(256, 1) void gemm16_kernel(GemmArgs a) {
  constexpr bool LO4 = LO == 4;
  constexpr int NL = 8, NQ = 16, TM = 8, TN = 8, MM = 64;
  extern __shared__ __attribute__((aligned(16))) f16 smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int K = a.K;
  const int KT = K / DBK / a.ksplit;  // k-tiles per work unit (LO4: a multiple of 5)
  const int ldw = a.ldw ? a.ldw : a.kw;
  const int tiles_n = a.N / DBN, tiles_m = (a.M + DBM - 1) / DBM;
  const int ntiles = tiles_n * tiles_m, nunits = ntiles * a.ksplit;
  int seq0, seq_end, seq_step;
  {
    const int nblk = gridDim.x, b = blockIdx.x;
    if (nblk < nunits && (nblk & 7) == 0) {
      const int per_xcd = nblk >> 3, x = b & 7, li = b >> 3;
      const int chunk = (nunits + 7) >> 3;
      seq0 = x * chunk + li;
      seq_end = min(nunits, (x + 1) * chunk);
      seq_step = per_xcd;
    } else {
      seq0 = b;
      seq_end = b + 1;
      seq_step = 1;
    }
  }
  auto tile_rc = [&](int sq, int& tm, int& tn, int& kt0) __attribute__((always_inline)) {
    kt0 = (sq / ntiles) * KT;
    sq %= ntiles;
    constexpr int G = 4;
    if (tiles_m % G == 0) {
      const int per = G * tiles_n;
      const int gg = sq / per, w = sq - gg * per;
      tm = gg * G + w % G;
      tn = w / G;
    } else {
      tm = sq / tiles_n;
      tn = sq - tm * tiles_n;
    }
  };
  int voa[8], vob[8];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int p = (wave * NL + i) * 64 + lane;
    const int r = p >> 3, c = (p & 7) ^ dswz(r);
    voa[i] = (r * a.lda + 8 * c) * 2 - (i & 3) * 1024;
    vob[i] = (r * ldw + 8 * c) * 2 - (i & 3) * 1024;
  }
  auto rsrc_a = [&](int m0) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a.A + (size_t)m0 * a.lda), 0,
                                             (min(a.M - m0, DBM) - 1) * a.lda * 2 + K * 2, 0x00020000);
  };
  auto rsrc_b = [&](int n0) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a.W + (size_t)n0 * ldw), 0, DBN * ldw * 2, 0x00020000);
  };
  const int KTW = a.kw / DBK;
  int kt0 = 0;
  // load q of unit-local k-tile t into stage st (as in gemm_dma_kernel)
  auto load1 = [&](__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int st, int t, int q) __attribute__((always_inline)) {
    const bool w = q >= NL;
    const int i = w ? q - NL : q;
    f16* base = smem + st * DSTAGE + (w ? DBM * DBK : 0) + (wave * NL + (i & ~3)) * 64 * 8;
    const __amdgpu_buffer_rsrc_t r = w ? rb : ra;
    const int vo = w ? vob[i] : voa[i];
    const int tg = kt0 + t;
    const int so = (w && tg >= KTW ? tg - KTW : tg) * DBK * 2;
    switch (i & 3) {
      case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, vo, so, 0, 0); break;
      case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, vo, so, 1024, 0); break;
      case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, vo, so, 2048, 0); break;
      default: __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, vo, so, 3072, 0); break;
    }
  };
  floatx4 acc[TM][TN];
  half8 af[TM], bf[2][TN];
  // this lane's row offsets (halves) in a stage for k-steps 0 and 1: row
  // l16 of each 16-row slice (whose swizzle is that of l16), chunk 4 s + g4
  const int sw = dswz(l16);
  const int ro0 = l16 * DBK + ((g4 ^ sw) * 8);
  const int ro1 = l16 * DBK + (((4 + g4) ^ sw) * 8);
  auto readA = [&](int st, int kq, int i) __attribute__((always_inline)) {
    const f16* sa = smem + st * DSTAGE + (kq ? ro1 : ro0);
    af[i] = *reinterpret_cast<const half8*>(sa + (wm * 128 + i * 16) * DBK);
  };
  auto readB = [&](int st, int kq, int b, int j) __attribute__((always_inline)) {
    const f16* sa = smem + st * DSTAGE + (kq ? ro1 : ro0);
    bf[b][j] = *reinterpret_cast<const half8*>(sa + DBM * DBK + (wn * 128 + j * 16) * DBK);
  };
  // scale dwords of a group (LO4): per A row and per W row of the lane,
  // shifted so that bytes 0 and 2 are k-steps 0 and 1
  int asc[TM], wsc[TN];
  auto mfma1 = [&](bool fp4, int b, int k) __attribute__((always_inline)) {
    const int i = k / TN, j = k % TN;
    if (!fp4) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[b][j], af[i], acc[i][j], 0, 0, 0);
    } else {
      const i32x8 wv = __builtin_bit_cast(i32x8, __builtin_shufflevector(__builtin_bit_cast(u32x4, bf[b][j]),
                                                                         u32x4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7));
      const i32x8 av = __builtin_bit_cast(i32x8, __builtin_shufflevector(__builtin_bit_cast(u32x4, af[i]),
                                                                         u32x4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7));
      if (b == 0)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, av, acc[i][j], 4, 4, 0, wsc[j], 0, asc[i]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, av, acc[i][j], 4, 4, 2, wsc[j], 2, asc[i]);
    }
  };
  // One k-step: the MFMAs of k-step b (B buffer b); when rd, the fragments
  // of k-step rkq of stage rst (B into buffer b ^ 1 after MFMA 8 j + BPOS,
  // A i in place after MFMA 8 i + 7); when ld, the loads of k-tile tl into
  // stage lst.
  auto step = [&](bool fp4, int b, bool rd, int rst, int rkq, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                  bool ld, int lst, int tl) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < MM; ++k) {
      mfma1(fp4, b, k);
      if (ld && k % LSP == LOFF && k / LSP < NQ) load1(ra, rb, lst, tl, k / LSP);
      if (rd && k % 8 == BPOS) readB(rst, rkq, b ^ 1, k / 8);
      if (rd && k % 8 == 7) readA(rst, rkq, k / 8);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The accumulators held in AGPRs, at every k-tile and loop head: without
  // this the register allocator may give the loop-carried values VGPR
  // homes, or park some in VGPRs where registers run short, and copy them
  // back and forth (the MFMAs read and write AGPRs directly, so pinning
  // costs nothing).
  auto pin_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) asm volatile("" : "+a"(acc[i][j]));
  };
  auto sync_tile = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(wait_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // LO4 scales pass through LDS: two 4 KB buffers after the stages, each
  // one group's A-row scale bytes of the tile (2 KB) and W-row ones (2 KB).
  // Wave w moves 1 KB of a group (A scales for w < 2, W scales above, half
  // w & 1) with one LDS-direct load, right after a barrier like the
  // k-tile loads; a lane reads its 16 dwords at the group's fp4 k-tile.
  constexpr int SCH = DNS * DSTAGE;  // halves offset of the scale buffers
  auto load_sc = [&](int m0_, int n0_, int sb, int grp) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r =
        wave >= 2 ? __builtin_amdgcn_make_buffer_rsrc((void*)(a.wsc + (size_t)n0_ * a.ldws), 0, DBN * a.ldws, 0x00020000)
                  : __builtin_amdgcn_make_buffer_rsrc((void*)(a.asc + (size_t)m0_ * a.lds), 0, DBM * a.lds, 0x00020000);
    f16* base = smem + SCH + sb * 2048 + wave * 512;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base, 16, lane * 16, grp * 2048 + (wave & 1) * 1024, 0, 0);
  };
  // this lane's scale dwords of buffer sb; shift_sc then moves bytes so
  // that bytes 0 and 2 are k-steps 0 and 1
  const int sh = 8 * (g4 >> 1);
  auto read_sc = [&](int sb) __attribute__((always_inline)) {
    const unsigned* sp = reinterpret_cast<const unsigned*>(smem + SCH + sb * 2048) + (g4 & 1);
#pragma unroll
    for (int i = 0; i < TM; ++i) asc[i] = (int)sp[(wm * 128 + i * 16 + l16) * 2];
#pragma unroll
    for (int j = 0; j < TN; ++j) wsc[j] = (int)sp[512 + (wn * 128 + j * 16 + l16) * 2];
  };
  auto shift_sc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i) asc[i] = (int)((unsigned)asc[i] >> sh);
#pragma unroll
    for (int j = 0; j < TN; ++j) wsc[j] = (int)((unsigned)wsc[j] >> sh);
  };
  // k-tile t of stage s: k-step 0 (reads k-step 1), barrier, k-step 1
  // (reads k-step 0 of the next k-tile when rdn; loads k-tile t + 2 into
  // stage s when ld)
  // (rsc: after the barrier, also read the scale dwords of buffer sb, for
  // the fp4 k-tile that follows)
  auto ktile = [&](bool fp4, int s, int t, bool rdn, bool ld, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                   bool rsc = false, int sb = 0) __attribute__((always_inline)) {
    pin_acc();
    step(fp4, 0, true, s, 1, ra, rb, false, 0, 0);
    sync_tile();
    if constexpr (LO4)
      if (rsc) read_sc(sb);
    step(fp4, 1, rdn, s ^ 1, 0, ra, rb, ld, s, t + 2);
  };
  // k-tiles 0 and 1 of the unit at (tm, tn, kt0) (LO4: and its first
  // group's scales, into buffer 0)
  auto prologue = [&](int tm, int tn) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ra = rsrc_a(tm * DBM), rb = rsrc_b(tn * DBN);
#pragma unroll
    for (int q = 0; q < NQ; ++q) load1(ra, rb, 0, 0, q);
#pragma unroll
    for (int q = 0; q < NQ; ++q) load1(ra, rb, 1, 1, q);
    if constexpr (LO4) load_sc(tm * DBM, tn * DBN, 0, kt0 / 5);
  };

  int tm, tn;
  tile_rc(seq0, tm, tn, kt0);
  prologue(tm, tn);
  for (int sq = seq0; sq < seq_end; sq += seq_step) {
    const int m0 = tm * DBM, n0 = tn * DBN;
    const size_t obase = (size_t)(kt0 / KT) * a.pstride;  // partial plane of a split unit
    const __amdgpu_buffer_rsrc_t ra = rsrc_a(m0), rb = rsrc_b(n0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    // the unit's last k-step, after the next unit's prologue
    auto finish = [&](bool fp4) __attribute__((always_inline)) {
      const int nsq = sq + seq_step;
      if (nsq < seq_end) {
        tile_rc(nsq, tm, tn, kt0);
        prologue(tm, tn);
      }
      step(fp4, 1, false, 0, 0, ra, rb, false, 0, 0);
    };
    if constexpr (LO4) {
      // k-tile 0 landed (with the first unit, the later loads of the
      // prologue, k-tile 1 and the scales, may still be in flight; after an
      // epilogue, its stores share the counter)
      if (sq == seq0)
        __builtin_amdgcn_s_waitcnt(wait_imm(NQ + 1, 15));
      else
        __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int r = 0; r < 8; ++r) { readA(0, 0, r); readB(0, 0, 0, r); }
      __builtin_amdgcn_sched_barrier(0);
      // The fp4 k-tile t + 4 of a group from stage s whose scales sit in
      // buffer sb (their dwords were read one k-step before).  nx: a group follows (right after the barrier, its
      // scales go out into the other buffer; then read its first
      // fragments and load its second k-tile).
      auto fp4_tile = [&](int s, int sb, int t, bool nx) __attribute__((always_inline)) {
        pin_acc();
        shift_sc();
        step(true, 0, true, s, 1, ra, rb, false, 0, 0);
        sync_tile();
        if (nx) {
          load_sc(m0, n0, sb ^ 1, (kt0 + t + 5) / 5);
          step(true, 1, true, s ^ 1, 0, ra, rb, true, s, t + 6);
        } else {
          finish(true);
        }
      };
      auto group = [&](int s, int t, bool nx) __attribute__((always_inline)) {
        ktile(false, s, t, true, true, ra, rb);
        ktile(false, s ^ 1, t + 1, true, true, ra, rb);
        ktile(false, s, t + 2, true, true, ra, rb);
        ktile(false, s ^ 1, t + 3, true, nx, ra, rb, true, s);  // + the fp4 k-tile's scale dwords
        fp4_tile(s, s, t, nx);  // groups alternate stages and scale buffers alike
      };
      // groups in pairs (an even number of groups); the last ends with the
      // unit's last k-step
      for (int t = 0; t < KT - 10; t += 10) {
        pin_acc();
        group(0, t, true);
        group(1, t + 5, true);
      }
      group(0, KT - 10, true);
      group(1, KT - 5, false);
    } else {
      // k-tile 0 landed.  After an epilogue its stores share the vector
      // memory counter with these loads, so wait for all of them.
      if (sq == seq0)
        __builtin_amdgcn_s_waitcnt(wait_imm(NQ, 15));
      else
        __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int r = 0; r < 8; ++r) { readA(0, 0, r); readB(0, 0, 0, r); }
      __builtin_amdgcn_sched_barrier(0);
      // k-tiles in pairs (an even number of them)
      for (int t = 0; t < KT - 2; t += 2) {
        pin_acc();
        ktile(false, 0, t, true, true, ra, rb);
        ktile(false, 1, t + 1, true, true, ra, rb);
      }
      ktile(false, 0, KT - 2, true, false, ra, rb);
      step(false, 0, true, 1, 1, ra, rb, false, 0, 0);
      sync_tile();
      finish(false);
    }
    epilogue16<EPI>(a, acc, m0 + wm * 128, n0 + wn * 128, lane, obase);
  }
  __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));  // no LDS-bound load outlives the block
}

// ───────────────────── small-M kernel: register-staged, BM x BN x 64 ─────────────────────
namespace {
__device__ __forceinline__ int swz8(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }
}  // namespace

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_rs_kernel(GemmArgs a) {
  constexpr int BK = 64;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int AL = BM * 8 / 256;  // 16-byte chunks per thread, A tile
  constexpr int BL = BN * 8 / 256;  // 16-byte chunks per thread, B tile
  extern __shared__ u32x4 smem4[];  // [2][(BM + BN) * 8]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(a.M, a.N, BM, BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = a.K;

  const u32x4* ag[AL];
  const u32x4* bg[BL];
  int aslot[AL], bslot[BL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    int q = tid + 256 * i, r = q >> 3, c = q & 7;
    int row = min(m0 + r, a.M - 1);
    ag[i] = reinterpret_cast<const u32x4*>(a.A + (size_t)row * a.lda + c * 8);
    aslot[i] = swz8(r, c);
  }
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    int q = tid + 256 * i, r = q >> 3, c = q & 7;
    bg[i] = reinterpret_cast<const u32x4*>(a.W + (size_t)(n0 + r) * a.kw + c * 8);
    bslot[i] = BM * 8 + swz8(r, c);
  }

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  u32x4 ra[AL], rb[BL];
#pragma unroll
  for (int i = 0; i < AL; ++i) ra[i] = ag[i][0];
#pragma unroll
  for (int i = 0; i < BL; ++i) rb[i] = bg[i][0];
#pragma unroll
  for (int i = 0; i < AL; ++i) smem4[aslot[i]] = ra[i];
#pragma unroll
  for (int i = 0; i < BL; ++i) smem4[bslot[i]] = rb[i];
  __syncthreads();

  const int KT = K / BK;
  const int arow0 = wm * WM + (lane & 31), brow0 = wn * WN + (lane & 31);
  const int hsel = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const u32x4* s = smem4 + cur * (BM + BN) * 8;
    if (kt + 1 < KT) {
      const int off = (kt + 1) * (BK / 8);  // in 16-byte units along K
      const int offw = off >= a.kw / 8 ? off - a.kw / 8 : off;  // W wraps every kw (K is kw or 2 kw)
#pragma unroll
      for (int i = 0; i < AL; ++i) ra[i] = ag[i][off];
#pragma unroll
      for (int i = 0; i < BL; ++i) rb[i] = bg[i][offw];
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + hsel;
      half8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = __builtin_bit_cast(half8, s[swz8(arow0 + i * 32, c)]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = __builtin_bit_cast(half8, s[BM * 8 + swz8(brow0 + j * 32, c)]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      u32x4* d = smem4 + (cur ^ 1) * (BM + BN) * 8;
#pragma unroll
      for (int i = 0; i < AL; ++i) d[aslot[i]] = ra[i];
#pragma unroll
      for (int i = 0; i < BL; ++i) d[bslot[i]] = rb[i];
    }
    __syncthreads();
  }
  epilogue<EPI, TM, TN>(a, acc, m0 + wm * WM, n0 + wn * WN, lane);
}

namespace {

// the 16 x 16 x 32 kernel with the instruction order that keeps its
// accumulators in AGPRs (LSP = 4, LOFF = 1, BPOS = 1)
template <int EPI, int LO>
hipError_t launch16(const GemmArgs& a, hipStream_t s) {
  constexpr size_t lds = (size_t)DNS * DSTAGE * 2 + (LO == 4 ? 8192 : 0);  // + the lo4 scale buffers
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm16_kernel<EPI, LO, 4, 1, 1>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int tiles = ((a.M + DBM - 1) / DBM) * (a.N / DBN) * a.ksplit;
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
      cus = 256;
    cus &= ~7;
  }
  const int blocks = tiles > cus ? cus : tiles;
  hipLaunchKernelGGL((gemm16_kernel<EPI, LO, 4, 1, 1>), dim3(blocks), dim3(256), lds, s, a);
  return hipGetLastError();
}

// 4-wave launches of the f16 and lo4 forms run the 16 x 16 x 32 kernel
// when a work unit has an even number of k-tiles (lo4: of groups); lo8,
// the 8-wave form and the other counts the 32 x 32 x 16 one
template <int EPI, int NW, int LO = 0>
hipError_t launch_dma(const GemmArgs& a, hipStream_t s) {
  if constexpr (NW == 4 && LO != 8 && EPI != EPI_SWIGLU8) {
    const int kt = a.K / DBK / a.ksplit;  // k-tiles per unit
    if (LO == 4 ? kt % 10 == 0 : (kt % 2 == 0 && kt >= 2)) return launch16<EPI, LO>(a, s);
  }
  constexpr size_t lds = (size_t)DNS * DSTAGE * 2;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_dma_kernel<EPI, NW, LO>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int tiles = ((a.M + DBM - 1) / DBM) * (a.N / DBN) * a.ksplit;
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
      cus = 256;
    cus &= ~7;
  }
  // persistent: one block per CU walks several tiles; fewer tiles than CUs:
  // one block per tile
  const int blocks = tiles > cus ? cus : tiles;
  hipLaunchKernelGGL((gemm_dma_kernel<EPI, NW, LO>), dim3(blocks), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int EPI>
hipError_t launch_rs(const GemmArgs& a, hipStream_t s) {
  constexpr size_t lds = 2 * (BM + BN) * 8 * sizeof(u32x4);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_rs_kernel<BM, BN, EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int blocks = ((a.M + BM - 1) / BM) * (a.N / BN);
  hipLaunchKernelGGL((gemm_rs_kernel<BM, BN, EPI>), dim3(blocks), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& a, int tile, hipStream_t s) {
  if (tile == 0) return launch_dma<EPI, 4>(a, s);
  if (tile == 2) return launch_dma<EPI, 8>(a, s);
  return launch_rs<128, 128, EPI>(a, s);
}

}  // namespace

hipError_t launch_gemm(int epi, const GemmArgs& a, int tile, hipStream_t s) {
  if (a.lo == 8 || a.lo == 4) {  // residual k-tiles: the 4-wave 256 x 256 kernel
    const int group = a.lo == 8 ? 3 : 5;  // k-tiles per group of columns
    if (a.N % 256 != 0 || !a.asc || !a.wsc || (tile != 0 && tile != -1) || (a.K / 64) % (group * a.ksplit) != 0 ||
        (a.lo == 8 ? a.lds % 2 != 0 : (a.lds % 4 != 0 || a.ldws % 4 != 0)))
      return hipErrorInvalidValue;
    if (a.lo == 8) {
      if (a.ksplit > 1) return epi == EPI_F32 ? launch_dma<EPI_F32, 4, 8>(a, s) : hipErrorInvalidValue;
      switch (epi) {
        case EPI_F32: return launch_dma<EPI_F32, 4, 8>(a, s);
        case EPI_RESID: return launch_dma<EPI_RESID, 4, 8>(a, s);
        case EPI_SWIGLU8: return launch_dma<EPI_SWIGLU8, 4, 8>(a, s);
      }
      return hipErrorInvalidValue;
    }
    if (a.ksplit > 1) return epi == EPI_F32 ? launch_dma<EPI_F32, 4, 4>(a, s) : hipErrorInvalidValue;
    switch (epi) {
      case EPI_F32: return launch_dma<EPI_F32, 4, 4>(a, s);
      case EPI_RESID: return launch_dma<EPI_RESID, 4, 4>(a, s);
      case EPI_SWIGLU4: return launch_dma<EPI_SWIGLU4, 4, 4>(a, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.lo != 0) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU8) {
    if (a.N % 256 != 0 || (tile != 0 && tile != -1) || a.ksplit != 1) return hipErrorInvalidValue;
    return launch_dma<EPI_SWIGLU8, 4>(a, s);
  }
  if (a.ksplit > 1) {  // split units: 256 x 256 f32 partial products only
    if (epi != EPI_F32 || (tile != 0 && tile != 2) || a.N % 256 != 0 || (a.K / 64) % a.ksplit != 0)
      return hipErrorInvalidValue;
    return tile == 2 ? launch_dma<EPI_F32, 8>(a, s) : launch_dma<EPI_F32, 4>(a, s);
  }
  if (tile < 0) tile = gemm_pick_tile(a.M, a.N, a.K);
  if ((tile == 0 || tile == 2) && a.N % 256 != 0) tile = 1;
  switch (epi) {
    case EPI_F16: return launch_epi<EPI_F16>(a, tile, s);
    case EPI_F32: return launch_epi<EPI_F32>(a, tile, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, tile, s);
    case EPI_QKV: return launch_epi<EPI_QKV>(a, tile, s);
    case EPI_SWIGLU2: return launch_epi<EPI_SWIGLU2>(a, tile, s);
    case EPI_RESID: return launch_epi<EPI_RESID>(a, tile, s);
    case EPI_GELU: return launch_epi<EPI_GELU>(a, tile, s);
    case EPI_QKROPE:
      if (tile == 0) return launch_dma<EPI_QKROPE, 4>(a, s);
      if (tile == 2) return launch_dma<EPI_QKROPE, 8>(a, s);
      return hipErrorInvalidValue;
    case EPI_VT:
      if (tile == 0) return launch_dma<EPI_VT, 4>(a, s);
      if (tile == 2) return launch_dma<EPI_VT, 8>(a, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace qi21
