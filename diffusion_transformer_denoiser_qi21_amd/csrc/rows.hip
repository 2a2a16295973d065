// Bandwidth-bound row kernels of the denoiser step: the gated residual +
// modulated LayerNorm (rowop), the per-head q/k RMSNorm + RoPE (qkrope),
// the img_in embedding, the final LayerNorm + proj_out, and small helpers
// (gate tanh, weight-plane conversion, RoPE table packing, output commit,
// fill).
//
// Access pattern: every row is read with 16-byte (float4 / 8 x f16) or
// 4-byte-per-lane fully coalesced loads; reductions are wave64 shuffles
// followed by one LDS exchange between the waves of a block.
#include "qi21_internal.h"
#include "lores.h"

namespace qi21 {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// sum over a 256-thread block; red must hold 4 floats; all threads get it
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return r;
}

// mode & 8 of the row ops: chunk c (float4 c of the row, 4c .. 4c+3) of
// the value r written in the lo8 row form (lores.h) to row bytes xb; the
// 16 lanes holding one 64-column block (consecutive lanes, whole groups
// active or not) share its scale, which the first of them stores
__device__ __forceinline__ void lo8_store(bool act, int c, float4v r, uint8_t* __restrict__ xb,
                                          uint8_t* __restrict__ xsc, int row, int h) {
  const half4 hi = half4{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
  const float4v lo = r - float4v{(float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3]};  // exact in f32
  float mx = act ? fmaxf(fmaxf(fabsf(lo[0]), fabsf(lo[1])), fmaxf(fabsf(lo[2]), fabsf(lo[3]))) : 0.0f;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const int ex = lo8_exp(mx);
  if (act) {
    const int e0 = 4 * c;
    *reinterpret_cast<half4*>(xb + 2 * lo8_hi_at(e0)) = hi;
    const float4v v = lo * __builtin_ldexpf(1.0f, -ex);
    *reinterpret_cast<unsigned*>(xb + lo8_lo_at(e0)) = pack_e4m3(v[0], v[1], v[2], v[3]);
    if ((c & 15) == 0) xsc[lo8_sc_at(row, e0, h)] = (uint8_t)(ex + 127);
  }
}

// mode & 16: the same in the lo4 row form, the 8 lanes of a 32-column
// block sharing its scale
__device__ __forceinline__ void lo4_store(bool act, int c, float4v r, uint8_t* __restrict__ xb,
                                          uint8_t* __restrict__ xsc, int row, int h) {
  const half4 hi = half4{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
  const float4v lo = r - float4v{(float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3]};  // exact in f32
  float mx = act ? fmaxf(fmaxf(fabsf(lo[0]), fabsf(lo[1])), fmaxf(fabsf(lo[2]), fabsf(lo[3]))) : 0.0f;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const int ex = lo4_exp(mx);
  if (act) {
    const int e0 = 4 * c;
    *reinterpret_cast<half4*>(xb + 2 * lo4_hi_at(e0)) = hi;
    const float4v v = lo * __builtin_ldexpf(1.0f, -ex);
    *reinterpret_cast<uint16_t*>(xb + lo4_lo_at(e0)) = (uint16_t)pack_e2m1(v[0], v[1], v[2], v[3]);
    if ((c & 7) == 0) xsc[lo4_sc_at(row, e0, h)] = (uint8_t)(ex + 127);
  }
}

// ───────────────────────────── rowop ─────────────────────────────
// One wave per row, four rows per 256-thread block; lane l owns the float4
// chunks l, l + 64, ... of the row (h/4 chunks, at most NJ per lane), so
// both reductions are wave shuffles and no block barrier is needed.  y is
// the sum of nparts planes pstride floats apart (the partial products of a
// GEMM split over K), added in plane order.
template <int MODE, int NJ>
__global__ __launch_bounds__(256) void rowop_kernel(int rows, int h, float* __restrict__ x, const float* __restrict__ y,
                                                   int nparts, size_t pstride, f16* __restrict__ xn, int ldxn,
                                                   const float* __restrict__ mods, int g_off, int s_off, float eps,
                                                   float oscale, uint8_t* __restrict__ xsc) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nc = h >> 2;
  float4v* xr = reinterpret_cast<float4v*>(x + (size_t)row * h);
  float4v v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = lane + 64 * j;
    if (c < nc) {
      v[j] = xr[c];
      if (MODE & 1) {
        float4v yv = reinterpret_cast<const float4v*>(y + (size_t)row * h)[c];
        for (int p = 1; p < nparts; ++p) yv += reinterpret_cast<const float4v*>(y + p * pstride + (size_t)row * h)[c];
        const float4v g = reinterpret_cast<const float4v*>(mods + g_off)[c];
        v[j] = v[j] + g * yv;
        xr[c] = v[j];
      }
    }
  }
  if (!(MODE & 2)) return;
  float sm = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (lane + 64 * j < nc) sm += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  const float mean = wave_sum(sm) / (float)h;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (lane + 64 * j < nc) {
      const float4v d = v[j] - mean;
      q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  const float inv = rsqrtf(wave_sum(q) / (float)h + eps);
  if constexpr ((MODE & 24) != 0) {
    uint8_t* xb = reinterpret_cast<uint8_t*>(xn + (size_t)row * ldxn);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = lane + 64 * j;
      const bool act = c < nc;
      float4v r = float4v{0.0f, 0.0f, 0.0f, 0.0f};
      if (act) r = (v[j] - mean) * inv * (1.0f + reinterpret_cast<const float4v*>(mods + s_off)[c]) * oscale;
      if constexpr ((MODE & 8) != 0)
        lo8_store(act, c, r, xb, xsc, row, h);
      else
        lo4_store(act, c, r, xb, xsc, row, h);
    }
    return;
  }
  half4* xo = reinterpret_cast<half4*>(xn + (size_t)row * ldxn);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = lane + 64 * j;
    if (c < nc) {
      const float4v s = reinterpret_cast<const float4v*>(mods + s_off)[c];
      const float4v r = (v[j] - mean) * inv * (1.0f + s) * oscale;
      const half4 hi = half4{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
      xo[c] = hi;
      if (MODE & 4) {  // rounding error of hi, exact in f32, as the second half
        const float4v e = r - float4v{(float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3]};
        xo[nc + c] = half4{(f16)e[0], (f16)e[1], (f16)e[2], (f16)e[3]};
      }
    }
  }
}

// The same row op with one 256-thread block per row, for wide rows (h >=
// 2048): thread t owns float4 chunks t, t + 256, ... (NJ per thread).  Four
// times as many waves as the one-wave-per-row form, and every load of a
// thread (x, then the nparts planes of y) is issued before its first use,
// so a pass over a few thousand rows keeps enough bytes in flight to
// stream at HBM rate.  y's planes are added in plane order, as above.
// Two rows per block for the modulated LayerNorm alone (mode 2, wide rows):
// both rows' loads go out before either row's reductions, and the two
// rows' reductions share their barriers.  Same arithmetic, in the same
// order, as rowop_wide_kernel.  An odd last row is loaded twice and
// written once.  LO4: xn in the lo4 row form (mode 2 | 16), as
// rowop_wide_kernel writes it.
template <int NJ, bool LO4>
__global__ __launch_bounds__(256) void rownorm2_kernel(int rows, int h, const float* __restrict__ x,
                                                       f16* __restrict__ xn, int ldxn, const float* __restrict__ mods,
                                                       int s_off, float eps, float oscale, uint8_t* __restrict__ xsc) {
  __shared__ float red[2][4];
  const int t = threadIdx.x, w = t >> 6;
  const int r0 = blockIdx.x * 2;
  const bool two = r0 + 1 < rows;
  const int nc = h >> 2;
  float4v v[2][NJ];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float4v* xr = reinterpret_cast<const float4v*>(x + (size_t)(two ? r0 + k : r0) * h);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = t + 256 * j;
      if (c < nc) v[k][j] = xr[c];
    }
  }
  float sm[2] = {0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (t + 256 * j < nc) sm[k] += (v[k][j][0] + v[k][j][1]) + (v[k][j][2] + v[k][j][3]);
#pragma unroll
  for (int k = 0; k < 2; ++k) sm[k] = wave_sum(sm[k]);
  if ((t & 63) == 0) {
    red[0][w] = sm[0];
    red[1][w] = sm[1];
  }
  __syncthreads();
  float mean[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) mean[k] = (red[k][0] + red[k][1] + red[k][2] + red[k][3]) / (float)h;
  __syncthreads();
  float q[2] = {0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (t + 256 * j < nc) {
        const float4v d = v[k][j] - mean[k];
        q[k] += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
      }
#pragma unroll
  for (int k = 0; k < 2; ++k) q[k] = wave_sum(q[k]);
  if ((t & 63) == 0) {
    red[0][w] = q[0];
    red[1][w] = q[1];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (k == 1 && !two) break;
    const float inv = rsqrtf((red[k][0] + red[k][1] + red[k][2] + red[k][3]) / (float)h + eps);
    if constexpr (LO4) {
      uint8_t* xb = reinterpret_cast<uint8_t*>(xn + (size_t)(r0 + k) * ldxn);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = t + 256 * j;
        const bool act = c < nc;
        float4v r = float4v{0.0f, 0.0f, 0.0f, 0.0f};
        if (act) r = (v[k][j] - mean[k]) * inv * (1.0f + reinterpret_cast<const float4v*>(mods + s_off)[c]) * oscale;
        lo4_store(act, c, r, xb, xsc, r0 + k, h);
      }
    } else {
      half4* xo = reinterpret_cast<half4*>(xn + (size_t)(r0 + k) * ldxn);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = t + 256 * j;
        if (c < nc) {
          const float4v sc = reinterpret_cast<const float4v*>(mods + s_off)[c];
          const float4v r = (v[k][j] - mean[k]) * inv * (1.0f + sc) * oscale;
          xo[c] = half4{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
        }
      }
    }
  }
}

// NP > 0: the number of planes of y, known at compile time (1 to 4); 0:
// nparts at run time.
template <int MODE, int NJ, int NP>
__global__ __launch_bounds__(256) void rowop_wide_kernel(int rows, int h, float* __restrict__ x,
                                                         const float* __restrict__ y, int nparts, size_t pstride,
                                                         f16* __restrict__ xn, int ldxn, const float* __restrict__ mods,
                                                         int g_off, int s_off, float eps, float oscale,
                                                         uint8_t* __restrict__ xsc) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const int nc = h >> 2;
  float4v* xr = reinterpret_cast<float4v*>(x + (size_t)row * h);
  float4v v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = t + 256 * j;
    if (c < nc) v[j] = xr[c];
  }
  if (MODE & 1) {
    float4v yv[NJ];
    const float4v* yr = reinterpret_cast<const float4v*>(y + (size_t)row * h);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = t + 256 * j;
      if (c < nc) yv[j] = yr[c];
    }
    if (NP > 0) {
      // a known plane count: every plane's loads go out before the first
      // add (the sum stays in plane order)
      float4v yq[NP > 1 ? NP - 1 : 1][NJ];
#pragma unroll
      for (int p = 1; p < NP; ++p) {
        const float4v* yp = reinterpret_cast<const float4v*>(y + p * pstride + (size_t)row * h);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int c = t + 256 * j;
          if (c < nc) yq[p - 1][j] = yp[c];
        }
      }
#pragma unroll
      for (int p = 1; p < NP; ++p)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (t + 256 * j < nc) yv[j] += yq[p - 1][j];
    } else {
      for (int p = 1; p < nparts; ++p) {
        const float4v* yp = reinterpret_cast<const float4v*>(y + p * pstride + (size_t)row * h);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int c = t + 256 * j;
          if (c < nc) yv[j] += yp[c];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = t + 256 * j;
      if (c < nc) {
        const float4v g = reinterpret_cast<const float4v*>(mods + g_off)[c];
        v[j] = v[j] + g * yv[j];
        xr[c] = v[j];
      }
    }
  }
  if (!(MODE & 2)) return;
  float sm = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (t + 256 * j < nc) sm += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  const float mean = block_sum256(sm, red) / (float)h;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (t + 256 * j < nc) {
      const float4v d = v[j] - mean;
      q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
  const float inv = rsqrtf(block_sum256(q, red) / (float)h + eps);
  if constexpr ((MODE & 24) != 0) {
    uint8_t* xb = reinterpret_cast<uint8_t*>(xn + (size_t)row * ldxn);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = t + 256 * j;
      const bool act = c < nc;
      float4v r = float4v{0.0f, 0.0f, 0.0f, 0.0f};
      if (act) r = (v[j] - mean) * inv * (1.0f + reinterpret_cast<const float4v*>(mods + s_off)[c]) * oscale;
      if constexpr ((MODE & 8) != 0)
        lo8_store(act, c, r, xb, xsc, row, h);
      else
        lo4_store(act, c, r, xb, xsc, row, h);
    }
    return;
  }
  half4* xo = reinterpret_cast<half4*>(xn + (size_t)row * ldxn);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = t + 256 * j;
    if (c < nc) {
      const float4v s = reinterpret_cast<const float4v*>(mods + s_off)[c];
      const float4v r = (v[j] - mean) * inv * (1.0f + s) * oscale;
      const half4 hi = half4{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
      xo[c] = hi;
      if (MODE & 4) {  // rounding error of hi, exact in f32, as the second half
        const float4v e = r - float4v{(float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3]};
        xo[nc + c] = half4{(f16)e[0], (f16)e[1], (f16)e[2], (f16)e[3]};
      }
    }
  }
}

namespace {
#define QI21_ROWOP_ARGS rows, h, x, y, np, ps, xn, ldxn, mods, g_off, s_off, eps, oscale, xsc
template <int NJ, int NP>
hipError_t launch_rowop_wide_np(int rows, int h, int mode, float* x, const float* y, int np, size_t ps, f16* xn,
                                int ldxn, const float* mods, int g_off, int s_off, float eps, float oscale, uint8_t* xsc,
                                hipStream_t s) {
  const dim3 grid(rows), block(256);
  switch (mode) {
    case 1: hipLaunchKernelGGL((rowop_wide_kernel<1, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 2: hipLaunchKernelGGL((rowop_wide_kernel<2, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 3: hipLaunchKernelGGL((rowop_wide_kernel<3, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 6: hipLaunchKernelGGL((rowop_wide_kernel<6, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 7: hipLaunchKernelGGL((rowop_wide_kernel<7, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 10: hipLaunchKernelGGL((rowop_wide_kernel<10, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 11: hipLaunchKernelGGL((rowop_wide_kernel<11, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 18: hipLaunchKernelGGL((rowop_wide_kernel<18, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 19: hipLaunchKernelGGL((rowop_wide_kernel<19, NJ, NP>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NJ>
hipError_t launch_rowop_wide(int rows, int h, int mode, float* x, const float* y, int np, size_t ps, f16* xn,
                             int ldxn, const float* mods, int g_off, int s_off, float eps, float oscale, uint8_t* xsc,
                             hipStream_t s) {
  // three or four planes with every plane's loads issued up front (1024
  // rows x 4096: 22.1 against 23.6 us with four planes, 16.5 against 21.1
  // with three); one or two planes with the plane loop, which measured
  // faster there (2048 rows, two planes: 31.0 against 36.7 us)
#define QI21_WIDE_ARGS rows, h, mode, x, y, np, ps, xn, ldxn, mods, g_off, s_off, eps, oscale, xsc, s
  if ((mode & 1) && np == 3) return launch_rowop_wide_np<NJ, 3>(QI21_WIDE_ARGS);
  if ((mode & 1) && np == 4) return launch_rowop_wide_np<NJ, 4>(QI21_WIDE_ARGS);
  return launch_rowop_wide_np<NJ, 0>(QI21_WIDE_ARGS);
#undef QI21_WIDE_ARGS
}
}  // namespace

namespace {
template <int NJ>
hipError_t launch_rowop_nj(int rows, int h, int mode, float* x, const float* y, int np, size_t ps, f16* xn,
                           int ldxn, const float* mods, int g_off, int s_off, float eps, float oscale, uint8_t* xsc,
                           hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
  switch (mode) {
    case 1: hipLaunchKernelGGL((rowop_kernel<1, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 2: hipLaunchKernelGGL((rowop_kernel<2, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 3: hipLaunchKernelGGL((rowop_kernel<3, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 6: hipLaunchKernelGGL((rowop_kernel<6, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 7: hipLaunchKernelGGL((rowop_kernel<7, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 10: hipLaunchKernelGGL((rowop_kernel<10, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 11: hipLaunchKernelGGL((rowop_kernel<11, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 18: hipLaunchKernelGGL((rowop_kernel<18, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    case 19: hipLaunchKernelGGL((rowop_kernel<19, NJ>), grid, block, 0, s, QI21_ROWOP_ARGS); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
#undef QI21_ROWOP_ARGS
}  // namespace

hipError_t launch_rowop(int rows, int h, int mode, float* x, const float* y, f16* xn, const float* mods,
                        int g_off, int s_off, float eps, float oscale, hipStream_t s, int nparts, size_t pstride,
                        uint8_t* xsc, int ldxn) {
  if (rows <= 0) return hipSuccess;
  if ((mode & 8) && (!xsc || h % 128 != 0 || (mode & 20) || !(mode & 2))) return hipErrorInvalidValue;
  if ((mode & 16) && (!xsc || h % 256 != 0 || (mode & 12) || !(mode & 2))) return hipErrorInvalidValue;
  if (!ldxn) ldxn = (mode & 4) ? 2 * h : (mode & 8) ? 3 * h / 2 : (mode & 16) ? 5 * h / 4 : h;
#define QI21_LAUNCH_ARGS rows, h, mode, x, y, nparts, pstride, xn, ldxn, mods, g_off, s_off, eps, oscale, xsc, s
  if (h <= 1024) return launch_rowop_nj<4>(QI21_LAUNCH_ARGS);
  // the block-per-row form for wide rows, except on long passes that also
  // add a residual: there the one-wave-per-row form streamed faster
  // (4096 rows x 4096: 41 against 47 us; without the residual 19 against
  // 23 us for the block form, and 24 against 27 us on 1024 rows with four
  // planes)
  if (h < 2048 || (h <= 4096 && (mode & 1) && rows > 2048)) return launch_rowop_nj<16>(QI21_LAUNCH_ARGS);
  if (h <= 4096) {
    // the LayerNorm passes of long steps: two rows per block (4096 rows: 17.0
    // against 19.5 us; even at 16384 rows, 0.3 us slower at 1024)
    if (mode == 2 && rows > 2048) {
      hipLaunchKernelGGL((rownorm2_kernel<4, false>), dim3((rows + 1) / 2), dim3(256), 0, s, rows, h, x, xn, ldxn, mods,
                         s_off, eps, oscale, xsc);
      return hipGetLastError();
    }
    if (mode == (2 | 16) && rows > 2048) {
      hipLaunchKernelGGL((rownorm2_kernel<4, true>), dim3((rows + 1) / 2), dim3(256), 0, s, rows, h, x, xn, ldxn, mods,
                         s_off, eps, oscale, xsc);
      return hipGetLastError();
    }
    return launch_rowop_wide<4>(QI21_LAUNCH_ARGS);
  }
  return launch_rowop_wide<8>(QI21_LAUNCH_ARGS);
#undef QI21_LAUNCH_ARGS
}

// ───────────────────────────── RoPE table packing ─────────────────────────────
// One thread per float4 of the packed table: out[r][4m ..] = cos[r][2m],
// cos[r][2m + 1], sin[r][2m], sin[r][2m + 1], so the q|k epilogue reads the
// cos and sin of two adjacent pairs in one 16-byte load.
__global__ __launch_bounds__(256) void rope_pack_kernel(int n, const float* __restrict__ cosb,
                                                        const float* __restrict__ sinb, float* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;  // (row, m)
  if (i >= (long)n * 32) return;
  const long r = i >> 5;
  const int mm = (int)(i & 31);
  const floatx2 c = *reinterpret_cast<const floatx2*>(cosb + r * 64 + 2 * mm);
  const floatx2 s = *reinterpret_cast<const floatx2*>(sinb + r * 64 + 2 * mm);
  *reinterpret_cast<float4v*>(out + r * 128 + 4 * mm) = float4v{c[0], c[1], s[0], s[1]};
}

hipError_t launch_rope_pack(int n, const float* cos, const float* sin, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_pack_kernel, dim3((unsigned)(((long)n * 32 + 255) / 256)), dim3(256), 0, s, n, cos, sin, out);
  return hipGetLastError();
}

// ───────────────────────────── txt_in norm ─────────────────────────────
// One 256-thread block per text row of width c (c % 4 == 0, c <= 8192):
// xn = f16(f32(v / sqrt(mean(v^2) + eps)) * (w + 1)), the sum of squares
// and the scaling in float64 ([QI] embed_text).
__global__ __launch_bounds__(256) void txtnorm_kernel(int c, const float* __restrict__ feats,
                                                      const float* __restrict__ w, float eps, f16* __restrict__ xn) {
  __shared__ double red[4];
  const int row = blockIdx.x, t = threadIdx.x;
  const int nc = c >> 2;
  const float4v* fr = reinterpret_cast<const float4v*>(feats + (size_t)row * c);
  float4v v[8];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = t + 256 * j;
    if (k < nc) {
      v[j] = fr[k];
      ss += ((double)v[j][0] * v[j][0] + (double)v[j][1] * v[j][1]) + ((double)v[j][2] * v[j][2] + (double)v[j][3] * v[j][3]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  const double inv = 1.0 / sqrt((red[0] + red[1] + red[2] + red[3]) / (double)c + (double)eps);
  half4* xo = reinterpret_cast<half4*>(xn + (size_t)row * c);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = t + 256 * j;
    if (k < nc) {
      const float4v wv = reinterpret_cast<const float4v*>(w)[k];
      half4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (f16)((float)((double)v[j][e] * inv) * (wv[e] + 1.0f));
      xo[k] = o;
    }
  }
}

hipError_t launch_txtnorm(int rows, int c, const float* feats, const float* w, float eps, f16* xn, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(txtnorm_kernel, dim3(rows), dim3(256), 0, s, c, feats, w, eps, xn);
  return hipGetLastError();
}

// ───────────────────────────── qkrope ─────────────────────────────
// One wave per (row, head, q|k); lane l owns the interleaved pair
// (2l, 2l+1) of the head, which is also RoPE column l.
__global__ __launch_bounds__(256) void qkrope_kernel(int rows, int heads, f16* __restrict__ panel, int ldp,
                                                     const float* __restrict__ norm_q,
                                                     const float* __restrict__ norm_k,
                                                     const float* __restrict__ cosb,
                                                     const float* __restrict__ sinb, float eps,
                                                     f16* __restrict__ kdst, int ldk) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);  // (head, q|k) index
  const int row = blockIdx.y;
  if (item >= 2 * heads) return;
  const bool isk = item >= heads;
  const int hd = isk ? item - heads : item;
  const int col = (isk ? heads * 128 : 0) + hd * 128 + 2 * lane;
  const half2v pv = *reinterpret_cast<const half2v*>(panel + (size_t)row * ldp + col);
  const float a = (float)pv[0], b = (float)pv[1];
  const float ss = wave_sum(a * a + b * b);
  const float inv = rsqrtf(ss * (1.0f / 128.0f) + eps);
  const float* w = isk ? norm_k : norm_q;
  const float na = (a * inv) * w[2 * lane], nb = (b * inv) * w[2 * lane + 1];
  const float c = cosb[(size_t)row * 64 + lane], sn = sinb[(size_t)row * 64 + lane];
  const half2v r = half2v{(f16)(na * c - nb * sn), (f16)(na * sn + nb * c)};
  if (isk && kdst)
    *reinterpret_cast<half2v*>(kdst + (size_t)row * ldk + hd * 128 + 2 * lane) = r;
  else
    *reinterpret_cast<half2v*>(panel + (size_t)row * ldp + col) = r;
}

hipError_t launch_qkrope(int rows, int heads, f16* panel, int ldp, const float* norm_q, const float* norm_k,
                         const float* cosb, const float* sinb, float eps, f16* kdst, int ldk, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((2 * heads + 3) / 4, rows);
  hipLaunchKernelGGL(qkrope_kernel, grid, dim3(256), 0, s, rows, heads, panel, ldp, norm_q, norm_k, cosb, sinb,
                     eps, kdst, ldk);
  return hipGetLastError();
}

// ───────────────────────────── embed ─────────────────────────────
// Block tile 64 rows x 64 columns, K = 64; tok and img_in tiles in LDS,
// each thread 4 rows x 4 columns (columns tx, tx+16, tx+32, tx+48).
__global__ __launch_bounds__(256) void embed_kernel(int rows, int h, const float* __restrict__ tok,
                                                    const float* __restrict__ w, float* __restrict__ x) {
  __shared__ float st[64][65];
  __shared__ float sw[64][65];
  const int t = threadIdx.x;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = t; i < 64 * 64; i += 256) {
    const int r = i >> 6, k = i & 63;
    st[r][k] = tok[(size_t)min(r0 + r, rows - 1) * 64 + k];
    sw[r][k] = w[(size_t)(c0 + r) * 64 + k];
  }
  __syncthreads();
  const int ty = t >> 4, tx = t & 15;
  float acc[4][4] = {};
  for (int k = 0; k < 64; ++k) {
    float av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = st[ty * 4 + i][k];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = sw[tx + 16 * j][k];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + ty * 4 + i;
    if (r < rows)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[(size_t)r * h + c0 + tx + 16 * j] = acc[i][j];
  }
}

hipError_t launch_embed(int rows, int h, const float* tok, const float* img_in, float* x, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  dim3 grid(h / 64, (rows + 63) / 64);
  hipLaunchKernelGGL(embed_kernel, grid, dim3(256), 0, s, rows, h, tok, img_in, x);
  return hipGetLastError();
}

// ───────────────────────────── final ─────────────────────────────
// out[r][o] = sum_c LN(x[r])[c] fs[c] W[o][c] for the 64 outputs o, W the
// proj_out weight [64][h].  A block takes 16 rows with 16 waves.  Phase 1:
// wave w finds mean and inverse std of row w in one pass of sums shifted by
// the row's first element (the shift keeps the variance free of
// cancellation when the mean is large).  Phase 2: wave w contracts the
// sixteenth [w h/16, (w+1) h/16) of the c range on v_mfma_f32_16x16x4_f32.
// For a 16-wide c-slice at c0, lane l (row l % 16, quarter q = l / 16) holds
// the normalised x[row][c0 + 4q .. +3] and W[16 nb + l % 16][c0 + 4q .. +3]
// for the four 16-column blocks nb of o; MFMA j pairs element j of both, so
// the four MFMAs of a slice cover its 16 c once each.  Loads run one to two
// slices ahead of the MFMAs.  Phase 3: the 16 partial 16 x 64 tiles are summed
// through LDS.
namespace {
struct FinalSlice {
  float4v x, f, w[4];
};
}  // namespace

// v = (LN(x) fs) proj_out^T for 16 rows per block in one pass over x.  With
// s the row's first element, LN(x)_c fs_c = inv (x_c - mean) fs_c, so
//   v_o = inv (sum_c (x_c - s) fs_c w_oc - (mean - s) sum_c fs_c w_oc).
// Wave w streams columns [w h / 16, (w + 1) h / 16) of all 16 rows: the
// 16x16x4 f32 MFMAs take (x - s) fs against proj_out, and the same loads
// give each row's sums of (x - s) and (x - s)^2 (the shift keeps the
// variance sum well conditioned) and each output's sum_c fs_c w_oc.
// (amdgpu_waves_per_eu: the scheduler may keep 128 registers per lane, so the
// loads run ahead instead of being moved next to their use)
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4, 4))) void final_kernel(int rows, int h, const float* __restrict__ x,
                                                     const float* __restrict__ fs, const float* __restrict__ w,
                                                     float eps, float* __restrict__ out, int* __restrict__ flag) {
  constexpr int NWV = 16;
  __shared__ float part[NWV][16][64];
  __shared__ float bpart[NWV][64];
  __shared__ float s1p[NWV][16], s2p[NWV][16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r0 = blockIdx.x * 16;
  const int rl = lane & 15, q = lane >> 4;
  // rows of the block past the end read as zeros (and are not stored)
  const float shift = r0 + rl < rows ? x[(size_t)(r0 + rl) * h] : 0.0f;
  // Buffer loads (an intrinsic, not a plain load, so the compiler does not
  // fold the two buffers' loads back into one load next to the MFMAs).
  const auto rx = __builtin_amdgcn_make_buffer_rsrc((void*)(x + (size_t)r0 * h), 0, min(rows - r0, 16) * h * 4,
                                                    0x00020000);
  const auto rf = __builtin_amdgcn_make_buffer_rsrc((void*)fs, 0, h * 4, 0x00020000);
  const auto rw = __builtin_amdgcn_make_buffer_rsrc((void*)w, 0, 64 * h * 4, 0x00020000);
  const int xo = (rl * h + 4 * q) * 4, fo = 4 * q * 4, wo = (rl * h + 4 * q) * 4, wnb = 16 * h * 4;
  const int cq = h / NWV, cb = wave * cq, ce = cb + cq;
  auto ld = [&](__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  };
  auto fetch = [&](int c, FinalSlice& sl) {
    c = min(c, ce - 16) * 4;  // past the end: the last slice again
    sl.x = ld(rx, xo + c);
    sl.f = ld(rf, fo + c);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) sl.w[nb] = ld(rw, wo + nb * wnb + c);
  };
  // lane (rl, q) of a slice: row rl, columns 4q .. 4q + 3 (MFMA A row rl,
  // k = q) and, for output 16 nb + rl, the same columns of proj_out (B k =
  // q, column rl)
  floatx4 acc[4];
  float bsum[4], s1 = 0.0f, s2 = 0.0f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    acc[nb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    bsum[nb] = 0.0f;
  }
  auto mma = [&](const FinalSlice& sl) {
    const float4v d = sl.x - shift;
    s1 += (d[0] + d[1]) + (d[2] + d[3]);
    s2 += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    const float4v av = d * sl.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], sl.w[nb][j], acc[nb], 0, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      bsum[nb] += (sl.f[0] * sl.w[nb][0] + sl.f[1] * sl.w[nb][1]) + (sl.f[2] * sl.w[nb][2] + sl.f[3] * sl.w[nb][3]);
  };
  // two slices in flight: each buffer is refilled right after its MFMAs
  // (cq is a multiple of 16; an odd count of slices skips the last sb)
  FinalSlice sa, sb;
  fetch(cb, sa);
  fetch(cb + 16, sb);
  for (int c0 = cb; c0 < ce; c0 += 32) {
    mma(sa);
    fetch(c0 + 32, sa);
    if (c0 + 16 < ce) {
      mma(sb);
      fetch(c0 + 48, sb);
    }
  }
  // the four lanes of a row (q = 0..3) hold its four column classes
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    s1 += __shfl_xor(s1, o);
    s2 += __shfl_xor(s2, o);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) bsum[nb] += __shfl_xor(bsum[nb], o);
  }
  if (q == 0) {
    s1p[wave][rl] = s1;
    s2p[wave][rl] = s2;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) bpart[wave][16 * nb + rl] = bsum[nb];
  }
  // lane l holds rows 4q .. 4q+3 of column l % 16 of each 16-column block
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][4 * q + i][nb * 16 + rl] = acc[nb][i];
  __syncthreads();
  const int r = t >> 6, o = t & 63;  // one output per thread
  float a = 0.0f, b = 0.0f, m1 = 0.0f, m2 = 0.0f;
#pragma unroll
  for (int k = 0; k < NWV; ++k) {
    a += part[k][r][o];
    b += bpart[k][o];
    m1 += s1p[k][r];
    m2 += s2p[k][r];
  }
  m1 /= (float)h;  // mean - shift
  const float var = fmaxf(m2 / (float)h - m1 * m1, 0.0f);
  const float v = rsqrtf(var + eps) * (a - m1 * b);
  if (r0 + r < rows) {
    out[(size_t)(r0 + r) * 64 + o] = v;
    if (!__builtin_isfinite(v)) atomicOr(flag, 1);
  }
}

hipError_t launch_final(int rows, int h, const float* x, const float* fs, const float* proj_out, float eps, float* out,
                        int* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(final_kernel, dim3((rows + 15) / 16), dim3(1024), 0, s, rows, h, x, fs, proj_out, eps, out, flag);
  return hipGetLastError();
}

// ───────────────────────────── helpers ─────────────────────────────
__global__ void commit_kernel(int count, const float* __restrict__ src, float* __restrict__ dst,
                              const int* __restrict__ flag) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (*flag == 0 && i < count / 4)
    reinterpret_cast<float4v*>(dst)[i] = reinterpret_cast<const float4v*>(src)[i];
}

hipError_t launch_commit(int count, const float* src, float* dst, const int* flag, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(commit_kernel, dim3((count / 4 + 255) / 256), dim3(256), 0, s, count, src, dst, flag);
  return hipGetLastError();
}

__global__ void mods_kernel(int h, const float* __restrict__ m, float* __restrict__ d) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < 4 * h) {
    const int chunk = i / h;
    d[i] = (chunk == 1 || chunk == 3) ? tanhf(m[i]) : m[i];
  }
}

hipError_t launch_mods(int h, const float* mods, float* mods_dev, hipStream_t s) {
  hipLaunchKernelGGL(mods_kernel, dim3((4 * h + 255) / 256), dim3(256), 0, s, h, mods, mods_dev);
  return hipGetLastError();
}

__global__ void plane_kernel(int src_dtype, const void* __restrict__ src, int rows, int cols, f16* __restrict__ dst,
                             int group, int gstride, int goff, int ldd, int lo) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)rows * cols) return;
  const int r = (int)(i / cols), c = (int)(i - (size_t)r * cols);
  float v;
  if (src_dtype == 0) {
    v = reinterpret_cast<const float*>(src)[i];
  } else if (src_dtype == 1) {
    const unsigned short b = reinterpret_cast<const unsigned short*>(src)[i];
    v = __uint_as_float((unsigned)b << 16);
  } else {
    v = (float)reinterpret_cast<const f16*>(src)[i];
  }
  const int dr = (r / group) * gstride + goff + r % group;
  dst[(size_t)dr * ldd + (lo == 8 ? lo8_hi_at(c) : lo == 4 ? lo4_hi_at(c) : c)] = (f16)v;
}

hipError_t launch_plane(int src_dtype, const void* src, int rows, int cols, f16* dst, int group, int gstride,
                        int goff, hipStream_t s, int ldd, int lo) {
  const size_t n = (size_t)rows * cols;
  if ((lo == 8 && cols % 128 != 0) || (lo == 4 && cols % 256 != 0) || (lo != 0 && lo != 8 && lo != 4))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(plane_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src_dtype, src, rows, cols,
                     dst, group, gstride, goff, ldd ? ldd : cols, lo);
  return hipGetLastError();
}

// One 256-thread block per row of a lo8 weight plane: the row's largest
// |w| over its f16 values (a block max), then every residual byte =
// e4m3(w 2^-e) and the row's E8M0 scale.
__global__ __launch_bounds__(256) void plane8_kernel(int cols, f16* __restrict__ plane, int ld,
                                                     uint8_t* __restrict__ sc) {
  __shared__ float red[4];
  const int row = blockIdx.x, t = threadIdx.x;
  f16* pr = plane + (size_t)row * ld;
  uint8_t* pb = reinterpret_cast<uint8_t*>(pr);
  float mx = 0.0f;
  for (int c = 4 * t; c < cols; c += 1024) {
    const half4 w = *reinterpret_cast<const half4*>(pr + lo8_hi_at(c));
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf((float)w[0]), fabsf((float)w[1])), fmaxf(fabsf((float)w[2]), fabsf((float)w[3]))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int ex = lo8_exp(mx);
  const float inv = __builtin_ldexpf(1.0f, -ex);
  for (int c = 4 * t; c < cols; c += 1024) {
    const half4 w = *reinterpret_cast<const half4*>(pr + lo8_hi_at(c));
    *reinterpret_cast<unsigned*>(pb + lo8_lo_at(c)) =
        pack_e4m3((float)w[0] * inv, (float)w[1] * inv, (float)w[2] * inv, (float)w[3] * inv);
  }
  if (t == 0) sc[row] = (uint8_t)(ex + 127);
}

// One 256-thread block per row of a lo4 weight plane: per 32-column block
// (8 consecutive threads) the largest |w| of its f16 values, then the
// block's e2m1 copy w 2^-e and its E8M0 scale in the blocked lo4 order.
__global__ __launch_bounds__(256) void plane4_kernel(int cols, f16* __restrict__ plane, int ld,
                                                     uint8_t* __restrict__ sc) {
  const int row = blockIdx.x, t = threadIdx.x;
  f16* pr = plane + (size_t)row * ld;
  uint8_t* pb = reinterpret_cast<uint8_t*>(pr);
  for (int c0 = 0; c0 < cols; c0 += 1024) {
    // (cols % 256 == 0: whole waves are active or not)
    const int c = c0 + 4 * t;
    const bool act = c < cols;
    half4 w = half4{(f16)0.0f, (f16)0.0f, (f16)0.0f, (f16)0.0f};
    if (act) w = *reinterpret_cast<const half4*>(pr + lo4_hi_at(c));
    float mx = fmaxf(fmaxf(fabsf((float)w[0]), fabsf((float)w[1])), fmaxf(fabsf((float)w[2]), fabsf((float)w[3])));
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const int ex = lo4_exp(mx);
    if (act) {
      const float inv = __builtin_ldexpf(1.0f, -ex);
      *reinterpret_cast<uint16_t*>(pb + lo4_lo_at(c)) =
          (uint16_t)pack_e2m1((float)w[0] * inv, (float)w[1] * inv, (float)w[2] * inv, (float)w[3] * inv);
      if ((t & 7) == 0) sc[lo4_sc_at(row, c, cols)] = (uint8_t)(ex + 127);
    }
  }
}

hipError_t launch_plane4(int rows, int cols, f16* plane, int ld, uint8_t* sc, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cols % 256 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plane4_kernel, dim3(rows), dim3(256), 0, s, cols, plane, ld, sc);
  return hipGetLastError();
}

hipError_t launch_plane8(int rows, int cols, f16* plane, int ld, uint8_t* sc, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cols % 128 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plane8_kernel, dim3(rows), dim3(256), 0, s, cols, plane, ld, sc);
  return hipGetLastError();
}

__global__ void fill32_kernel(uint32_t* p, uint32_t v, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void scale_kernel(int n, const float* __restrict__ src, float f, float* __restrict__ dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i] * f;
}

hipError_t launch_scale(int n, const float* src, float f, float* dst, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, src, f, dst);
  return hipGetLastError();
}

hipError_t launch_fill32(void* p, uint32_t value, size_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(fill32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(p), value, count);
  return hipGetLastError();
}

}  // namespace qi21
