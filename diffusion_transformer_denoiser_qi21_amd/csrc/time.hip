// Time path of the denoiser on the device, and the sampler's update.
//
// The sinusoidal timestep embedding and the small bias-free projections
// that turn it into the shared block modulation and the final-norm scale
// ([QI] Qi21Dit::temb, Qi21Dit::mods) run here, so a multi-step sampler
// needs no host work per step.  The projections are matrix-vector products
// over f32 weights with float64 partial sums, the host path's precision.
// They are HBM-bound (about 0.4 GB of f32 weights per step at dim 4096),
// so each row is one wave streaming 16-byte loads.
#include "qi21_internal.h"

namespace qi21 {

typedef float float4v __attribute__((ext_vector_type(4)));

// e[i] = cos(1000 t f_i), e[128 + i] = sin(1000 t f_i), f_i = exp(-ln(10000) i / 128),
// each step in f32 as on the host path; 128 threads
__global__ void temb_sin_kernel(float t, float* __restrict__ e) {
  const int i = threadIdx.x;
  const float ts = 1000.0f * t;
  const float f = expf(-logf(10000.0f) * (float)i / 128.0f);
  const float a = ts * f;
  e[i] = cosf(a);
  e[128 + i] = sinf(a);
}

// y[o] = f32(sum_k w[o][k] x[k]) with float64 partial sums, one wave per
// row (cols % 4 == 0).  MODE 1: y = silu(y); MODE 2: y = 1 + y.
template <int MODE>
__global__ __launch_bounds__(256) void gemv_kernel(int rows, int cols, const float* __restrict__ w,
                                                   const float* __restrict__ x, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float4v* wr = reinterpret_cast<const float4v*>(w + (size_t)row * cols);
  const float4v* xv = reinterpret_cast<const float4v*>(x);
  double acc = 0.0;
  for (int c = lane; c < (cols >> 2); c += 64) {
    const float4v a = wr[c], b = xv[c];
    acc += ((double)a[0] * b[0] + (double)a[1] * b[1]) + ((double)a[2] * b[2] + (double)a[3] * b[3]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  float v = (float)acc;
  if (MODE == 1) v = v / (1.0f + expf(-v));
  if (MODE == 2) v = 1.0f + v;
  if (lane == 0) y[row] = v;
}

// x += dt v, the product and the sum each rounded (no contraction)
__global__ void axpy_kernel(int n, float dt, const float* __restrict__ v, float* __restrict__ x) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = __fadd_rn(x[i], __fmul_rn(dt, v[i]));
}

// dst[i] = f32(src[i]); src_dtype 0 f32, 1 bf16, 2 f16
__global__ void to_f32_kernel(int src_dtype, const void* __restrict__ src, size_t n, float* __restrict__ dst) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v;
  if (src_dtype == 0)
    v = reinterpret_cast<const float*>(src)[i];
  else if (src_dtype == 1)
    v = __uint_as_float((unsigned)reinterpret_cast<const unsigned short*>(src)[i] << 16);
  else
    v = (float)reinterpret_cast<const f16*>(src)[i];
  dst[i] = v;
}

hipError_t launch_time_mods(int h, float t, const float* t_lin1, const float* t_lin2, const float* modulation,
                            const float* norm_out, float* work, float* mods, float* fs, hipStream_t s) {
  float* e = work;            // [256]
  float* hid = work + 256;    // [h]
  float* sv = hid + h;        // [h] = silu(temb)
  hipLaunchKernelGGL(temb_sin_kernel, dim3(1), dim3(128), 0, s, t, e);
  hipLaunchKernelGGL(gemv_kernel<1>, dim3((h + 3) / 4), dim3(256), 0, s, h, 256, t_lin1, e, hid);
  hipLaunchKernelGGL(gemv_kernel<1>, dim3((h + 3) / 4), dim3(256), 0, s, h, h, t_lin2, hid, sv);
  hipLaunchKernelGGL(gemv_kernel<0>, dim3((4 * h + 3) / 4), dim3(256), 0, s, 4 * h, h, modulation, sv, mods);
  hipLaunchKernelGGL(gemv_kernel<2>, dim3((h + 3) / 4), dim3(256), 0, s, h, h, norm_out, sv, fs);
  return hipGetLastError();
}

hipError_t launch_axpy(int n, float dt, const float* v, float* x, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(axpy_kernel, dim3((n + 255) / 256), dim3(256), 0, s, n, dt, v, x);
  return hipGetLastError();
}

hipError_t launch_to_f32(int src_dtype, const void* src, size_t n, float* dst, hipStream_t s) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(to_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src_dtype, src, n, dst);
  return hipGetLastError();
}

}  // namespace qi21
