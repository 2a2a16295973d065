// MFMA GEMM of the denoiser's four projection sites (qkv, O, gate/up, down).
//
// C[M][N] = A[M][K] * W[N][K]^T with f16 operands and f32 accumulation,
// the contraction done by v_mfma_f32_32x32x16_f16 (gfx950).  Both operands
// are K-contiguous in HBM (activations row-major, weight planes [out][in]),
// which is exactly the layout the MFMA A and B fragments want, so no
// operand is ever transposed.
//
// Block tile BM x BN x 64, 256 threads = 4 waves in a 2 x 2 arrangement,
// each wave owning a (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA tiles.  The
// A and B tiles go global -> registers -> LDS, double-buffered so the next
// k-tile's global loads are in flight while the current one is multiplied;
// one barrier per k-tile.  LDS rows are 64 halves (8 chunks of 16 bytes);
// chunk c of row r is stored at slot c ^ (r & 7), so the 16-byte fragment
// reads of 8 consecutive rows hit 8 different bank groups.
//
// Epilogues (fused, from the registers): f16 store, f32 store, the SwiGLU
// of the interleaved gate/up plane, and the qkv split that writes the v
// columns transposed (V^T, the layout the attention kernel streams).
// Range-guard factors are powers of two folded into oscale / inscale.
#include "qi21_internal.h"

namespace qi21 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ (r & 7)); }

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + __expf(-v)); }

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  constexpr int BK = 64;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int AL = BM * 8 / 256;  // 16-byte chunks per thread, A tile
  constexpr int BL = BN * 8 / 256;  // 16-byte chunks per thread, B tile
  extern __shared__ u32x4 smem[];   // [2][(BM + BN) * 8]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = a.N / BN;
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  // Blocks are dealt to the 8 XCDs round-robin (block b -> XCD b % 8); remap
  // so that each XCD works on a contiguous run of tiles, which share their
  // A row panel in that XCD's L2.
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tm = bid / tiles_n, tn = bid - tm * tiles_n;
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
    aslot[i] = swz(r, c);
  }
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    int q = tid + 256 * i, r = q >> 3, c = q & 7;
    bg[i] = reinterpret_cast<const u32x4*>(a.W + (size_t)(n0 + r) * K + c * 8);
    bslot[i] = BM * 8 + swz(r, c);
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
  for (int i = 0; i < AL; ++i) smem[aslot[i]] = ra[i];
#pragma unroll
  for (int i = 0; i < BL; ++i) smem[bslot[i]] = rb[i];
  __syncthreads();

  const int KT = K / BK;
  const int arow0 = wm * WM + (lane & 31), brow0 = wn * WN + (lane & 31);
  const int hsel = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const u32x4* s = smem + cur * (BM + BN) * 8;
    if (kt + 1 < KT) {
      const int off = (kt + 1) * (BK / 8);  // in 16-byte units along K
#pragma unroll
      for (int i = 0; i < AL; ++i) ra[i] = ag[i][off];
#pragma unroll
      for (int i = 0; i < BL; ++i) rb[i] = bg[i][off];
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + hsel;
      half8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        u32x4 v = s[swz(arow0 + i * 32, c)];
        af[i] = __builtin_bit_cast(half8, v);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        u32x4 v = s[BM * 8 + swz(brow0 + j * 32, c)];
        bf[j] = __builtin_bit_cast(half8, v);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      u32x4* d = smem + (cur ^ 1) * (BM + BN) * 8;
#pragma unroll
      for (int i = 0; i < AL; ++i) d[aslot[i]] = ra[i];
#pragma unroll
      for (int i = 0; i < BL; ++i) d[bslot[i]] = rb[i];
    }
    __syncthreads();
  }

  // ── epilogue ── lane (col l%32) holds rows 8g + 4*(l/32) + e of each tile
  const int rbase = m0 + wm * WM + 4 * hsel;
  const int cbase = n0 + wn * WN + (lane & 31);
  if constexpr (EPI == EPI_F32 || EPI == EPI_F16) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
          const int col = cbase + j * 32;
          if (row < a.M) {
            const float v = acc[i][j][e] * a.oscale;
            if constexpr (EPI == EPI_F32)
              reinterpret_cast<float*>(a.out)[(size_t)row * a.ldo + col] = v;
            else
              reinterpret_cast<f16*>(a.out)[(size_t)row * a.ldo + col] = (f16)v;
          }
        }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // tiles (2p, 2p+1) of a wave hold matching gate / up columns
    const int hc0 = (n0 + wn * WN) / 2 + (lane & 31);
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
            reinterpret_cast<f16*>(a.out)[(size_t)row * a.ldo + hc0 + p * 32] =
                (f16)(silu_f(g) * u * a.oscale);
          }
        }
  } else {  // EPI_QKV
    const int two_h = (a.N / 3) * 2;
    if (n0 < two_h) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = rbase + i * 32 + 8 * (e >> 2) + (e & 3);
            if (row < a.M)
              reinterpret_cast<f16*>(a.out)[(size_t)row * a.ldo + cbase + j * 32] =
                  (f16)(acc[i][j][e] * a.oscale);
          }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          f16* dst = a.out2 + (size_t)(cbase + j * 32 - two_h) * a.ld2;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int row = rbase + i * 32 + 8 * g;
            half4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (f16)(acc[i][j][4 * g + e] * a.oscale);
            if (row + 3 < a.M) {
              *reinterpret_cast<half4*>(dst + row) = v;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (row + e < a.M) dst[row + e] = v[e];
            }
          }
        }
    }
  }
}

template <int BM, int BN, int EPI>
static hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
  constexpr size_t lds = 2 * (BM + BN) * 8 * sizeof(u32x4);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<BM, BN, EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int blocks = ((a.M + BM - 1) / BM) * (a.N / BN);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI>), dim3(blocks), dim3(256), lds, s, a);
  return hipGetLastError();
}

int gemm_pick_tile(int M, int N, int K) {
  (void)K;
  if (N % 256 == 0 && M >= 2048) return 0;
  return 1;
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& a, int tile, hipStream_t s) {
  if (tile == 0) return launch_tile<256, 256, EPI>(a, s);
  return launch_tile<128, 128, EPI>(a, s);
}

hipError_t launch_gemm(int epi, const GemmArgs& a, int tile, hipStream_t s) {
  if (tile < 0) tile = gemm_pick_tile(a.M, a.N, a.K);
  if (tile == 0 && a.N % 256 != 0) tile = 1;
  switch (epi) {
    case EPI_F16: return launch_epi<EPI_F16>(a, tile, s);
    case EPI_F32: return launch_epi<EPI_F32>(a, tile, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, tile, s);
    case EPI_QKV: return launch_epi<EPI_QKV>(a, tile, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qi21
