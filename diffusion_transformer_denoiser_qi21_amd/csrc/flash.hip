// Flash attention of the denoiser step and prefill (head_dim 128).
//
// Computes, per head, softmax(q k^T / sqrt(128)) v with the online
// softmax, keys streamed from two sources: the per-layer prefix cache and
// the pass's own rows.  Query i may be limited to keys [0, vis[i]) (the
// prefill's block-causal mask, a non-decreasing leading run); a block walks
// only the key tiles its last live query sees.
//
// Everything is computed transposed so that one lane owns one query:
//   S^T = K Q^T      (A = K tile from LDS, B = Q fragments in registers)
//   O^T += V^T P^T   (A = V^T tile from LDS, B = P from the S^T registers)
// with v_mfma_f32_32x32x16_f16.  The S^T accumulator of a lane holds 32
// keys of its query, and those registers, converted to f16, are already
// the B operand of the P V product: P never goes through LDS.  The online
// softmax statistics (running max, partial row sum) and the O^T rescale
// are lane-local; the two lanes that share a query (l and l ^ 32) exchange
// their maxima once per key tile and their sums once at the end.
//
// Block: 4 waves x 32 queries; key tile 64.  K tile [64][128] and V^T tile
// [128][64] live in LDS, double-buffered (global -> registers -> LDS, next
// tile in flight during the current one's MFMAs).  V arrives transposed
// from HBM (the qkv GEMM epilogue writes V^T), so both tiles load with
// 16-byte coalesced reads.
#include "qi21_internal.h"

namespace qi21 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

namespace {
constexpr int BQ = 128;       // queries per block
constexpr int BKV = 64;       // keys per tile
constexpr int VT_LD = 17;     // V^T LDS row: 16 units of 8 bytes + 1 pad unit
constexpr float LOG2E = 1.4426950408889634f;
}  // namespace

template <bool VIS>
__global__ __launch_bounds__(256) void flash_kernel(FlashArgs a) {
  __shared__ u32x4 sk[2][BKV * 16];
  __shared__ u32x2 svt[2][128 * VT_LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hs = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.y;
  const int q0 = blockIdx.x * BQ;
  const int myq = q0 + wave * 32 + l32;
  const bool live = myq < a.nq;
  const int qrow = min(myq, a.nq - 1);
  const int ntot = a.n1 + a.n2;

  // Q fragments: dims 16c + 8*hs .. +8 of this lane's query
  half8 qf[8];
  {
    const f16* qp = a.q + (size_t)qrow * a.ldq + head * 128 + 8 * hs;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const half8*>(qp + 16 * c);
  }
  int lim = ntot, kmax = ntot;
  if (VIS) {
    lim = min(ntot, (int)a.vis[qrow]);
    kmax = min(ntot, (int)a.vis[min(q0 + BQ, a.nq) - 1]);
  }
  const int t1 = (min(a.n1, kmax) + BKV - 1) / BKV;
  const int t2 = kmax > a.n1 ? (min(a.n2, kmax - a.n1) + BKV - 1) / BKV : 0;
  const int T = t1 + t2;

  u32x4 rk[4], rv[4];
  auto load_tile = [&](int t) {
    const bool s1 = t < t1;
    const int j0 = (s1 ? t : t - t1) * BKV;
    const int ns = s1 ? a.n1 : a.n2;
    const f16* kb = s1 ? a.k1 : a.k2;
    const int ldk = s1 ? a.ldk1 : a.ldk2;
    const f16* vb = s1 ? a.vt1 : a.vt2;
    const int ldv = s1 ? a.ldvt1 : a.ldvt2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      const int key = q >> 4, c = q & 15;
      const int row = min(j0 + key, ns - 1);
      rk[i] = *reinterpret_cast<const u32x4*>(kb + (size_t)row * ldk + head * 128 + 8 * c);
      const int d = q >> 3, cv = q & 7;
      rv[i] = *reinterpret_cast<const u32x4*>(vb + (size_t)(head * 128 + d) * ldv + j0 + 8 * cv);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      const int key = q >> 4, c = q & 15;
      sk[buf][key * 16 + (c ^ (key & 15))] = rk[i];
      const int d = q >> 3, cv = q & 7;
      svt[buf][d * VT_LD + 2 * cv] = u32x2{rv[i][0], rv[i][1]};
      svt[buf][d * VT_LD + 2 * cv + 1] = u32x2{rv[i][2], rv[i][3]};
    }
  };

  floatx16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;
  float mrun = -INFINITY, lsum = 0.0f;
  const float c2 = LOG2E * 0.08838834764831845f;  // log2(e) / sqrt(128)

  if (T > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    if (t + 1 < T) load_tile(t + 1);

    // S^T = K Q^T : two 32-key sub-tiles
    floatx16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[st][e] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int key = st * 32 + l32;
        const u32x4 kv = sk[cur][key * 16 + ((2 * c + hs) ^ (key & 15))];
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, kv), qf[c], s[st], 0, 0, 0);
      }
    }

    // mask: keys past the source's end, or past vis[i]
    const bool s1 = t < t1;
    const int j0 = (s1 ? t : t - t1) * BKV;
    const int cnt = min(BKV, (s1 ? a.n1 : a.n2) - j0);
    const int gbase = (s1 ? 0 : a.n1) + j0;
    if (VIS || cnt < BKV) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = st * 32 + 8 * (e >> 2) + 4 * hs + (e & 3);
          if (kk >= cnt || gbase + kk >= lim) s[st][e] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[st][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrun, mx);
    const float msafe = mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = __builtin_amdgcn_exp2f((mrun - msafe) * c2);
    const float mc = msafe * c2;
    mrun = mnew;
    float ps = 0.0f;
    half8 pf[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][8 * u + j], c2, -mc));
          ps += p;
          pf[st][u][j] = (f16)p;
        }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d][e] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int unit = 8 * st + 4 * u + hs;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int row = (32 * d + l32) * VT_LD;
          const u32x2 lo = svt[cur][row + unit];
          const u32x2 hi = svt[cur][row + unit + 2];
          const u32x4 vv = u32x4{lo[0], lo[1], hi[0], hi[1]};
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, vv), pf[st][u], o[d], 0, 0, 0);
        }
      }

    if (t + 1 < T) store_tile(cur ^ 1);
    __syncthreads();
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.0f ? a.oscale / ltot : 0.0f;
  if (live) {
    f16* op = a.out + (size_t)myq * a.ldo + head * 128 + 4 * hs;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        half4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (f16)(o[d][4 * g + e] * inv);
        *reinterpret_cast<half4*>(op + 32 * d + 8 * g) = v;
      }
  }
}

hipError_t launch_flash(const FlashArgs& a, hipStream_t s) {
  dim3 grid((a.nq + BQ - 1) / BQ, a.heads);
  if (a.vis)
    hipLaunchKernelGGL(flash_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(flash_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qi21
