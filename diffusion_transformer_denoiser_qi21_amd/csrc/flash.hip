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
// Block: 4 waves x 32 queries; key tile 64.  The K tile [64][128] and the
// V^T tile [128][64] of each step are fetched by buffer loads that write
// straight into LDS (two stages: the next tile is in flight while the
// current one is multiplied); keys past a source's end read as zeros and
// are masked.  At most 256 registers per lane, so two blocks share a CU and
// one block's softmax overlaps the other's MFMAs.
//
// V^T rows hold their keys permuted inside each group of 16 (bits 2 and 3
// of the key index swapped; the qkv GEMM epilogue writes them so), which
// puts the 8 keys one lane contributes to a P V k-step in one contiguous
// 16-byte chunk: one conflict-free 16-byte LDS read per fragment.
//
// Softmax: exp2 with log2(e)/sqrt(128) folded into one FMA, the running
// maximum updated lazily -- the O^T rescale runs only when some query of
// the wave sees its maximum grow by more than 2^8 (a wave-uniform branch),
// so P = 2^(s - m) stays below 2^8 and exact in f16; row sums by v_dot2 on
// the f16 P that also feeds the P V product.
#include "qi21_internal.h"

namespace qi21 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

namespace {
constexpr int BQ = 128;   // queries per block
constexpr int BKV = 64;   // keys per tile
constexpr int TILE_H = BKV * 128;       // halves in the K tile (and in the V^T tile)
constexpr int STAGE_H = 2 * TILE_H;     // K tile then V^T tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float THR = 8.0f;             // lazy-rescale threshold, log2 units

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// K tile rows: 256 bytes = 16 chunks; chunk c of key row j at slot c ^ (j & 15).
// V^T tile rows: 128 bytes = 8 chunks; chunk c of dim row d at slot c ^ ((d >> 1) & 7).
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
}  // namespace

template <bool VIS>
__global__ __launch_bounds__(256, 2) void flash_kernel(FlashArgs a) {
  __shared__ __attribute__((aligned(16))) f16 sm[2 * STAGE_H];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = lane >> 5, l32 = lane & 31;
  // Blocks are dealt to the 8 XCDs round-robin (block b -> XCD b % 8).  All
  // query blocks of a head go to one XCD, so the head's K / V^T tiles are
  // fetched into that XCD's L2 once and shared by its query blocks.
  const int nqb = (a.nq + BQ - 1) / BQ;
  int head, qb;
  {
    const int b = blockIdx.x;
    if ((a.heads & 7) == 0) {
      const int li = b >> 3;
      head = (b & 7) + 8 * (li / nqb);
      qb = li % nqb;
    } else {
      head = b / nqb;
      qb = b % nqb;
    }
  }
  const int q0 = qb * BQ;
  const int myq = q0 + wave * 32 + l32;
  const bool live = myq < a.nq;
  const int qrow = min(myq, a.nq - 1);
  const int ntot = a.n1 + a.n2;

  // Q fragments (B operand of S^T = K Q^T): dims 16c + 8*hs .. +8 of this lane's query
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

  // buffer resources of the two sources (this head's columns); K rows past
  // the source's end fall outside the range and read as zeros
  __amdgpu_buffer_rsrc_t kr[2], vr[2];
  int ldk[2], ldv[2];
  {
    const f16* kb[2] = {a.k1, a.k2};
    const f16* vb[2] = {a.vt1, a.vt2};
    const int ns[2] = {a.n1, a.n2};
    ldk[0] = a.ldk1;
    ldk[1] = a.ldk2;
    ldv[0] = a.ldvt1;
    ldv[1] = a.ldvt2;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int n = max(ns[s], 1);
      kr[s] = __builtin_amdgcn_make_buffer_rsrc((void*)(kb[s] + head * 128), 0, (n - 1) * ldk[s] * 2 + 256,
                                                0x00020000);
      vr[s] = __builtin_amdgcn_make_buffer_rsrc((void*)(vb[s] + (size_t)head * 128 * ldv[s]), 0, 128 * ldv[s] * 2,
                                                0x00020000);
    }
  }
  // Load i (0..3) of wave w fills 16-byte LDS positions (4i + w) * 64 + lane
  // of the K tile (key p / 16, slot p % 16) and of the V^T tile (dim p / 8,
  // slot p % 8).  The key offset of a tile goes into the per-lane offset,
  // which the buffer range check covers, so keys past a source's end read
  // as zeros (V^T columns past the end are in range: the leading dimension
  // covers whole 64-key tiles).
  int lkey[4], lck[4], ldim[4], lcv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = (i * 4 + wave) * 64 + lane;
    lkey[i] = p >> 4;
    lck[i] = ((p & 15) ^ (lkey[i] & 15)) * 16;
    ldim[i] = p >> 3;
    lcv[i] = ((p & 7) ^ vswz(ldim[i])) * 16;
  }
  auto issue = [&](int t, int stage) {
    const bool s1 = t < t1;
    const int j0 = (s1 ? t : t - t1) * BKV;
    const int lk2 = (s1 ? ldk[0] : ldk[1]) * 2, lv2 = (s1 ? ldv[0] : ldv[1]) * 2;
    const __amdgpu_buffer_rsrc_t krs = s1 ? kr[0] : kr[1];
    const __amdgpu_buffer_rsrc_t vrs = s1 ? vr[0] : vr[1];
    const int sv = __builtin_amdgcn_readfirstlane(j0 * 2);
    f16* base = sm + stage * STAGE_H + wave * 64 * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, base + i * 4 * 64 * 8, 16, (j0 + lkey[i]) * lk2 + lck[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, base + TILE_H + i * 4 * 64 * 8, 16, ldim[i] * lv2 + lcv[i], sv, 0,
                                               0);
    }
  };

  floatx16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;
  float mused = -INFINITY, lsum = 0.0f;
  const float c2 = LOG2E * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const float thr_raw = THR / c2;
  const half2v ones = half2v{(f16)1.0f, (f16)1.0f};

  if (T > 0) issue(0, 0);
  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    // tile t resident; every wave is done with tile t - 1, whose stage
    // receives tile t + 1
    __builtin_amdgcn_s_waitcnt(0x7 << 4 | 0xF << 8);  // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (t + 1 < T) issue(t + 1, cur ^ 1);
    const f16* sk = sm + cur * STAGE_H;
    const f16* sv = sk + TILE_H;

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
        const half8 kv = *reinterpret_cast<const half8*>(sk + key * 128 + (((2 * c + hs) ^ (key & 15)) * 8));
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kv, qf[c], s[st], 0, 0, 0);
      }
    }

    // mask: keys past the source's end, or past vis[i] (tail tiles and the
    // prefill only; a wave-uniform branch)
    const bool s1 = t < t1;
    const int j0 = (s1 ? t : t - t1) * BKV;
    const int cnt = min(BKV, (s1 ? a.n1 : a.n2) - j0);
    const int gbase = (s1 ? 0 : a.n1) + j0;
    if (__builtin_amdgcn_readfirstlane((int)(VIS || cnt < BKV))) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = st * 32 + 8 * (e >> 2) + 4 * hs + (e & 3);
          if (kk >= cnt || gbase + kk >= lim) s[st][e] = -INFINITY;
        }
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int e = 2; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s[0][e], s[0][e + 1]));
#pragma unroll
    for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s[1][e], s[1][e + 1]));
    mx = pair_max(mx);
    if (__any(mx > mused + thr_raw)) {  // wave-uniform: rescale O^T and the sum
      const float mnew = fmaxf(mused, mx);
      const float alpha = __builtin_amdgcn_exp2f((mused - mnew) * c2);
      mused = mnew;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
    }
    const float mc = mused == -INFINITY ? 0.0f : mused * c2;
    // P in f16, packed pairwise straight into the B operand registers
    half8 pf[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][8 * u + 2 * j], c2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][8 * u + 2 * j + 1], c2, -mc));
          const half2v ph = half2v{(f16)p0, (f16)p1};
          lsum = __builtin_amdgcn_fdot2(ph, ones, lsum, false);
          pk[j] = __builtin_bit_cast(unsigned int, ph);
        }
        pf[st][u] = __builtin_bit_cast(half8, pk);
      }

    // O^T += V^T P^T : the lane's 8 keys of k-step (st, u) are the 16-byte
    // chunk 4st + 2u + hs of its dim row
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int row = 32 * d + l32;
          const half8 vv = *reinterpret_cast<const half8*>(sv + row * 64 + (((4 * st + 2 * u + hs) ^ vswz(row)) * 8));
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv, pf[st][u], o[d], 0, 0, 0);
        }
      }
  }

  const float ltot = pair_sum(lsum);
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
  dim3 grid(((a.nq + BQ - 1) / BQ) * a.heads);
  if (a.vis)
    hipLaunchKernelGGL(flash_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(flash_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qi21
