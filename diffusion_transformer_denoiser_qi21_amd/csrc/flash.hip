// Flash attention of the denoiser step and prefill (head_dim 128).
//
// Computes, per head, softmax(q k^T / sqrt(128)) v with the online
// softmax, from q given in log2 units (q log2(e) / sqrt(128), the scale the
// q producers apply through their norm weights), keys streamed from two sources: the per-layer prefix cache and
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
// Block: NW waves x 32 queries (NW = 8, or 4 for grids too small to fill
// the chip; grids of at most one round of 128-query blocks use the
// key-split form below), key tile 64.  The K tile [64][128] and the V^T tile [128][64]
// of each step are fetched by buffer loads that write straight into LDS,
// through a ring of NST stages (4 with 8 waves: 128 KB, one block per CU;
// 2 with 4 waves: 64 KB, two blocks per CU), so a tile's loads have NST - 1
// steps to land; keys past a source's end read as zeros and are masked.
// All 16 K fragments of a step are read from LDS before its first MFMA and
// the V^T fragments before the softmax, so LDS latency is paid once per
// phase.  Either way each SIMD holds two waves, whose matrix and vector
// work interleave.
//
// V^T rows hold their keys permuted inside each group of 16 (bits 2 and 3
// of the key index swapped; the qkv GEMM epilogue writes them so), which
// puts the 8 keys one lane contributes to a P V k-step in one contiguous
// 16-byte chunk: one conflict-free 16-byte LDS read per fragment.
//
// Softmax: S^T is already the base-2 exponent, and the S^T accumulators
// are seeded with minus the running maximum m, so P = exp2 of them with no
// further arithmetic.  m is updated lazily -- the rescale of O^T and of the
// sum, and the shift of the tile's scores, run only when some query of the
// wave sees its maximum grow by more than 2^8 (a wave-uniform branch), so
// P = 2^(s - m) stays below 2^8 and exact in f16; row sums by v_dot2 on the
// f16 P that also feeds the P V product.
#include "qi21_internal.h"

namespace qi21 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

namespace {
constexpr int BKV = 64;   // keys per tile
constexpr int TILE_B = BKV * 128 * 2;   // bytes of a K tile (and of a V^T tile)
constexpr int STAGE_B = 2 * TILE_B;     // K tile then V^T tile
constexpr float THR = 8.0f;             // lazy-rescale threshold, log2 units

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// K tile rows: 256 bytes = 16 chunks; chunk c of key row j at slot c ^ (j & 15).
// V^T tile rows: 128 bytes = 8 chunks; chunk c of dim row d at slot c ^ ((d >> 1) & 7).
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

// Maximum of a lane's 32 scores (two 16-element sub-tiles): one chain of
// 3-input maxima per sub-tile, 16 instructions plus one to join them (the
// compiler's own tree takes 24).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float lane_max(const floatx16 (&s)[2]) {
  float m[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    m[st] = max3f(s[st][0], s[st][1], s[st][2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) m[st] = max3f(m[st], s[st][e], s[st][e + 1]);
    m[st] = fmaxf(m[st], s[st][15]);
  }
  return fmaxf(m[0], m[1]);
}
// The lazy rescale of one lane: mx is the maximum of the tile's S^T - base.
// The running maximum moves to mnew (the larger of the old one and this
// tile's); O^T and the sum are scaled by 2^(mused - mnew) (0 while mused =
// -inf), the tile's scores are shifted to S^T - mnew, and nb / thr follow.
// A lane that has seen no key yet (mnew = -inf) keeps base 0, thr = -inf and
// its -inf scores.
__device__ __forceinline__ void rebase(floatx16 (&s)[2], float mx, float& mused, float& base, float& thr,
                                       floatx16& nb, float& lsum, floatx16 (&o)[4]) {
  const float mnew = fmaxf(mused, mx + base);
  const float alpha = mused == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mused - mnew);
  const float shift = mnew == -INFINITY ? 0.0f : mnew - base;
  mused = mnew;
  base = mnew == -INFINITY ? 0.0f : mnew;
  thr = mnew == -INFINITY ? -INFINITY : THR;
#pragma unroll
  for (int e = 0; e < 16; ++e) nb[e] = -base;
  lsum *= alpha;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[st][e] -= shift;
}
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
}  // namespace

template <bool VIS, int NW, int NST>
__global__ __launch_bounds__(NW * 64, 8 / NW) void flash_kernel(FlashArgs a0, FlashArgs a1, int nb0) {
  // blocks [0, nb0) work on segment a0, the rest on a1 (one launch for the
  // rows of two programs, each attending to its own keys)
  const bool seg1 = (int)blockIdx.x >= nb0;
  const FlashArgs& a = seg1 ? a1 : a0;
  const int bid = (int)blockIdx.x - (seg1 ? nb0 : 0);
  constexpr int BQ = NW * 32;          // queries per block
  constexpr int NLD = 16 / NW;         // 16-byte loads per lane per K (and per V^T) tile
  extern __shared__ __attribute__((aligned(16))) char smb[];  // NST stages of [K tile | V^T tile]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // With 8 waves the two waves of a SIMD (w and w + 4) take its issue slots
  // in a fixed order, waves 0-3 first: the lower wave runs each step's
  // phases ahead of its partner, so one's matrix phase meets the other's
  // vector phase instead of both contending for the same unit.
  if (NW == 8 && wave < 4) __builtin_amdgcn_s_setprio(1);
  const int hs = lane >> 5, l32 = lane & 31;
  // Blocks are dealt to the 8 XCDs round-robin (block b -> XCD b % 8).  All
  // query blocks of a head go to one XCD, so the head's K / V^T tiles are
  // fetched into that XCD's L2 once and shared by its query blocks.
  const int nqb = (a.nq + BQ - 1) / BQ;
  int head, qb;
  {
    const int b = bid;
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
  // n1 / n2 as opaque scalars: the loop's mask reads them from registers.
  // A reload of the kernel argument there would leave a scalar load in
  // flight at the loop's first LDS reads, and the LDS wait before the
  // first MFMA would then have to drain every read, not just the first.
  int n1 = a.n1, n2 = a.n2;
  asm volatile("" : "+s"(n1), "+s"(n2));
  const int ntot = n1 + n2;

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
  const int t1 = (min(n1, kmax) + BKV - 1) / BKV;
  const int t2 = kmax > n1 ? (min(n2, kmax - n1) + BKV - 1) / BKV : 0;
  const int T = t1 + t2;

  // buffer resources of the two sources (this head's columns); K rows past
  // the source's end fall outside the range and read as zeros
  __amdgpu_buffer_rsrc_t kr[2], vr[2];
  int lk2[2], lv2[2];
  {
    const f16* kb[2] = {a.k1, a.k2};
    const f16* vb[2] = {a.vt1, a.vt2};
    const int ns[2] = {n1, n2};
    const int ldk[2] = {a.ldk1, a.ldk2}, ldv[2] = {a.ldvt1, a.ldvt2};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int n = max(ns[s], 1);
      lk2[s] = ldk[s] * 2;
      lv2[s] = ldv[s] * 2;
      kr[s] = __builtin_amdgcn_make_buffer_rsrc((void*)(kb[s] + head * 128), 0, (n - 1) * ldk[s] * 2 + 256,
                                                0x00020000);
      vr[s] = __builtin_amdgcn_make_buffer_rsrc((void*)(vb[s] + (size_t)head * 128 * ldv[s]), 0, 128 * ldv[s] * 2,
                                                0x00020000);
    }
  }
  // Load i (0..NLD-1) of wave w fills 16-byte LDS positions p = (NW i + w)
  // * 64 + lane of the K tile (key p / 16 = 4 NW i + 4w + lane / 16, slot
  // p % 16) and of the V^T tile (dim p / 8 = 8 NW i + 8w + lane / 8, slot
  // p % 8); a lane's swizzled chunk is the same for all of them.  The key offset of a tile goes
  // into the per-lane offset, which the buffer range check covers, so keys
  // past a source's end read as zeros (V^T columns past the end are in
  // range: the leading dimension covers whole 64-key tiles, and the tile's
  // first column goes into the scalar offset).
  const int lkey0 = 4 * wave + (lane >> 4);
  const int lck = ((lane & 15) ^ (lkey0 & 15)) * 16;
  const int ldim0 = 8 * wave + (lane >> 3);
  const int lcv = ((lane & 7) ^ vswz(ldim0)) * 16;
  // tile t -> stage t % NST
  auto issue = [&](int t) {
    const bool s1 = t < t1;
    const int j0 = (s1 ? t : t - t1) * BKV;
    const int kl2 = s1 ? lk2[0] : lk2[1], vl2 = s1 ? lv2[0] : lv2[1];
    const __amdgpu_buffer_rsrc_t krs = s1 ? kr[0] : kr[1];
    const __amdgpu_buffer_rsrc_t vrs = s1 ? vr[0] : vr[1];
    const int ko = (j0 + lkey0) * kl2 + lck;
    const int vo = ldim0 * vl2 + lcv;
    const int sv = __builtin_amdgcn_readfirstlane(j0 * 2);
    char* base = smb + (t % NST) * STAGE_B + wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, base + i * NW * 64 * 16, 16, ko + i * 4 * NW * kl2, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, base + TILE_B + i * NW * 64 * 16, 16, vo + i * 8 * NW * vl2, sv,
                                               0, 0);
    }
  };
  // Byte offsets of this lane's LDS fragments inside a tile.  K: key l32
  // (sub-tile 1 is 32 rows = 8192 bytes further), chunk 2c + hs.  V^T: dim
  // row l32 (dim block d is 32 rows = 4096 bytes further), chunk 4st + 2u +
  // hs = 2su + hs.  The swizzles depend on l32 only.
  int kofs[8], vofs[4];
#pragma unroll
  for (int c = 0; c < 8; ++c) kofs[c] = l32 * 256 + (((2 * c + hs) ^ (l32 & 15)) * 16);
#pragma unroll
  for (int su = 0; su < 4; ++su) vofs[su] = l32 * 128 + (((2 * su + hs) ^ vswz(l32)) * 16);

  floatx16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;
  // Q arrives in log2 units (q log2(e) / sqrt(128)), so S^T is the base-2
  // exponent itself.  The S^T accumulators are seeded with nb = -base, where
  // base is the running maximum mused (0 while that is -inf): they leave
  // the MFMAs as S^T - mused and P = exp2 of them.  thr is the lazy-rescale
  // threshold on that difference (-inf until a lane has seen a key).
  float mused = -INFINITY, lsum = 0.0f, base = 0.0f, thr = -INFINITY;
  floatx16 nb;
#pragma unroll
  for (int e = 0; e < 16; ++e) nb[e] = 0.0f;
  const half2v ones = half2v{(f16)1.0f, (f16)1.0f};

#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
    if (t < T) issue(t);
  for (int t = 0; t < T; ++t) {
    // tile t resident (the loads of up to NST - 2 later tiles may still be
    // in flight, 2 NLD per tile); after the barrier every wave is done with
    // tile t - 1, whose stage receives tile t + NST - 1
    if (NST == 4 && t + 2 < T)
      __builtin_amdgcn_s_waitcnt(wait_imm(4 * NLD, 15));
    else if (NST >= 3 && t + 1 < T)
      __builtin_amdgcn_s_waitcnt(wait_imm(2 * NLD, 15));
    else
      __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
    __builtin_amdgcn_s_barrier();
    if (t + NST - 1 < T) issue(t + NST - 1);
    const char* sk = smb + (t % NST) * STAGE_B;
    const char* sv = sk + TILE_B;

    // S^T = K Q^T : two 32-key sub-tiles
    // all 16 K fragments are read before the first MFMA, so one LDS
    // latency is paid per tile instead of one per pair of MFMAs
    half8 kv[16];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int st = 0; st < 2; ++st) kv[2 * c + st] = *reinterpret_cast<const half8*>(sk + kofs[c] + st * 8192);
    floatx16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kv[st], qf[0], nb, 0, 0, 0);
#pragma unroll
    for (int c = 1; c < 8; ++c)
#pragma unroll
      for (int st = 0; st < 2; ++st) s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kv[2 * c + st], qf[c], s[st], 0, 0, 0);
    // the V^T fragments do not depend on P: their reads are issued now and
    // land while the softmax runs
    half8 vv[16];
#pragma unroll
    for (int su = 0; su < 4; ++su)
#pragma unroll
      for (int d = 0; d < 4; ++d) vv[4 * su + d] = *reinterpret_cast<const half8*>(sv + vofs[su] + d * 4096);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_barrier(0);

    // mask: keys past the source's end, or past vis[i] (tail tiles and the
    // prefill only; a wave-uniform branch).  Element e of sub-tile st is key
    // st*32 + 8(e/4) + 4hs + e%4 of the tile: its constant part is compared
    // against one per-lane bound.
    const bool s1 = t < t1;
    const int j0 = (s1 ? t : t - t1) * BKV;
    const int cnt = min(BKV, (s1 ? n1 : n2) - j0);
    const int gbase = (s1 ? 0 : n1) + j0;
    if (__builtin_amdgcn_readfirstlane((int)(VIS || cnt < BKV))) {
      const int bound = min(cnt, lim - gbase) - 4 * hs;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (st * 32 + 8 * (e >> 2) + (e & 3) >= bound) s[st][e] = -INFINITY;
    }
    const float mx = pair_max(lane_max(s));  // of S^T - base
    if (__any(mx > thr)) {  // wave-uniform: move the reference maximum
      rebase(s, mx, mused, base, thr, nb, lsum, o);
    }
    // P in f16, packed pairwise straight into the B operand registers
    half8 pf[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(s[st][8 * u + 2 * j]);
          const float p1 = __builtin_amdgcn_exp2f(s[st][8 * u + 2 * j + 1]);
          const half2v ph = half2v{(f16)p0, (f16)p1};
          lsum = __builtin_amdgcn_fdot2(ph, ones, lsum, false);
          pk[j] = __builtin_bit_cast(unsigned int, ph);
        }
        pf[st][u] = __builtin_bit_cast(half8, pk);
      }

    // O^T += V^T P^T : the lane's 8 keys of k-step (st, u) are the 16-byte
    // chunk 4st + 2u + hs of its dim row
#pragma unroll
    for (int su = 0; su < 4; ++su)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv[4 * su + d], pf[su >> 1][su & 1], o[d], 0, 0, 0);
  }

  const float ltot = pair_sum(lsum);
  const float inv = ltot > 0.0f ? a.oscale / ltot : 0.0f;
  // Lane l holds dims 32 d + 8 g + 4 hs .. + 3 of its query, lane l ^ 32
  // the other 4 of each 8; one v_permlane32_swap per register of a pair of
  // g gives lane hs the 8 dims of g = 2 k + hs: one 16-byte store each.
  f16* op = a.out + (size_t)myq * a.ldo + head * 128;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x2 x[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        half4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (f16)(o[d][4 * (2 * k + u) + e] * inv);
        x[u] = __builtin_bit_cast(u32x2, v);
      }
      const auto s0 = __builtin_amdgcn_permlane32_swap(x[0][0], x[1][0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x[0][1], x[1][1], false, false);
      if (live) *reinterpret_cast<u32x4*>(op + 32 * d + 8 * (2 * k + hs)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
}

// The key-split form for grids too small to give each SIMD two waves
// (1024 queries x 32 heads: 1024 waves of 32 queries).  A block of 8 waves
// takes 128 queries: waves w and w + 4 own the same 32 queries, wave group
// g = w / 4 the key tiles t = 2s + g of step s.  Each step the block's 8
// waves fetch the step's two tiles (one per group) into a 4-stage ring, one
// step ahead.  At the end group 1 hands its unnormalised output, running
// maximum and partial sums to group 0 through LDS, and group 0 merges them
// (both rescaled to the larger maximum) and stores the result.
template <bool VIS>
__global__ __launch_bounds__(512, 1) void flash_split_kernel(FlashArgs a0, FlashArgs a1, int nb0) {
  // blocks [0, nb0) work on segment a0, the rest on a1 (one launch for the
  // rows of two programs, each attending to its own keys)
  const bool seg1 = (int)blockIdx.x >= nb0;
  const FlashArgs& a = seg1 ? a1 : a0;
  const int bid = (int)blockIdx.x - (seg1 ? nb0 : 0);
  constexpr int NW = 8, NST = 4;
  constexpr int BQ = 128;       // queries per block
  constexpr int NLD = 16 / NW;  // 16-byte loads per lane per K (and per V^T) tile
  extern __shared__ __attribute__((aligned(16))) char smb[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // group 0 first in the issue order (as in flash_kernel)
  if (wave < 4) __builtin_amdgcn_s_setprio(1);
  const int grp = wave >> 2, qw = wave & 3;
  const int hs = lane >> 5, l32 = lane & 31;
  const int nqb = (a.nq + BQ - 1) / BQ;
  int head, qb;
  {
    const int b = bid;
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
  const int myq = q0 + qw * 32 + l32;
  const bool live = myq < a.nq;
  const int qrow = min(myq, a.nq - 1);
  // n1 / n2 as opaque scalars: the loop's mask reads them from registers.
  // A reload of the kernel argument there would leave a scalar load in
  // flight at the loop's first LDS reads, and the LDS wait before the
  // first MFMA would then have to drain every read, not just the first.
  int n1 = a.n1, n2 = a.n2;
  asm volatile("" : "+s"(n1), "+s"(n2));
  const int ntot = n1 + n2;

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
  const int t1 = (min(n1, kmax) + BKV - 1) / BKV;
  const int t2 = kmax > n1 ? (min(n2, kmax - n1) + BKV - 1) / BKV : 0;
  const int T = t1 + t2;
  const int S = (T + 1) / 2;  // steps of two tiles

  __amdgpu_buffer_rsrc_t kr[2], vr[2];
  int lk2[2], lv2[2];
  {
    const f16* kb[2] = {a.k1, a.k2};
    const f16* vb[2] = {a.vt1, a.vt2};
    const int ns[2] = {n1, n2};
    const int ldk[2] = {a.ldk1, a.ldk2}, ldv[2] = {a.ldvt1, a.ldvt2};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int n = max(ns[s], 1);
      lk2[s] = ldk[s] * 2;
      lv2[s] = ldv[s] * 2;
      kr[s] = __builtin_amdgcn_make_buffer_rsrc((void*)(kb[s] + head * 128), 0, (n - 1) * ldk[s] * 2 + 256,
                                                0x00020000);
      vr[s] = __builtin_amdgcn_make_buffer_rsrc((void*)(vb[s] + (size_t)head * 128 * ldv[s]), 0, 128 * ldv[s] * 2,
                                                0x00020000);
    }
  }
  // tile t into stage t % NST by all 8 waves, as in flash_kernel with NW = 8
  const int lkey0 = 4 * wave + (lane >> 4);
  const int lck = ((lane & 15) ^ (lkey0 & 15)) * 16;
  const int ldim0 = 8 * wave + (lane >> 3);
  const int lcv = ((lane & 7) ^ vswz(ldim0)) * 16;
  auto issue = [&](int t) {
    const bool s1 = t < t1;
    const int j0 = (s1 ? t : t - t1) * BKV;
    const int kl2 = s1 ? lk2[0] : lk2[1], vl2 = s1 ? lv2[0] : lv2[1];
    const __amdgpu_buffer_rsrc_t krs = s1 ? kr[0] : kr[1];
    const __amdgpu_buffer_rsrc_t vrs = s1 ? vr[0] : vr[1];
    const int ko = (j0 + lkey0) * kl2 + lck;
    const int vo = ldim0 * vl2 + lcv;
    const int sv = __builtin_amdgcn_readfirstlane(j0 * 2);
    char* base = smb + (t % NST) * STAGE_B + wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, base + i * NW * 64 * 16, 16, ko + i * 4 * NW * kl2, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, base + TILE_B + i * NW * 64 * 16, 16, vo + i * 8 * NW * vl2, sv,
                                               0, 0);
    }
  };
  int kofs[8], vofs[4];
#pragma unroll
  for (int c = 0; c < 8; ++c) kofs[c] = l32 * 256 + (((2 * c + hs) ^ (l32 & 15)) * 16);
#pragma unroll
  for (int su = 0; su < 4; ++su) vofs[su] = l32 * 128 + (((2 * su + hs) ^ vswz(l32)) * 16);

  floatx16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.0f;
  // scores in log2 units, seeded with nb = -base as in flash_kernel
  float mused = -INFINITY, lsum = 0.0f, base = 0.0f, thr = -INFINITY;
  floatx16 nb;
#pragma unroll
  for (int e = 0; e < 16; ++e) nb[e] = 0.0f;
  const half2v ones = half2v{(f16)1.0f, (f16)1.0f};

  // step 0's tiles
  if (0 < T) issue(0);
  if (1 < T) issue(1);
  for (int s = 0; s < S; ++s) {
    // this step's two tiles have landed; after the barrier every wave is
    // done with step s - 1, whose stages receive step s + 1
    __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
    __builtin_amdgcn_s_barrier();
    if (2 * s + 2 < T) issue(2 * s + 2);
    if (2 * s + 3 < T) issue(2 * s + 3);
    const int t = 2 * s + grp;
    if (t < T) {  // (wave-uniform; a group without a tile in the last step only keeps the barriers)
      const char* sk = smb + (t % NST) * STAGE_B;
      const char* sv = sk + TILE_B;
      half8 kv[16];
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int st = 0; st < 2; ++st) kv[2 * c + st] = *reinterpret_cast<const half8*>(sk + kofs[c] + st * 8192);
      floatx16 sc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) sc[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kv[st], qf[0], nb, 0, 0, 0);
#pragma unroll
      for (int c = 1; c < 8; ++c)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          sc[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kv[2 * c + st], qf[c], sc[st], 0, 0, 0);
      half8 vv[16];
#pragma unroll
      for (int su = 0; su < 4; ++su)
#pragma unroll
        for (int d = 0; d < 4; ++d) vv[4 * su + d] = *reinterpret_cast<const half8*>(sv + vofs[su] + d * 4096);
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      __builtin_amdgcn_sched_barrier(0);
      const bool s1 = t < t1;
      const int j0 = (s1 ? t : t - t1) * BKV;
      const int cnt = min(BKV, (s1 ? n1 : n2) - j0);
      const int gbase = (s1 ? 0 : n1) + j0;
      if (__builtin_amdgcn_readfirstlane((int)(VIS || cnt < BKV))) {
        const int bound = min(cnt, lim - gbase) - 4 * hs;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (st * 32 + 8 * (e >> 2) + (e & 3) >= bound) sc[st][e] = -INFINITY;
      }
      const float mx = pair_max(lane_max(sc));
      // (a lane whose keys so far were all masked -- group 1 starts at tile
      // 1, past what an early prefix query sees -- still has mused = -inf
      // and nothing accumulated; rebase keeps it so)
      if (__any(mx > thr)) rebase(sc, mx, mused, base, thr, nb, lsum, o);
      half8 pf[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p0 = __builtin_amdgcn_exp2f(sc[st][8 * u + 2 * j]);
            const float p1 = __builtin_amdgcn_exp2f(sc[st][8 * u + 2 * j + 1]);
            const half2v ph = half2v{(f16)p0, (f16)p1};
            lsum = __builtin_amdgcn_fdot2(ph, ones, lsum, false);
            pk[j] = __builtin_bit_cast(unsigned int, ph);
          }
          pf[st][u] = __builtin_bit_cast(half8, pk);
        }
#pragma unroll
      for (int su = 0; su < 4; ++su)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv[4 * su + d], pf[su >> 1][su & 1], o[d], 0, 0, 0);
    }
  }
  // merge: group 1's (o, mused, lsum) per lane through LDS (the ring is free
  // once every wave is past this barrier)
  __builtin_amdgcn_s_waitcnt(wait_imm(0, 15));
  __syncthreads();
  float* xo = reinterpret_cast<float*>(smb) + (size_t)(qw * 64 + lane) * 66;  // [4 waves][64 lanes][64 + 2]
  if (grp == 1) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) xo[d * 16 + e] = o[d][e];
    xo[64] = mused;
    xo[65] = lsum;
  }
  __syncthreads();
  if (grp == 0) {
    const float m1 = xo[64], l1 = xo[65];
    const float m = fmaxf(mused, m1);
    const float a0 = mused == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mused - m);
    const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
    const float ltot = pair_sum(lsum * a0 + l1 * a1);
    const float inv = ltot > 0.0f ? a.oscale / ltot : 0.0f;
    // 16-byte stores of 8 dims per lane, as in flash_kernel (group 0 is
    // whole waves, so every lane takes part in the swaps)
    f16* op = a.out + (size_t)myq * a.ldo + head * 128;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        u32x2 x[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int g = 2 * k + u;
          half4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = (f16)((o[d][4 * g + e] * a0 + xo[d * 16 + 4 * g + e] * a1) * inv);
          x[u] = __builtin_bit_cast(u32x2, v);
        }
        const auto s0 = __builtin_amdgcn_permlane32_swap(x[0][0], x[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x[0][1], x[1][1], false, false);
        if (live) *reinterpret_cast<u32x4*>(op + 32 * d + 8 * (2 * k + hs)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
      }
  }
}

namespace {
// Blocks of `bq` queries over the heads of one segment.
long seg_blocks(const FlashArgs& a, int bq) { return (long)((a.nq + bq - 1) / bq) * a.heads; }

template <int NW, int NST>
hipError_t launch_shape(const FlashArgs& a0, const FlashArgs& a1, int nseg, hipStream_t s) {
  constexpr size_t lds = (size_t)NST * STAGE_B;
  static bool attr = false;
  if (!attr) {
    for (const void* f : {reinterpret_cast<const void*>(&flash_kernel<true, NW, NST>),
                          reinterpret_cast<const void*>(&flash_kernel<false, NW, NST>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    attr = true;
  }
  const int nb0 = (int)seg_blocks(a0, NW * 32);
  dim3 grid(nb0 + (nseg > 1 ? (int)seg_blocks(a1, NW * 32) : 0));
  if (a0.vis)
    hipLaunchKernelGGL((flash_kernel<true, NW, NST>), grid, dim3(NW * 64), lds, s, a0, a1, nb0);
  else
    hipLaunchKernelGGL((flash_kernel<false, NW, NST>), grid, dim3(NW * 64), lds, s, a0, a1, nb0);
  return hipGetLastError();
}
hipError_t launch_split(const FlashArgs& a0, const FlashArgs& a1, int nseg, hipStream_t s) {
  constexpr size_t lds = (size_t)4 * STAGE_B;
  static bool attr = false;
  if (!attr) {
    for (const void* f : {reinterpret_cast<const void*>(&flash_split_kernel<true>),
                          reinterpret_cast<const void*>(&flash_split_kernel<false>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    attr = true;
  }
  const int nb0 = (int)seg_blocks(a0, 128);
  dim3 grid(nb0 + (nseg > 1 ? (int)seg_blocks(a1, 128) : 0));
  if (a0.vis)
    hipLaunchKernelGGL((flash_split_kernel<true>), grid, dim3(512), lds, s, a0, a1, nb0);
  else
    hipLaunchKernelGGL((flash_split_kernel<false>), grid, dim3(512), lds, s, a0, a1, nb0);
  return hipGetLastError();
}

// One launch over one or two segments (both with or both without vis).
hipError_t launch_segs(const FlashArgs& a0, const FlashArgs& a1, int nseg, hipStream_t s) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
  }
  const long blocks8 = seg_blocks(a0, 256) + (nseg > 1 ? seg_blocks(a1, 256) : 0);
  const long blocks_split = seg_blocks(a0, 128) + (nseg > 1 ? seg_blocks(a1, 128) : 0);
  // 8-wave blocks (one per CU) once they make at least two rounds over the
  // chip
  if (blocks8 >= 2L * cus) return launch_shape<8, 4>(a0, a1, nseg, s);
  // one round or less of 128-query blocks: split each block's keys over two
  // wave groups (two waves per SIMD instead of one)
  if (blocks_split <= cus) return launch_split(a0, a1, nseg, s);
  // otherwise 4-wave blocks, two per CU
  return launch_shape<4, 2>(a0, a1, nseg, s);
}
}  // namespace

hipError_t launch_flash(const FlashArgs& a, hipStream_t s) { return launch_segs(a, a, 1, s); }

hipError_t launch_flash(const FlashArgs* segs, int nseg, hipStream_t s) {
  // pairs of segments share a launch (the grid is sized from their
  // combined blocks); a pair that mixes masked and unmasked segments runs
  // as two launches
  for (int i = 0; i < nseg; i += 2) {
    hipError_t e;
    if (i + 1 < nseg && !segs[i].vis == !segs[i + 1].vis)
      e = launch_segs(segs[i], segs[i + 1], 2, s);
    else if (i + 1 < nseg) {
      e = launch_segs(segs[i], segs[i], 1, s);
      if (e == hipSuccess) e = launch_segs(segs[i + 1], segs[i + 1], 1, s);
    } else
      e = launch_segs(segs[i], segs[i], 1, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qi21
