/* qi21 single-kernel entry points.
 *
 * Each call runs ONE of the denoiser step's kernels on caller-owned device
 * buffers, enqueued on `stream` (hipStream_t, NULL = default) without
 * synchronising, after host-side shape checks (QI21_EINVAL when a shape or
 * alignment the kernel relies on does not hold; nothing is launched then).
 * They allocate nothing.  They exist so that each kernel can be checked and
 * timed alone at the step's real shapes; qi21_step runs the same kernels.
 * Element types: f16 buffers are IEEE binary16, everything else float32.
 * Sources as in qi21.h.
 */
#ifndef QI21_OPS_H
#define QI21_OPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { QI21_EPI_F16 = 0, QI21_EPI_F32 = 1, QI21_EPI_SWIGLU = 2, QI21_EPI_QKV = 3, QI21_EPI_SWIGLU2 = 4,
       QI21_EPI_RESID = 7, QI21_EPI_SWIGLU8 = 9, QI21_EPI_SWIGLU4 = 10 };

/* out = A W^T ([QI] lin; the four projection sites of [WG] blocks):
 * A f16 [M][lda] (K contiguous), W f16 [N][K].  Epilogues:
 *   F16:    out f16 [M][ldo] = acc * oscale
 *   F32:    out f32 [M][ldo] = acc * oscale
 *   SWIGLU: W interleaved in groups of 32 gate rows then the matching 32 up
 *           rows; out f16 [M][ldo], N/2 columns, = silu(g * inscale) *
 *           (u * inscale) * oscale   ([QI] block_cpu FFN)
 *   QKV:    columns [0, 2N/3) -> out f16 [M][ldo]; columns [2N/3, N) ->
 *           out2 f16 transposed, out2[(c - 2N/3) * ld2 + vt_pos(row)], both
 *           * oscale, where vt_pos swaps bits 2 and 3 of the row index (the
 *           V^T key order the attention kernel reads, see qi21_op_flash)
 *   SWIGLU2: as SWIGLU, each hidden value h stored as the f16 pair
 *           out[r][c] = f16(h), out[r][N/2 + c] = f16(h - f16(h)); ldo >= N
 *           (the hidden of the QI21_FFN_PAIR option, qi21.h)
 * Requires M >= 1, N % 128 == 0, K % 64 == 0, lda % 8 == 0, lda >= K,
 * ldo >= output columns, ldo % 8 == 0 for f16 outputs (rows are written in
 * 16-byte vectors) and % 4 for F32 and QKV, 16-byte aligned A, W and out,
 * for QKV (N/3) % 128 == 0, ld2 % 4 == 0, ld2 >= M.
 * tile: -1 automatic, 0 = 256x256 with 4 waves, 2 = 256x256 with 8 waves
 * (both need N % 256 == 0), 1 = 128x128. */
int qi21_op_gemm(int epi, int M, int N, int K, const void* A, int lda, const void* W, void* out, int ldo,
                 void* out2, int ld2, float oscale, float inscale, int tile, void* stream);

/* The same product with A given as f16 pairs (the QI21_FFN_PAIR option of
 * qi21.h): A f16 [M][lda], lda >= 2K, holds hi in columns [0, K) and lo in
 * [K, 2K); out = (A_hi + A_lo) W^T, W f16 [N][K], accumulated in f32 over
 * both halves (each W row is read for both).  Epilogues F16, F32, SWIGLU,
 * SWIGLU2 with the requirements above (QKV: EINVAL). */
int qi21_op_gemm_pair(int epi, int M, int N, int K, const void* A, int lda, const void* W, void* out, int ldo,
                      float oscale, float inscale, int tile, void* stream);

/* The gated residual of a block branch in the GEMM's epilogue ([QI]
 * gated_add): x f32 [M][ldx] += gate[c] * oscale * sum_k A[m][k] W[c][k % kw]
 * in place, for c < N.  A f16 [M][lda] with K columns read; W f16 [N][kw];
 * K == kw, or K == 2 kw for an A of f16 (hi, lo) pairs (the QI21_FFN_PAIR option
 * of qi21.h).  gate f32 [N], already tanh-ed.  Requires M >= 1, N % 128 ==
 * 0, kw % 64 == 0, lda % 8 == 0, lda >= K, ldx % 4 == 0, ldx >= N.  tile as
 * qi21_op_gemm. */
int qi21_op_gemm_resid(int M, int N, int K, int kw, const void* A, int lda, const void* W, float* x, int ldx,
                       const float* gate, float oscale, int tile, void* stream);

/* A GEMM split over K, for shapes whose whole tiles would leave most CUs
 * idle: part f32 [ksplit][M][N] with part[p][m][c] = oscale * sum over k
 * in [p K/ksplit, (p+1) K/ksplit) of A[m][k] W[c][k % kw]; the sum of the
 * planes is the product (qi21_op_rowop_parts adds them into a gated
 * residual).  A f16 [M][lda], W f16 [N][kw], K == kw or 2 kw as for
 * qi21_op_gemm_resid.  Requires M >= 1, N % 256 == 0, 1 <= ksplit <= 8,
 * K % (64 ksplit) == 0, kw % 64 == 0, lda % 8 == 0, lda >= K, 16-byte
 * aligned pointers.  tile: -1 or 0 (4 waves), 2 (8 waves). */
int qi21_op_gemm_split(int M, int N, int K, int kw, const void* A, int lda, const void* W, float* part, int ksplit,
                       float oscale, int tile, void* stream);

/* The q|k projection with the per-head RMSNorm + RoPE in its epilogue
 * ([QI] block_cpu, qk_norm_rope: the fused form of the QKV GEMM's q|k
 * columns followed by qi21_op_qkrope).  A f16 [M][lda] (H columns), W f16
 * [2H][H] = to_q rows then to_k rows.  For every row and 128-column head
 * the f32 accumulators a are normalised, a * rsqrt(mean(a^2) + eps) *
 * norm_q / norm_k [128] (eps in the accumulators' scale), then pairs
 * (2j, 2j+1) are rotated by the RoPE cos / sin of row r, read from the
 * packed table rope f32 [M][128] that qi21_op_rope_pack writes; q heads go
 * to q_out f16 [M][ldq], k heads to k_out f16 [M][ldk], both at column
 * head*128.  Requires M >= 1, H % 128 == 0, lda % 8 == 0, lda >= H, ldq,
 * ldk >= H and % 8 == 0, 16-byte aligned pointers.  tile: -1 or 0 (4
 * waves), 2 (8 waves). */
int qi21_op_qk_gemm(int M, int H, const void* A, int lda, const void* W, void* q_out, int ldq, void* k_out, int ldk,
                    const float* norm_q, const float* norm_k, const float* rope, float eps, int tile, void* stream);

/* The RoPE tables of n rows ([QI] rope_tables: cos, sin f32 [n][64],
 * row-major, column j = pair (2j, 2j+1)) packed for qi21_op_qk_gemm:
 * out f32 [n][128] with out[r][4m + 0..3] = cos[r][2m], cos[r][2m+1],
 * sin[r][2m], sin[r][2m+1], so the epilogue reads the cos and sin of two
 * adjacent pairs in one 16-byte load.  All three are device pointers,
 * 8-byte aligned (out 16-byte).  Requires n >= 1; EINVAL otherwise. */
int qi21_op_rope_pack(int n, const float* cos, const float* sin, float* out, void* stream);

/* V^T of nkeys rows: out[d][vt_pos(j)] = oscale * sum_k Wv[d][k] X[j][k]
 * for d < H, j < nkeys, where vt_pos swaps bits 2 and 3 of j (the key
 * order qi21_op_flash reads); other columns are not written.  Wv f16
 * [H][lda], X f16 rows of K columns (row stride K); X must hold
 * round_up(nkeys, 256) readable rows (the kernel reads whole 256-row
 * tiles, and rows past nkeys only feed unwritten columns).  Requires
 * K % 64 == 0, lda % 8 == 0, lda >= K, ldo % 8 == 0, ldo >=
 * round_up(nkeys, 16).  tile: -1 or 0 (4 waves), 2 (8 waves). */
int qi21_op_vt_gemm(int H, int nkeys, int K, const void* Wv, int lda, const void* X, void* out, int ldo, float oscale,
                    int tile, void* stream);

/* Attention, head_dim 128 ([QI] attention; [WG] qi_flash): per head h,
 * out[i][h*128 + d] = oscale * sum_j softmax_j(q_i . k_j / sqrt(128)) v_j[d]
 * over keys j < min(n1 + n2, vis[i]) (vis == NULL: all keys).  Keys
 * j < n1 come from k1 [j][ldk1] (column h*128) and V^T vt1 [h*128+d][ldvt1];
 * keys n1 + j from k2 / vt2 likewise.  In a V^T row, key j of a source sits
 * at column vt_pos(j) = j with bits 2 and 3 swapped (a permutation inside
 * each group of 16 keys, as the QKV epilogue of qi21_op_gemm writes it).
 * q f16 [nq][ldq] at column h*128 holds q_i in base-2 units, q_i * log2(e)
 * / sqrt(128): the score's exponent of 2 is then q_i . k_j itself (the
 * model's q norm weights carry that factor, so the q that qi21_op_qk_gemm /
 * qi21_op_qkrope produce with them arrives so scaled).
 * Requires nq >= 1, heads >= 1, n1, n2 >= 0, n1 + n2 >= 1, all leading
 * dimensions % 8 == 0, ldvt >= round_up(n_src, 64) with finite values in
 * the padding columns.  vis (device, uint32 [nq]) should be non-decreasing
 * in [1, n1 + n2]; other values never read out of bounds but give an
 * undefined (finite) result. */
int qi21_op_flash(int nq, int heads, const void* q, int ldq, const void* k1, int ldk1, const void* vt1,
                  int ldvt1, int n1, const void* k2, int ldk2, const void* vt2, int ldvt2, int n2,
                  const uint32_t* vis, void* out, int ldo, float oscale, void* stream);

/* Row op ([WG] qi_rowop; [QI] gated_add, norm_mod) over rows of width h:
 * mode bit 0: x += mods[g_off + c] * y  (gate already tanh-ed)
 * mode bit 1: xn f16 [rows][ldxn] = (LN(x) * (1 + mods[s_off + c])) * oscale
 * mode bit 2 (with bit 1): that value v as the pair xn[r][c] = f16(v),
 *   xn[r][h + c] = f16(v - f16(v)) (QI21_FFN_PAIR, qi21.h)
 * ldxn is xn's row stride in halves: at least h (2h with bit 2) and a
 * multiple of 4; the row op writes columns [0, h) (with bit 2: [0, 2h)) of
 * each row and nothing else (ldxn is ignored without bit 1).
 * Requires rows >= 1, mode in {1, 2, 3, 6, 7}, h % 4 == 0, 4 <= h <= 8192,
 * g_off, s_off % 4 == 0; EINVAL otherwise, before any launch. */
int qi21_op_rowop(int rows, int h, int mode, float* x, const float* y, void* xn, int ldxn, const float* mods,
                  int g_off, int s_off, float eps, float oscale, void* stream);

/* qi21_op_rowop with y the sum of nparts planes [rows][h] pstride floats
 * apart, added in plane order (the partial products of qi21_op_gemm_split).
 * Requires 1 <= nparts <= 8 and, for nparts > 1, pstride >= rows * h;
 * otherwise as qi21_op_rowop. */
int qi21_op_rowop_parts(int rows, int h, int mode, float* x, const float* y, int nparts, size_t pstride, void* xn,
                        int ldxn, const float* mods, int g_off, int s_off, float eps, float oscale, void* stream);

/* The residual operand forms (QI21_FFN_LO8 and QI21_FFN_LO4, qi21.h): a
 * float value v is kept as hi = f16(v) plus its residual in a narrow float
 * times a power-of-two scale.  Scales are E8M0 bytes b, the factor 2^(b -
 * 127).
 *   lo8: columns grouped by 128: group g of a row takes 384 bytes, 128
 *   halves (halves offset 192 g + c % 128) and then 128 OCP e4m3 (fp8)
 *   bytes (byte offset 384 g + 256 + c % 128).  Scales chosen so that a
 *   block's largest |value| / factor lies in [128, 256).
 *   lo4: columns grouped by 256: group g takes 640 bytes, 256 halves
 *   (halves offset 320 g + c % 256) and then 128 bytes of e2m1 (fp4)
 *   values, two per byte, column c (even) in the low nibble of byte 640 g +
 *   512 + (c % 256) / 2.  One scale per 32 columns, the smallest with the
 *   block's largest |value| / factor <= 6.
 *   Activation rows: the halves hold hi = f16(v) and the narrow values the
 *   residual (v - hi) / factor; lo8 has one scale per row and 64 columns,
 *   lo4 one per 32.  The row represents hi + narrow * factor, about 2^-16
 *   (lo8) or 2^-14 (lo4) of v from v.
 *   Weight rows: the halves hold w in f16 and the narrow values a copy
 *   w / factor; lo8 has one scale per row, lo4 one per 32 columns.
 * Scale arrays (uint8) are blocked by 256 rows so that a GEMM reads 32
 * rows' scales from a few cache lines: with q scale bytes per group (lo8
 * activations 2, lo4 8) and G groups per row, the scale of row r, group g,
 * position b sits at byte (r / 256) * 256 G q + g * 256 q + (r % 256) * q +
 * b.  Position b: lo8, the 64-column half (c / 64) % 2; lo4, 4 h + s for
 * the 32-column block 2 s + h of the group (the order the fp4 MFMA's lanes
 * read).  An array holds whole blocks: round_up(rows, 256) rows.  lo8
 * weight scales are one byte per row, sc[r].
 * fmt below is QI21_FFN_LO8 or QI21_FFN_LO4. */

/* qi21_op_rowop_parts writing xn in a residual form: mode 2 or 3 (bits 0
 * and 1 as above), h % 128 (lo8) / 256 (lo4) == 0, xn rows of ldxn halves
 * (ldxn >= 1.5 h / 1.25 h, % 4), and the scales in the blocked array xsc
 * (h / 64 or h / 32 bytes per row).  Otherwise as qi21_op_rowop_parts. */
int qi21_op_rowop_lo(int fmt, int rows, int h, int mode, float* x, const float* y, int nparts, size_t pstride,
                     void* xn, int ldxn, uint8_t* xsc, const float* mods, int g_off, int s_off, float eps,
                     float oscale, void* stream);

/* out = A W^T over operands in a residual form ([QI] lin, the FFN sites of
 * [WG] blocks, with the storage of qi21.h's ffn_mode): A holds M
 * activation rows of lda halves, W N weight rows of ldw halves, each with
 * K columns in the form (lda, ldw >= 1.5 K (lo8) / 1.25 K (lo4), % 8); asc
 * is A's blocked scale array (whole 256-row blocks, K / 64 or K / 32 bytes
 * per row), wsc W's (lo8: [N]; lo4: blocked, K / 32 bytes per row).
 * Computes, in f32 on f16 and scaled fp8 / fp4 MFMAs,
 *   acc[m][n] = sum_k hiA[m][k] w[n][k] + sum_k resA[m][k] wq[n][k]
 * with resA and wq the scaled narrow values (the residual meets the
 * weight's narrow copy).  Epilogues:
 *   F32:     out f32 [M][ldo] = acc * oscale; with ksplit > 1 out is
 *            [ksplit][M][N] (ldo == N) of partial products over the column
 *            ranges [p K / ksplit, (p + 1) K / ksplit) (K / 128 (lo8) or
 *            K / 256 (lo4) a multiple of ksplit)
 *   RESID:   out f32 [M][ldo] += gate[c] * acc * oscale, in place
 *   SWIGLU8 (lo8) / SWIGLU4 (lo4): W the interleaved gate/up plane (see
 *            SWIGLU); the hidden h = silu(g * inscale) * (u * inscale) *
 *            oscale of N/2 columns to out as activation rows in the same
 *            form (rows of ldo halves, ldo >= 0.75 N / 0.625 N and % 8,
 *            written in 16-byte vectors) with scales in the blocked array osc
 * Requires M >= 1, N % 256 == 0, K % 128 (lo8) / 256 (lo4) == 0, 16-byte
 * aligned A, W, out.  Runs the 256 x 256 4-wave kernel. */
int qi21_op_gemm_lo(int fmt, int epi, int M, int N, int K, const void* A, int lda, const uint8_t* asc, const void* W,
                    int ldw, const uint8_t* wsc, void* out, int ldo, const float* gate, uint8_t* osc, int ksplit,
                    float oscale, float inscale, void* stream);

/* The f16 part of a residual-form weight plane: source row r of src
 * [rows][cols] (QI21_F32 / BF16 / F16) goes to dst row (r / group) *
 * gstride + goff + r % group (rows of ld halves, ld >= 1.5 cols (lo8) /
 * 1.25 cols (lo4), % 4), its values at their positions in the form; the
 * narrow values are left for qi21_op_plane_lo_fill.  cols % 128 / 256. */
int qi21_op_plane_lo(int fmt, int src_dtype, const void* src, int rows, int cols, void* dst, int ld, int group,
                     int gstride, int goff, void* stream);

/* The narrow part of a residual-form weight plane whose f16 values are
 * set: lo8, per row the scale e with the row's largest |w| 2^-e in [128,
 * 256), each byte e4m3(w 2^-e), sc[r] = e + 127; lo4, per row and 32
 * columns the smallest e with the block's largest |w| 2^-e <= 6, each
 * nibble e2m1(w 2^-e), the scales in the blocked array sc (whole 256-row
 * blocks, cols / 32 bytes per row).  Round to nearest even.  cols % 128 /
 * 256 == 0, ld as above. */
int qi21_op_plane_lo_fill(int fmt, int rows, int cols, void* plane, int ld, uint8_t* sc, void* stream);

/* Per-head RMSNorm(norm_q | norm_k) then interleaved-pair RoPE on the q
 * (column 0) and k (column heads*128) parts of panel f16 [rows][ldp], in
 * place ([QI] qk_norm_rope).  cos, sin: [rows][64].  kdst != NULL: the
 * normalised k goes to kdst f16 [rows][ldk] instead.  Requires ldp >=
 * 2*heads*128, ldp % 2 == 0. */
int qi21_op_qkrope(int rows, int heads, void* panel, int ldp, const float* norm_q, const float* norm_k,
                   const float* cos, const float* sin, float eps, void* kdst, int ldk, void* stream);

/* x [rows][h] = tok [rows][64] img_in^T, img_in [h][64] ([QI] embed_image).
 * Requires h % 64 == 0. */
int qi21_op_embed(int rows, int h, const float* tok, const float* img_in, float* x, void* stream);

/* out [rows][64] = (LN(x) * fs) proj_out^T, proj_out the Linear weight
 * [64][h] (f32, row-major) ([QI] step_cpu final layer); *flag |= 1 if any
 * output is not finite.  Requires h % 256 == 0. */
int qi21_op_final(int rows, int h, const float* x, const float* fs, const float* proj_out, float eps,
                  float* out, int* flag, void* stream);

/* mods_dev [4h] = [s1 | tanh g1 | s2 | tanh g2] ([WG] mods_dev). */
int qi21_op_mods(int h, const float* mods, float* mods_dev, void* stream);

/* f16 weight plane: source row r of src [rows][cols] (QI21_F32 / BF16 /
 * F16) goes to dst row (r / group) * gstride + goff + r % group. */
int qi21_op_plane(int src_dtype, const void* src, int rows, int cols, void* dst, int group, int gstride,
                  int goff, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QI21_OPS_H */
