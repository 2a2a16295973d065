/* qi21 -- the Qwen-Image-2.1 single-stream denoiser step on AMD MI355X (gfx950).
 *
 * A plain C ABI over hand-written HIP kernels.  Sources cited below:
 *   [QI]  docs.rs, cortiq-engine 0.8.4, src/cortiq_engine/qwen_image21.rs
 *         (the CPU reference: module doc "Semantics", Qi21Layout, rope_tables,
 *         block_cpu, prefill, step, step_cpu, target_rope)
 *   [WG]  docs.rs, cortiq-engine 0.8.3, src/gpu_wgpu/qi21.rs (the device
 *         contract: module doc, Guards, geom_ok, mods_dev, prefill, step,
 *         release_key, release)
 *
 * Conventions for every call:
 *   - Array arguments of qi21_model_create, qi21_model_set_block,
 *     qi21_prefill, qi21_step and qi21_step_batch are DEVICE pointers (HBM of
 *     the current HIP device), row-major, float32 unless stated; the caller
 *     owns them and they are only read (or, for `out`, written) during the
 *     call.  Pointer arrays themselves (w[7], keys, xtok[], out[]) live in
 *     host memory.  Layout helpers (qi21_layout_*) take host pointers.
 *   - `stream` is a hipStream_t (NULL = the default stream).  qi21_prefill,
 *     qi21_step and qi21_step_batch synchronise that stream before returning.
 *   - Return value: QI21_OK or one of the error codes; on error
 *     qi21_last_error() (thread-local) explains it.  A call that fails leaves
 *     no partial result: `out` is written only when the call returns QI21_OK
 *     ([WG] step: a non-finite velocity is refused and the output untouched).
 *   - Shape errors and bad masks are found on the host before any device
 *     work (EINVAL); geometry the kernels do not support gives EUNSUPPORTED;
 *     allocation failure gives ENOMEM with no state left behind.
 */
#ifndef QI21_H
#define QI21_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QI21_OK = 0,
  QI21_EINVAL = 1,       /* bad argument: null pointer, length, mask, layer index */
  QI21_EUNSUPPORTED = 2, /* geometry outside what the kernels handle */
  QI21_ENOMEM = 3,       /* device allocation failed (nothing kept) */
  QI21_ENOKEY = 4,       /* no program for that key */
  QI21_ENONFINITE = 5,   /* the step produced a non-finite velocity; out untouched */
  QI21_EDEVICE = 6       /* a HIP call failed */
};

enum { QI21_F32 = 0, QI21_BF16 = 1, QI21_F16 = 2 };

/* Model geometry ([QI] Qi21Config; [WG] geom_ok).  Supported: head_dim 128,
 * heads * 128 == hidden, hidden % 128 == 0 and <= 8192, inter % 64 == 0,
 * in_ch == 64.  eps is the LayerNorm / RMSNorm epsilon (also the final
 * norm's, [WG] dims). */
typedef struct {
  int32_t hidden, heads, head_dim, inter, in_ch;
  float eps;
} qi21_geom;

/* Device allocator hook (e.g. a framework's caching allocator), in the
 * place of the device path's scoped allocation ([WG] alloc_scoped).  NULL
 * alloc = hipMalloc / hipFree; alloc and free are given together or not at
 * all (EINVAL).  alloc returns NULL on failure, which the calling entry
 * point reports as ENOMEM after handing back, through free, every block it
 * took itself (the model's earlier buffers stay).  free is called only
 * after the device has been synchronised, so the block may be reused at
 * once.  ctx is alloc_ctx, passed through. */
typedef void* (*qi21_alloc_fn)(size_t bytes, void* ctx);
typedef void (*qi21_free_fn)(void* ptr, void* ctx);

/* Options ([WG] Guards, knobs).  The five shifts are the power-of-two range
 * guards of the f16 sites (stored value = x * 2^-shift), each clamped to
 * 0..14: attention input (2), qkv panel (4), attention output (4), FFN
 * input (2), SwiGLU hidden (8).  max_programs: prefixes kept at once (2: a
 * positive and a negative prompt); a new key evicts the oldest.  profile:
 * bit mask of kernel classes (see qi21_profile_read) whose launches are
 * bracketed by HIP events on the launch stream; 0 = off.
 * ffn_mode (not on the pages, whose FFN sites are single f16) sets how the
 * FFN input and the SwiGLU hidden are stored:
 *   QI21_FFN_F16 (0, default): single f16, as on the pages; storage error
 *     about 2^-12 of the value at each of the two sites.
 *   QI21_FFN_PAIR (1): f16 (hi, lo) pairs, hi = f16(v), lo = f16(v - hi);
 *     storage error about 2^-23; the gate/up and down GEMMs run over twice
 *     their K, each weight row read for both halves (1.75x the step's
 *     GEMM work).
 *   QI21_FFN_LO8 (2): hi = f16(v) plus the residual v - hi in fp8 (OCP
 *     e4m3) scaled by a power of two per 64 columns; the two FFN weight
 *     planes carry an fp8 copy of each row (scaled per row) next to the
 *     f16 one, and the residual products run on gfx950's scaled fp8 MFMA
 *     (1.35x the step's GEMM work in MFMA cycles).  Storage error about
 *     2^-16 of the value.  Needs hidden % 256 == 0 and inter % 128 == 0
 *     (EUNSUPPORTED otherwise).
 *   QI21_FFN_LO4 (3): as LO8 with the residual and the planes' narrow copy
 *     in fp4 (e2m1) scaled per 32 columns (the MX block), on the scaled fp4
 *     MFMA at twice the fp8 rate (1.17x the step's GEMM work in MFMA
 *     cycles).  Storage error about 2^-14 of the value.  Needs hidden and
 *     inter % 256 == 0.
 * The residual forms' layouts are described in qi21_ops.h. */
enum { QI21_FFN_F16 = 0, QI21_FFN_PAIR = 1, QI21_FFN_LO8 = 2, QI21_FFN_LO4 = 3 };
typedef struct {
  int32_t shift_attn, shift_qkv, shift_ao, shift_ffn, shift_hid;
  int32_t max_programs;
  int32_t profile;
  int32_t gemm_tile; /* -1 = per-shape choice; otherwise a fixed GEMM tile id */
  int32_t ffn_mode;  /* QI21_FFN_F16 / _PAIR / _LO8 / _LO4, see above */
  qi21_alloc_fn alloc;
  qi21_free_fn free;
  void* alloc_ctx;
} qi21_options;

typedef struct qi21_model qi21_model;

void qi21_default_options(qi21_options* opt);

/* Create a model of `nblocks` blocks: the resident weights of the device
 * path ([WG] module doc and prefill: the f16 weight planes are built once
 * per model and kept for every program; [QI] Qi21Dit names the tensors).  img_in: [hidden][64]; proj_out:
 * [64][hidden] (both copied to library-owned f32 buffers).  Weight planes
 * of all blocks are allocated here (f16, ~ (4 H^2 + 3 H I) * 2 bytes per
 * block) and filled by qi21_model_set_block.  opt may be NULL (defaults).
 * Ownership: the model owns every buffer it allocates; destroy releases
 * them. */
int qi21_model_create(const qi21_geom* geom, const qi21_options* opt, int nblocks, const float* img_in,
                      const float* proj_out, void* stream, qi21_model** out);

/* Convert block `layer`'s weights into the model's f16 planes.  w[0..6] =
 * to_q [H][H], to_k [H][H], to_v [H][H], to_out [H][H], gate [I][H],
 * up [I][H], down [H][I] ([QI] Qi21Dit tensor names), row-major [out][in],
 * element type w_dtype (QI21_F32 / QI21_BF16 / QI21_F16).  norm_q, norm_k:
 * [128] f32.  The inputs may be freed after the call returns (it
 * synchronises the stream).  Every block must be set before a prefill. */
int qi21_model_set_block(qi21_model* m, int layer, int w_dtype, const void* const* w, const float* norm_q,
                         const float* norm_k, void* stream);

/* Prefill ([QI] prefill, [WG] prefill): run the lp prefix rows x [lp][H]
 * (already embedded) through every block once with the t = 0 modulation
 * mods0 [4H] (raw: [scale1|gate1|scale2|gate2], gates not yet tanh-ed) and
 * the visibility mask vis [lp] (uint32, query i sees keys [0, vis[i]);
 * must be non-decreasing with 1 <= vis[i] <= lp), keeping each layer's
 * post-RoPE K and V as the program `key`.  rope_p_cos/sin: [lp][64] tables
 * of the prefix rows; rope_t_cos/sin: [n][64] tables of the n target rows
 * under this prefix's layout ([QI] target_rope).  A program with the same
 * key is replaced; past max_programs the oldest is evicted.  Errors:
 * EINVAL (lengths, mask), ENOMEM, EDEVICE. */
int qi21_prefill(qi21_model* m, uint64_t key, int lp, int n, const float* x, const float* rope_p_cos,
                 const float* rope_p_sin, const float* rope_t_cos, const float* rope_t_sin, const uint32_t* vis,
                 const float* mods0, void* stream);

/* Step ([QI] step / step_cpu, [WG] step): latent tokens xtok [n][64] ->
 * velocity out [n][64] for program `key`, with the step modulation mods
 * [4H] (raw, gates tanh-ed inside) and fs [H] = 1 + final_scale.  Every
 * target row sees the lp cached prefix keys and all n target rows.
 * Errors: ENOKEY, EINVAL, ENONFINITE (out untouched), EDEVICE. */
int qi21_step(qi21_model* m, uint64_t key, const float* xtok, const float* mods, const float* fs, float* out,
              void* stream);

/* Several programs' steps as one batched pass (the classifier-free-guidance
 * pair of [WG] module doc): the GEMMs and row kernels run over all
 * programs' rows at once, attention per program against its own prefix.
 * keys[nprog], xtok[nprog] and out[nprog] are host arrays of device
 * pointers ([n_k][64] each); mods and fs are shared.  Same errors as
 * qi21_step; on ENONFINITE no out is written. */
int qi21_step_batch(qi21_model* m, int nprog, const uint64_t* keys, const float* const* xtok, const float* mods,
                    const float* fs, float* const* out, void* stream);

/* txt_in weights ([QI] Qi21Dit: txt_in.text_norm [context_in] f32, a
 * zero-centred RMSNorm weight; txt_in.in_layer [H][context_in] and
 * txt_in.out_layer [H][H] of element type w_dtype, row-major [out][in],
 * bias-free; the projections are kept as f16 planes).  context_in % 64 ==
 * 0, at most 8192.  The inputs may be freed after the call (it
 * synchronises).  Errors: EINVAL, ENOMEM, EDEVICE. */
int qi21_model_set_txt_in(qi21_model* m, int context_in, int w_dtype, const float* txt_norm, const void* txt_in1,
                          const void* txt_in2, void* stream);

/* Text features -> prefix rows on the device ([QI] Qi21Dit::embed_text):
 * feats f32 [n][context_in] -> out f32 [n][H] = txt_in2 gelu_tanh(txt_in1
 * xn), xn = (v / sqrt(mean(v^2) + eps)) * (w + 1) per row (float64 sum of
 * squares; xn and the GELU output are stored as f16).  out feeds
 * qi21_prefill as the text rows.  Enqueued on stream; out is ready when the
 * stream is. */
int qi21_txt_in(qi21_model* m, int n, const float* feats, float* out, void* stream);

/* qi21_txt_in for callers that cannot allocate device memory during the
 * call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same result, with the two
 * intermediates (normalised rows [n][context_in] and GELU hidden [n][H],
 * f16) in a scratch array of qi21_txt_in_noalloc_bytes() bytes (32 MiB)
 * that the library holds on each GPU it runs on until the process ends.
 * Rows fit while round_up(2 n context_in, 256) + 2 n H is within that size
 * (about 2500 rows at context_in 3584, H 3072); more gives EINVAL before
 * any device work.  The model (with its txt_in weights) must already
 * exist; the call allocates nothing and does not synchronise.  Every call
 * on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller.  Errors: EINVAL, EDEVICE. */
int qi21_txt_in_noalloc(qi21_model* m, int n, const float* feats, float* out, void* stream);

/* Size in bytes of qi21_txt_in_noalloc's scratch array. */
size_t qi21_txt_in_noalloc_bytes(void);

/* Time-path weights ([QI] Qi21Dit: time_text_embed.timestep_embedder
 * linear_1 [H][256] and linear_2 [H][H], modulation [4H][H], norm_out
 * [H][H]; row-major [out][in], bias-free), element type w_dtype, kept as f32
 * copies (about 28 H^2 bytes).  Needed by qi21_time_mods, qi21_step_t and
 * qi21_sample.  The inputs may be freed after the call (it synchronises).
 * Errors: EINVAL, ENOMEM, EDEVICE. */
int qi21_model_set_time(qi21_model* m, int w_dtype, const void* t_lin1, const void* t_lin2, const void* modulation,
                        const void* norm_out, void* stream);

/* The modulation of model time t on the device ([QI] Qi21Dit::temb and
 * Qi21Dit::mods): e = [cos(1000 t f_i) | sin(1000 t f_i)], f_i =
 * exp(-ln(10000) i / 128), i < 128; temb = linear_2 silu(linear_1 e);
 * mods [4H] = modulation silu(temb) (raw: [s1|g1|s2|g2]); fs [H] = 1 +
 * norm_out silu(temb), the final scale as qi21_step takes it.  Float64
 * partial sums in the projections.  Enqueued on stream, no
 * synchronisation. */
int qi21_time_mods(qi21_model* m, float t, float* mods, float* fs, void* stream);

/* qi21_step with the modulation of time t computed on the device. */
int qi21_step_t(qi21_model* m, uint64_t key, const float* xtok, float t, float* out, void* stream);

/* A flow-matching Euler sampler over program key ([WG] module doc: an
 * imagine call runs the step once per time; the update rule is not on the
 * pages, and this is the plainest reading): x [n][64] (device, in place)
 * goes through the times t[0..nsteps] (host array): for each k, v =
 * qi21_step_t(x, t[k]), x += (t[k+1] - t[k]) v.  One upload per prompt:
 * only x and the times cross from the host.  Errors as qi21_step; on
 * ENONFINITE at step k, x holds the state after step k - 1. */
int qi21_sample(qi21_model* m, uint64_t key, float* x, int nsteps, const float* t, void* stream);

/* Drop one program ([WG] release_key).  Returns ENOKEY if absent. */
int qi21_release_key(qi21_model* m, uint64_t key);

/* Free everything the model holds ([WG] release).  NULL is a no-op. */
void qi21_model_destroy(qi21_model* m);

/* The last error of the calling thread (empty string if none): the text
 * behind the status code, as the pages' calls return an error value with a
 * message ([WG] step, prefill, geom_ok; [QI] validate).  The pointer stays
 * valid until the thread's next qi21 call. */
const char* qi21_last_error(void);

/* Device bytes the model holds (planes, activations, prefix caches). */
size_t qi21_model_bytes(const qi21_model* m);

/* Change the profiled class mask of a model (as opt.profile). */
int qi21_set_profile(qi21_model* m, int class_mask);

/* Bracket only one launch in every `every` of each profiled class (every
 * >= 1; 1, the default, brackets all), counted from this call: an event
 * pair on the stream delays the launches around it by a few microseconds,
 * so a sample keeps that cost off most launches.  EINVAL for a NULL model
 * or every < 1.  Not from the pages: a measurement aid, like
 * qi21_set_profile. */
int qi21_set_profile_every(qi21_model* m, int every);

/* Profiling (opt.profile != 0): per-class device milliseconds summed over
 * the steps since the last read, and the number of launches of each
 * class; classes: 0 qkv GEMM, 1 qkrope, 2 flash, 3 O GEMM, 4 gate/up GEMM,
 * 5 down GEMM, 6 rowop, 7 embed + final + io.  ms and launches hold 8
 * entries (host).  The counters are reset. */
int qi21_profile_read(qi21_model* m, double* ms, int64_t* launches);

/* ── layout helpers (host memory, no device work) ──
 * A layout is the joint sequence of runs, prefix first, target image last
 * ([QI] Qi21Layout): kind 0 = text of h rows (w ignored), kind 1 = image
 * of h x w latent tokens in raster order. */
typedef struct {
  int32_t kind, h, w;
} qi21_seg;

/* Prefix length and target length of a layout; EINVAL unless the last run
 * is a non-empty image and the prefix is not empty ([QI] validate). */
int qi21_layout_sizes(const qi21_seg* segs, int nseg, int32_t* lp, int32_t* n);

/* Fill any non-NULL of: pos [total][3] (frame, row, col; [QI] positions),
 * vis [lp] (block-causal: text row i sees i+1 keys, an image row sees to
 * the end of its image block; [QI] prefill), cos_p/sin_p [lp][hd/2] and
 * cos_t/sin_t [n][hd/2] RoPE tables ([QI] rope_tables: per axis of width
 * d, frequency 1/theta^(2i/d) in float32, angle float32(pos) * frequency,
 * columns ordered frame, row, col).  axes must be even and sum to head_dim
 * (hd = axes sum). */
int qi21_layout_tables(const qi21_seg* segs, int nseg, const int32_t* axes, float theta, int64_t* pos,
                       uint32_t* vis, float* cos_p, float* sin_p, float* cos_t, float* sin_t);

#ifdef __cplusplus
}
#endif

#endif /* QI21_H */
