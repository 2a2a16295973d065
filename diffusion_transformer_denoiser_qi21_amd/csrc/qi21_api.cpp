// Host runtime of the qi21 C ABI: model and weight-plane ownership, the
// per-prompt programs (prefix K/V caches), argument validation, and the
// launch sequences of prefill and step.
//
// The per-layer launch list follows the device design of [WG] (docs.rs
// cortiq-engine 0.8.3, src/gpu_wgpu/qi21.rs, `blocks` and `build_prog`) and
// the block definition of [QI] (cortiq-engine 0.8.4,
// src/cortiq_engine/qwen_image21.rs, `block_cpu`):
//   qkv GEMM (xn -> q|k panel, V^T) -> qkrope -> attention -> O GEMM ->
//   rowop(x += tanh g1 * y; xn = LN(x)(1+s2)) -> gate/up GEMM + SwiGLU ->
//   down GEMM -> rowop(x += tanh g2 * y; xn = LN(x)(1+s1) for the next block)
// with the f16 sites scaled by power-of-two range guards that each consumer
// multiplies back in f32 ([WG] Guards).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <string>
#include <vector>

#include "../../include/qi21.h"
#include "../../include/qi21_ops.h"
#include "qi21_internal.h"
#include "status.h"

using qi21::f16;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_OK(expr)                                                                          \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(QI21_EDEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

inline float p2(int e) { return std::ldexp(1.0f, e); }
inline size_t round_up(size_t v, size_t m) { return (v + m - 1) / m * m; }

constexpr int NCLASS = 8;
enum Cls { C_QKV = 0, C_QKROPE, C_FLASH, C_O, C_W13, C_W2, C_ROW, C_IO };

struct Acts {
  int cap = 0;  // rows, a multiple of 256
  float* x = nullptr;
  f16* xn = nullptr;
  f16* panel = nullptr;  // [cap][2H] q | k
  f16* vt = nullptr;     // [H][cap] V^T of the pass's own rows
  f16* att = nullptr;    // [cap][H]
  f16* hid = nullptr;    // [cap][I] (pair: [cap][2I]; lo8: rows of 3I bytes)
  float* part = nullptr; // [4 min(cap, 2048)][H] partial products of a down GEMM split over K
  float* mods = nullptr; // [4H] tanh-ed modulation of the pass
  float* out = nullptr;  // [cap][64] velocity before the finite check
  float* rcs = nullptr;  // [cap][128] packed RoPE table of the pass's rows when
                         // they come from several programs, or of a prefill
  uint8_t* xsc = nullptr;  // lo8 / lo4: [cap][H / 64 or H / 32] scales of the FFN input's residuals
  uint8_t* hsc = nullptr;  // lo8 / lo4: [cap][I / 64 or I / 32] scales of the hidden's residuals
};

struct Prog {
  uint64_t key = 0;
  int lp = 0, n = 0, ldc = 0;
  std::vector<f16*> kc;   // per layer [lp][H] post-RoPE K (scale-free)
  std::vector<f16*> vtc;  // per layer [H][ldc] V^T (x 2^-qkv)
  float* rc = nullptr;    // [n][64] target RoPE cos
  float* rs = nullptr;    // [n][64] target RoPE sin
  float* rcs = nullptr;   // [n][128] the same, packed for the q|k GEMM epilogue
};

struct Prof {
  std::vector<hipEvent_t> ev[NCLASS];
  size_t used[NCLASS] = {};
  double ms[NCLASS] = {};
  int64_t n[NCLASS] = {};
  int every = 1;                // bracket one launch of a class in every `every`
  int64_t seen[NCLASS] = {};    // launches of each profiled class so far
};

}  // namespace

struct qi21_model {
  qi21_geom g{};
  qi21_options o{};
  int nb = 0;
  std::vector<f16*> wqkv, wo, w13, w2;
  std::vector<uint8_t*> w13s, w2s;  // lo8: per-row scales of the W13 / W2 fp8 copies; lo4: per row and 32 columns
  std::vector<float*> nq, nk;
  std::vector<char> set;
  float* img_in = nullptr;      // [H][64]
  float* proj_out = nullptr;  // [64][H]
  Acts acts;
  std::deque<Prog> progs;
  int* dflag = nullptr;
  int* hflag = nullptr;  // pinned host
  // time path (qi21_model_set_time): f32 t_lin1 [H][256], t_lin2 [H][H],
  // modulation [4H][H], norm_out [H][H]; work 256 + 2H; the last time's
  // mods [4H] and fs [H]
  float* tw[4] = {nullptr, nullptr, nullptr, nullptr};
  float* twork = nullptr;
  float* tmods = nullptr;
  float* tfs = nullptr;
  // txt_in front (qi21_model_set_txt_in): norm weight f32 [cin], f16 planes
  // txt_in1 [H][cin] and txt_in2 [H][H]; row buffers for txt_cap rows
  int txt_cin = 0, txt_cap = 0;
  float* txt_norm = nullptr;
  f16* txt_w1 = nullptr;
  f16* txt_w2 = nullptr;
  f16* txt_xn = nullptr;  // [txt_cap][cin]
  f16* txt_h = nullptr;   // [txt_cap][H]
  size_t bytes = 0;
  Prof prof;
};

namespace {

void* dalloc(qi21_model* m, size_t bytes) {
  if (bytes == 0) bytes = 256;
  void* p = nullptr;
  if (m->o.alloc) {
    p = m->o.alloc(bytes, m->o.alloc_ctx);
  } else if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    p = nullptr;
  }
  if (p) m->bytes += bytes;
  return p;
}

void dfree(qi21_model* m, void* p, size_t bytes) {
  if (!p) return;
  if (m->o.free) {
    // hipFree waits for the device; a pool allocator may hand the block out
    // again at once, so nothing of ours may still be running on it
    (void)hipDeviceSynchronize();
    m->o.free(p, m->o.alloc_ctx);
  } else {
    (void)hipFree(p);
  }
  m->bytes -= std::min(m->bytes, bytes ? bytes : (size_t)256);
}

constexpr int NACT = 12;

// Half-bytes per column of the FFN input's and the hidden's rows: 4
// (single f16), 8 (f16 pairs), 6 (lo8: f16 plus an fp8 residual), 5 (lo4:
// f16 plus an fp4 residual); likewise for the FFN weight planes (f16, lo8
// or lo4)
size_t ffn_row_nibbles(int mode) {
  return mode == QI21_FFN_PAIR ? 8 : mode == QI21_FFN_LO8 ? 6 : mode == QI21_FFN_LO4 ? 5 : 4;
}
// scale bytes per row of a residual activation of w columns
size_t ffn_scale_bytes(int mode, size_t w) { return mode == QI21_FFN_LO8 ? w / 64 : mode == QI21_FFN_LO4 ? w / 32 : 0; }

size_t acts_bytes(const qi21_geom& g, int ffn_mode, int cap, size_t* parts) {
  const size_t H = g.hidden, I = g.inter, c = cap, f = ffn_row_nibbles(ffn_mode);
  // slot 5: the partial products of a down GEMM split over K (4 planes of
  // up to 2048 rows; split GEMMs only run at fewer than 2048 rows)
  const size_t p[NACT] = {c * H * 4, c * H * f / 2, c * 2 * H * 2, H * c * 2, c * H * 2,
                          4 * std::min<size_t>(c, 2048) * H * 4, c * I * f / 2, 4 * H * 4, c * 64 * 4, c * 128 * 4,
                          c * ffn_scale_bytes(ffn_mode, H), c * ffn_scale_bytes(ffn_mode, I)};
  size_t t = 0;
  for (int i = 0; i < NACT; ++i) {
    if (parts) parts[i] = p[i];
    t += p[i];
  }
  return t;
}

void free_acts(qi21_model* m) {
  size_t parts[NACT];
  acts_bytes(m->g, m->o.ffn_mode, m->acts.cap, parts);
  void* ptrs[NACT] = {m->acts.x,   m->acts.xn,   m->acts.panel, m->acts.vt,  m->acts.att, m->acts.part,
                      m->acts.hid, m->acts.mods, m->acts.out,   m->acts.rcs, m->acts.xsc, m->acts.hsc};
  for (int i = 0; i < NACT; ++i) dfree(m, ptrs[i], parts[i]);
  m->acts = Acts{};
}

// Make the shared activations hold at least `rows` rows; zero-filled so
// padding rows read by GEMM / attention tiles are finite.
int ensure_acts(qi21_model* m, int rows, hipStream_t s) {
  if (m->acts.cap >= rows) return QI21_OK;
  free_acts(m);
  const int cap = (int)round_up((size_t)rows, 256);
  size_t parts[NACT];
  acts_bytes(m->g, m->o.ffn_mode, cap, parts);
  void* p[NACT];
  for (int i = 0; i < NACT; ++i) {
    if (!parts[i]) {
      p[i] = nullptr;
      continue;
    }
    p[i] = dalloc(m, parts[i]);
    if (!p[i]) {
      for (int j = 0; j < i; ++j) dfree(m, p[j], parts[j]);
      return fail(QI21_ENOMEM, "activations for %d rows (%.1f MB) did not fit", rows,
                  acts_bytes(m->g, m->o.ffn_mode, cap, nullptr) / 1e6);
    }
    HIP_OK(qi21::launch_fill32(p[i], 0u, parts[i] / 4, s));
  }
  Acts& a = m->acts;
  a.cap = cap;
  a.x = (float*)p[0];
  a.xn = (f16*)p[1];
  a.panel = (f16*)p[2];
  a.vt = (f16*)p[3];
  a.att = (f16*)p[4];
  a.part = (float*)p[5];
  a.hid = (f16*)p[6];
  a.mods = (float*)p[7];
  a.out = (float*)p[8];
  a.rcs = (float*)p[9];
  a.xsc = (uint8_t*)p[10];
  a.hsc = (uint8_t*)p[11];
  return QI21_OK;
}

void free_prog(qi21_model* m, Prog& p) {
  const size_t H = m->g.hidden;
  for (auto* k : p.kc) dfree(m, k, (size_t)p.lp * H * 2);
  for (auto* v : p.vtc) dfree(m, v, H * p.ldc * 2);
  dfree(m, p.rc, (size_t)p.n * 64 * 4);
  dfree(m, p.rs, (size_t)p.n * 64 * 4);
  dfree(m, p.rcs, (size_t)p.n * 128 * 4);
  p.kc.clear();
  p.vtc.clear();
  p.rc = p.rs = p.rcs = nullptr;
}

size_t time_floats(const qi21_geom& g, int i) {
  const size_t H = g.hidden;
  const size_t n[4] = {H * 256, H * H, 4 * H * H, H * H};
  return n[i];
}

void free_time(qi21_model* m) {
  for (int i = 0; i < 4; ++i) {
    dfree(m, m->tw[i], time_floats(m->g, i) * 4);
    m->tw[i] = nullptr;
  }
  const size_t H = m->g.hidden;
  dfree(m, m->twork, (256 + 2 * H) * 4);
  dfree(m, m->tmods, 4 * H * 4);
  dfree(m, m->tfs, H * 4);
  m->twork = m->tmods = m->tfs = nullptr;
}

void free_txt_rows(qi21_model* m) {
  const size_t H = m->g.hidden;
  dfree(m, m->txt_xn, (size_t)m->txt_cap * m->txt_cin * 2);
  dfree(m, m->txt_h, (size_t)m->txt_cap * H * 2);
  m->txt_xn = m->txt_h = nullptr;
  m->txt_cap = 0;
}

// qi21_txt_in's arguments, checked before any device work
int txt_in_check(const qi21_model* m, int n, const float* feats, const float* out) {
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (!m->txt_cin) return fail(QI21_EINVAL, "no txt_in weights (qi21_model_set_txt_in)");
  if (n < 1 || !feats || !out) return fail(QI21_EINVAL, "txt_in: n %d, feats or out NULL", n);
  return QI21_OK;
}

// The text front over n rows with the two intermediates in xn [n][cin] and
// h [n][H] (f16; only n rows of each are read or written)
int txt_in_run(qi21_model* m, int n, const float* feats, float* out, f16* xn, f16* h, hipStream_t s);

void free_txt(qi21_model* m) {
  free_txt_rows(m);
  const size_t H = m->g.hidden, c = m->txt_cin;
  dfree(m, m->txt_norm, c * 4);
  dfree(m, m->txt_w1, H * c * 2);
  dfree(m, m->txt_w2, H * H * 2);
  m->txt_norm = nullptr;
  m->txt_w1 = m->txt_w2 = nullptr;
  m->txt_cin = 0;
}

Prog* find_prog(qi21_model* m, uint64_t key) {
  for (auto& p : m->progs)
    if (p.key == key) return &p;
  return nullptr;
}

// ── profiling: events around each launch of a class ──
struct Scope {
  qi21_model* m;
  int cls;
  hipStream_t s;
  hipEvent_t stop = nullptr;
  Scope(qi21_model* m_, int c, hipStream_t s_) : m(m_), cls(c), s(s_) {
    if (!((m->o.profile >> cls) & 1)) return;
    Prof& P = m->prof;
    if (P.seen[cls]++ % P.every) return;
    const size_t i = P.used[cls] * 2;
    while (P.ev[cls].size() < i + 2) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return;
      P.ev[cls].push_back(e);
    }
    (void)hipEventRecord(P.ev[cls][i], s);
    stop = P.ev[cls][i + 1];
    P.used[cls]++;
  }
  ~Scope() {
    if (stop) (void)hipEventRecord(stop, s);
  }
};

void prof_collect(qi21_model* m) {
  if (!m->o.profile) return;
  Prof& P = m->prof;
  for (int c = 0; c < NCLASS; ++c) {
    for (size_t i = 0; i < P.used[c]; ++i) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, P.ev[c][2 * i], P.ev[c][2 * i + 1]) == hipSuccess) P.ms[c] += ms;
    }
    P.n[c] += (int64_t)P.used[c];
    P.used[c] = 0;
  }
}

int check_geom(const qi21_geom* g) {
  if (!g) return fail(QI21_EINVAL, "geometry is NULL");
  if (g->head_dim != 128 || g->heads < 1 || g->heads * g->head_dim != g->hidden || g->hidden % 128 != 0 ||
      g->hidden > 8192)
    return fail(QI21_EUNSUPPORTED,
                "geometry hidden %d heads %d head_dim %d: the kernels need head_dim 128, heads*128 == hidden, "
                "hidden %% 128 == 0 and <= 8192",
                g->hidden, g->heads, g->head_dim);
  if (g->inter < 64 || g->inter % 64 != 0 || g->in_ch != 64)
    return fail(QI21_EUNSUPPORTED, "geometry inter %d in_ch %d: the kernels need inter %% 64 == 0 and 64 channels",
                g->inter, g->in_ch);
  if (!(g->eps >= 0.0f) || !std::isfinite(g->eps)) return fail(QI21_EINVAL, "eps %g", (double)g->eps);
  return QI21_OK;
}

struct Guard {
  int attn, qkv, ao, ffn, hid;
};
Guard guards(const qi21_model* m) {
  auto c = [](int v) { return std::min(14, std::max(0, v)); };
  return Guard{c(m->o.shift_attn), c(m->o.shift_qkv), c(m->o.shift_ao), c(m->o.shift_ffn), c(m->o.shift_hid)};
}

qi21::GemmArgs gemm_args(int M, int N, int K, const f16* A, int lda, const f16* W, void* out, int ldo,
                         float oscale, float inscale = 1.0f, f16* out2 = nullptr, int ld2 = 0) {
  qi21::GemmArgs a;
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = A;
  a.lda = lda;
  a.W = W;
  a.kw = K;
  a.out = out;
  a.ldo = ldo;
  a.out2 = out2;
  a.ld2 = ld2;
  a.oscale = oscale;
  a.inscale = inscale;
  return a;
}

int txt_in_run(qi21_model* m, int n, const float* feats, float* out, f16* xn, f16* h, hipStream_t s) {
  const int H = m->g.hidden, c = m->txt_cin;
  HIP_OK(qi21::launch_txtnorm(n, c, feats, m->txt_norm, m->g.eps, xn, s));
  const int tile = m->o.gemm_tile;
  qi21::GemmArgs g1 = gemm_args(n, H, c, xn, c, m->txt_w1, h, H, 1.0f);
  HIP_OK(qi21::launch_gemm(qi21::EPI_GELU, g1, tile, s));
  qi21::GemmArgs g2 = gemm_args(n, H, H, h, H, m->txt_w2, out, H, 1.0f);
  HIP_OK(qi21::launch_gemm(qi21::EPI_F32, g2, tile, s));
  return QI21_OK;
}

// One segment of the rows of a pass (one program's rows in a batch).
struct Seg {
  int row0, rows;
  Prog* p;           // step: the program whose cache the rows attend to
  const float* rc;   // RoPE tables of these rows
  const float* rs;
  const float* rcs;  // the same, packed ([rows][128], launch_rope_pack)
};

// Blocks of one pass over `rows` rows of m->acts.  Prefill: one segment,
// `pre` receives the caches (keys written by qkrope, V^T by the GEMM), the
// mask is vis, and the last layer stops after the cache write.  Step: the
// caches of each segment's program are read.
int run_blocks(qi21_model* m, int rows, const std::vector<Seg>& segs, Prog* pre, const uint32_t* vis,
               hipStream_t s) {
  const qi21_geom& g = m->g;
  const int H = g.hidden, I = g.inter, nh = g.heads;
  const Guard gd = guards(m);
  Acts& a = m->acts;
  const int tile = m->o.gemm_tile;
  // With the large-M GEMM the per-head q/k RMSNorm + RoPE runs in the q|k
  // GEMM's epilogue and V^T comes from its own GEMM (Wv times the rows);
  // otherwise the qkv GEMM writes q|k and V^T and qkrope follows.
  const int tile_qk = tile >= 0 ? tile : qi21::gemm_pick_tile(rows, 2 * H, H);
  const bool fused = tile_qk == 0 || tile_qk == 2;
  const float* rope = segs[0].rcs;
  if (fused && (segs.size() > 1 || segs[0].row0 != 0)) {  // one table for all rows of the pass
    for (const Seg& sg : segs)
      HIP_OK(hipMemcpyAsync(a.rcs + (size_t)sg.row0 * 128, sg.rcs, (size_t)sg.rows * 128 * 4, hipMemcpyDeviceToDevice,
                            s));
    rope = a.rcs;
  }
  for (int l = 0; l < m->nb; ++l) {
    const bool last = l + 1 == m->nb;
    f16* vt = pre ? pre->vtc[l] : a.vt;
    const int ldv = pre ? pre->ldc : a.cap;
    if (fused) {
      Scope sc(m, C_QKV, s);
      // q|k: normalised and rotated in the epilogue (scale-free); the
      // accumulators carry 2^-attn, so the norm's eps does too
      qi21::GemmArgs qk = gemm_args(rows, 2 * H, H, a.xn, H, m->wqkv[l], a.panel, 2 * H, 1.0f);
      qk.nq = m->nq[l];
      qk.nk = m->nk[l];
      qk.rope = rope;
      qk.eps = g.eps * p2(-2 * gd.attn);
      qk.kout = pre ? pre->kc[l] : a.panel + H;
      qk.ldk = pre ? H : 2 * H;
      HIP_OK(qi21::launch_gemm(qi21::EPI_QKROPE, qk, tile_qk, s));
      // V^T = Wv xn^T (x 2^-qkv) over the rows padded to whole tiles
      qi21::GemmArgs v = gemm_args(H, (int)round_up((size_t)rows, 256), H, m->wqkv[l] + (size_t)2 * H * H, H, a.xn,
                                   vt, ldv, p2(gd.attn - gd.qkv));
      v.nvalid = rows;
      HIP_OK(qi21::launch_gemm(qi21::EPI_VT, v, tile_qk, s));
    } else {
      {  // qkv: panel q|k (x 2^-qkv), V^T to the cache (prefill) or acts.vt
        Scope sc(m, C_QKV, s);
        HIP_OK(qi21::launch_gemm(qi21::EPI_QKV,
                                 gemm_args(rows, 3 * H, H, a.xn, H, m->wqkv[l], a.panel, 2 * H,
                                           p2(gd.attn - gd.qkv), 1.0f, vt, ldv),
                                 tile, s));
      }
      {  // per-head RMSNorm + RoPE; the norm's eps follows the panel's guard
        Scope sc(m, C_QKROPE, s);
        const float eps = g.eps * p2(-2 * gd.qkv);
        for (const Seg& sg : segs)
          HIP_OK(qi21::launch_qkrope(sg.rows, nh, a.panel + (size_t)sg.row0 * 2 * H, 2 * H, m->nq[l], m->nk[l], sg.rc,
                                     sg.rs, eps, pre ? pre->kc[l] : nullptr, H, s));
      }
    }
    if (pre && last) break;  // only this layer's K/V leave a prefill
    {
      Scope sc(m, C_FLASH, s);
      std::vector<qi21::FlashArgs> fa;
      for (const Seg& sg : segs) {
        qi21::FlashArgs f{};
        f.q = a.panel + (size_t)sg.row0 * 2 * H;
        f.ldq = 2 * H;
        f.nq = sg.rows;
        f.heads = nh;
        if (pre) {
          f.k1 = pre->kc[l];
          f.ldk1 = H;
          f.vt1 = pre->vtc[l];
          f.ldvt1 = pre->ldc;
          f.n1 = pre->lp;
          f.n2 = 0;
          f.vis = vis;
        } else {
          f.k1 = sg.p->kc[l];
          f.ldk1 = H;
          f.vt1 = sg.p->vtc[l];
          f.ldvt1 = sg.p->ldc;
          f.n1 = sg.p->lp;
          f.k2 = a.panel + (size_t)sg.row0 * 2 * H + H;
          f.ldk2 = 2 * H;
          f.vt2 = a.vt + sg.row0;
          f.ldvt2 = a.cap;
          f.n2 = sg.rows;
          f.vis = nullptr;
        }
        f.out = a.att + (size_t)sg.row0 * H;
        f.ldo = H;
        f.oscale = p2(gd.qkv - gd.ao);
        fa.push_back(f);
      }
      HIP_OK(qi21::launch_flash(fa.data(), (int)fa.size(), s));
    }
    // The FFN input (in xn) and the hidden: single f16; f16 (hi, lo) pairs
    // in rows of 2H / 2I, both FFN GEMMs then running over K doubled with
    // each W row read twice; or lo8 (f16 plus scaled fp8 residuals, rows
    // of 3H / 3I bytes, with the weight planes in the same form).
    const int fm = m->o.ffn_mode;
    const bool lo8 = fm == QI21_FFN_LO8, lo4 = fm == QI21_FFN_LO4, lo = lo8 || lo4;
    const int pf = fm == QI21_FFN_PAIR ? 2 : 1;
    const int ffn_bits = fm == QI21_FFN_PAIR ? 4 : lo8 ? 8 : lo4 ? 16 : 0;  // the FFN-input row pass's mode bits
    const int kx = lo8 ? 3 * H / 2 : lo4 ? 5 * H / 4 : pf * H;          // the FFN input's row, in halves
    const int kh = lo8 ? 3 * I / 2 : lo4 ? 5 * I / 4 : pf * I;          // the hidden's row, in halves
    const int sx = lo8 ? H / 64 : H / 32, sh = lo8 ? I / 64 : I / 32;  // their scale bytes per row
    auto ffn_lo = [&](qi21::GemmArgs& ga, const uint8_t* asc, int lds, const uint8_t* wsc, int ldws) {
      ga.lo = lo8 ? 8 : 4;
      ga.asc = asc;
      ga.lds = lds;
      ga.wsc = wsc;
      ga.ldws = ldws;
    };
    // the O GEMM split over K like the down GEMM below, or with the gated
    // residual in its epilogue
    const int spo = tile < 0 ? qi21::gemm_split_count(rows, H, H, 4) : 1;
    if (spo > 1 && (size_t)spo * rows <= 4 * std::min<size_t>(a.cap, 2048)) {
      {
        Scope sc(m, C_O, s);
        qi21::GemmArgs o = gemm_args(rows, H, H, a.att, H, m->wo[l], a.part, H, p2(gd.ao));
        o.ksplit = spo;
        o.pstride = (size_t)rows * H;
        HIP_OK(qi21::launch_gemm(qi21::EPI_F32, o, 0, s));
      }
      Scope sc(m, C_ROW, s);  // x += tanh(g1) sum_p part_p; xn = LN(x)(1 + s2)
      HIP_OK(qi21::launch_rowop(rows, H, 3 | ffn_bits, a.x, a.part, a.xn, a.mods, H, 2 * H, g.eps, p2(-gd.ffn), s,
                                spo, (size_t)rows * H, a.xsc));
    } else {
      {  // x += tanh(g1) (att Wo^T) in the O GEMM's epilogue
        Scope sc(m, C_O, s);
        qi21::GemmArgs o = gemm_args(rows, H, H, a.att, H, m->wo[l], a.x, H, p2(gd.ao));
        o.gate = a.mods + H;
        HIP_OK(qi21::launch_gemm(qi21::EPI_RESID, o, tile, s));
      }
      {  // xn = LN(x)(1 + s2)
        Scope sc(m, C_ROW, s);
        HIP_OK(qi21::launch_rowop(rows, H, 2 | ffn_bits, a.x, nullptr, a.xn, a.mods, 0, 2 * H, g.eps, p2(-gd.ffn), s,
                                  1, 0, a.xsc));
      }
    }
    {
      Scope sc(m, C_W13, s);
      qi21::GemmArgs ga = gemm_args(rows, 2 * I, kx, a.xn, kx, m->w13[l], a.hid, kh, p2(-gd.hid), p2(gd.ffn));
      if (lo) {
        ffn_lo(ga, a.xsc, sx, m->w13s[l], lo4 ? H / 32 : 0);
        ga.osc = a.hsc;
        HIP_OK(qi21::launch_gemm(lo8 ? qi21::EPI_SWIGLU8 : qi21::EPI_SWIGLU4, ga, 0, s));
      } else {
        ga.kw = H;
        HIP_OK(qi21::launch_gemm(pf == 2 ? qi21::EPI_SWIGLU2 : qi21::EPI_SWIGLU, ga, tile, s));
      }
    }
    // Where whole 256 x 256 tiles would leave most CUs idle (512 to 2047
    // rows), the down GEMM runs split over K into partial products and the
    // row pass adds them: x += tanh(g2) sum_p part_p, then (but in the
    // last block) the next block's xn = LN(x)(1 + s1).  Otherwise the
    // gated residual runs in the GEMM's epilogue.  (lo8 / lo4: the split
    // falls on whole groups of 128 / 256 columns, so the count must divide
    // I / 128 / I / 256; gemm_split_count sees the K with that many k-tiles.)
    const int sp = tile < 0 ? qi21::gemm_split_count(rows, H, lo8 ? I / 2 : lo4 ? I / 4 : pf * I, 4) : 1;
    if (sp > 1 && (size_t)sp * rows <= 4 * std::min<size_t>(a.cap, 2048)) {
      {
        Scope sc(m, C_W2, s);
        qi21::GemmArgs ga = gemm_args(rows, H, kh, a.hid, kh, m->w2[l], a.part, H, p2(gd.hid));
        if (lo)
          ffn_lo(ga, a.hsc, sh, m->w2s[l], lo4 ? I / 32 : 0);
        else
          ga.kw = I;
        ga.ksplit = sp;
        ga.pstride = (size_t)rows * H;
        HIP_OK(qi21::launch_gemm(qi21::EPI_F32, ga, 0, s));
      }
      Scope sc(m, C_ROW, s);
      HIP_OK(qi21::launch_rowop(rows, H, last ? 1 : 3, a.x, a.part, a.xn, a.mods, 3 * H, 0, g.eps, p2(-gd.attn), s,
                                sp, (size_t)rows * H));
    } else {
      {  // x += tanh(g2) (hid W2^T) in the down GEMM's epilogue
        Scope sc(m, C_W2, s);
        qi21::GemmArgs ga = gemm_args(rows, H, kh, a.hid, kh, m->w2[l], a.x, H, p2(gd.hid));
        ga.gate = a.mods + 3 * H;
        if (lo)
          ffn_lo(ga, a.hsc, sh, m->w2s[l], lo4 ? I / 32 : 0);
        else
          ga.kw = I;
        HIP_OK(qi21::launch_gemm(qi21::EPI_RESID, ga, lo ? 0 : tile, s));
      }
      if (!last) {  // the next block's xn = LN(x)(1 + s1)
        Scope sc(m, C_ROW, s);
        HIP_OK(qi21::launch_rowop(rows, H, 2, a.x, nullptr, a.xn, a.mods, 0, 0, g.eps, p2(-gd.attn), s));
      }
    }
  }
  return QI21_OK;
}

int sync_stream(hipStream_t s) {
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(QI21_EDEVICE, "stream synchronize: %s", hipGetErrorString(e));
  return QI21_OK;
}

}  // namespace

// ───────────────────────────── C ABI ─────────────────────────────

extern "C" {

const char* qi21_last_error(void) { return g_err.c_str(); }

}  // extern "C"

void qi21::set_error_text(const char* msg) { g_err = msg; }

int qi21::txt_in_scratch(qi21_model* m, int n, const float* feats, float* out, void* scratch, size_t bytes,
                         void* stream) {
  g_err.clear();
  int rc = txt_in_check(m, n, feats, out);
  if (rc) return rc;
  const size_t H = m->g.hidden, c = m->txt_cin;
  const size_t xn_bytes = round_up((size_t)n * c * 2, 256), need = xn_bytes + (size_t)n * H * 2;
  if (!scratch) return fail(QI21_EINVAL, "txt_in: no scratch");
  if (need > bytes)
    return fail(QI21_EINVAL, "txt_in without allocation: %d rows need %zu scratch bytes, the limit is %zu (%zu rows)", n,
                need, bytes, bytes / ((c + H) * 2 + 256));
  f16* xn = (f16*)scratch;
  f16* h = (f16*)((char*)scratch + xn_bytes);
  return txt_in_run(m, n, feats, out, xn, h, (hipStream_t)stream);
}

extern "C" {

void qi21_default_options(qi21_options* o) {
  if (!o) return;
  std::memset(o, 0, sizeof *o);
  o->shift_attn = 2;
  o->shift_qkv = 4;
  o->shift_ao = 4;
  o->shift_ffn = 2;
  o->shift_hid = 8;
  o->max_programs = 2;
  o->profile = 0;
  o->gemm_tile = -1;
  o->ffn_mode = QI21_FFN_F16;
}

size_t qi21_model_bytes(const qi21_model* m) { return m ? m->bytes : 0; }

void qi21_model_destroy(qi21_model* m) {
  if (!m) return;
  (void)hipDeviceSynchronize();
  for (auto& p : m->progs) free_prog(m, p);
  m->progs.clear();
  free_acts(m);
  const size_t H = m->g.hidden, I = m->g.inter;
  const int pm = m->o.ffn_mode == QI21_FFN_PAIR ? QI21_FFN_F16 : m->o.ffn_mode;  // the planes' form
  const size_t fb = ffn_row_nibbles(pm);
  for (int l = 0; l < m->nb; ++l) {
    dfree(m, m->wqkv[l], 3 * H * H * 2);
    dfree(m, m->wo[l], H * H * 2);
    dfree(m, m->w13[l], 2 * I * H * fb / 2);
    dfree(m, m->w2[l], H * I * fb / 2);
    dfree(m, m->nq[l], 128 * 4);
    dfree(m, m->nk[l], 128 * 4);
    if (l < (int)m->w13s.size()) dfree(m, m->w13s[l], pm == QI21_FFN_LO4 ? 2 * I * H / 32 : 2 * I);
    if (l < (int)m->w2s.size()) dfree(m, m->w2s[l], pm == QI21_FFN_LO4 ? H * I / 32 : H);
  }
  dfree(m, m->img_in, H * 64 * 4);
  dfree(m, m->proj_out, H * 64 * 4);
  free_time(m);
  free_txt(m);
  dfree(m, m->dflag, 256);
  if (m->hflag) (void)hipHostFree(m->hflag);
  for (int c = 0; c < NCLASS; ++c)
    for (auto e : m->prof.ev[c]) (void)hipEventDestroy(e);
  delete m;
}

int qi21_model_create(const qi21_geom* geom, const qi21_options* opt, int nblocks, const float* img_in,
                      const float* proj_out, void* stream, qi21_model** out) {
  g_err.clear();
  if (!out) return fail(QI21_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_geom(geom);
  if (rc) return rc;
  if (nblocks < 1 || nblocks > 4096) return fail(QI21_EINVAL, "nblocks %d", nblocks);
  if (!img_in || !proj_out) return fail(QI21_EINVAL, "img_in / proj_out is NULL");
  hipStream_t s = (hipStream_t)stream;
  qi21_model* m = new qi21_model();
  m->g = *geom;
  if (opt)
    m->o = *opt;
  else
    qi21_default_options(&m->o);
  if ((m->o.alloc == nullptr) != (m->o.free == nullptr)) {
    delete m;
    return fail(QI21_EINVAL, "alloc and free hooks must be given together");
  }
  if (m->o.max_programs < 1) m->o.max_programs = 1;
  if (m->o.ffn_mode < QI21_FFN_F16 || m->o.ffn_mode > QI21_FFN_LO4) {
    const int fm = m->o.ffn_mode;
    delete m;
    return fail(QI21_EINVAL, "ffn_mode %d (0 to 3)", fm);
  }
  if ((m->o.ffn_mode == QI21_FFN_LO8 && (geom->hidden % 256 != 0 || geom->inter % 128 != 0)) ||
      (m->o.ffn_mode == QI21_FFN_LO4 && (geom->hidden % 256 != 0 || geom->inter % 256 != 0))) {
    const int fm = m->o.ffn_mode;
    delete m;
    return fail(QI21_EUNSUPPORTED, "ffn_mode %s needs hidden %% 256 == 0 and inter %% %d == 0 (hidden %d, inter %d)",
                fm == QI21_FFN_LO8 ? "lo8" : "lo4", fm == QI21_FFN_LO8 ? 128 : 256, geom->hidden, geom->inter);
  }
  m->nb = nblocks;
  const size_t H = geom->hidden, I = geom->inter;
  const int pm = m->o.ffn_mode == QI21_FFN_PAIR ? QI21_FFN_F16 : m->o.ffn_mode;  // the FFN planes' form
  const bool lop = pm == QI21_FFN_LO8 || pm == QI21_FFN_LO4;
  const size_t fb = ffn_row_nibbles(pm);  // half-bytes per FFN plane column
  m->wqkv.assign(nblocks, nullptr);
  m->wo.assign(nblocks, nullptr);
  m->w13.assign(nblocks, nullptr);
  m->w2.assign(nblocks, nullptr);
  m->nq.assign(nblocks, nullptr);
  m->nk.assign(nblocks, nullptr);
  m->set.assign(nblocks, 0);
  if (lop) {
    m->w13s.assign(nblocks, nullptr);
    m->w2s.assign(nblocks, nullptr);
  }
  const size_t s13 = pm == QI21_FFN_LO4 ? 2 * I * H / 32 : 2 * I, s2 = pm == QI21_FFN_LO4 ? H * I / 32 : H;
  bool ok = true;
  for (int l = 0; l < nblocks && ok; ++l) {
    ok = (m->wqkv[l] = (f16*)dalloc(m, 3 * H * H * 2)) && (m->wo[l] = (f16*)dalloc(m, H * H * 2)) &&
         (m->w13[l] = (f16*)dalloc(m, 2 * I * H * fb / 2)) && (m->w2[l] = (f16*)dalloc(m, H * I * fb / 2)) &&
         (m->nq[l] = (float*)dalloc(m, 128 * 4)) && (m->nk[l] = (float*)dalloc(m, 128 * 4));
    if (ok && lop) ok = (m->w13s[l] = (uint8_t*)dalloc(m, s13)) && (m->w2s[l] = (uint8_t*)dalloc(m, s2));
  }
  ok = ok && (m->img_in = (float*)dalloc(m, H * 64 * 4)) && (m->proj_out = (float*)dalloc(m, H * 64 * 4)) &&
       (m->dflag = (int*)dalloc(m, 256));
  if (!ok) {
    qi21_model_destroy(m);
    return fail(QI21_ENOMEM, "weight planes for %d blocks (%.2f GB) did not fit", nblocks,
                (double)nblocks * (8 * H * H + 3 * H * I * fb / 2) / 1e9);
  }
  if (hipHostMalloc((void**)&m->hflag, sizeof(int), hipHostMallocDefault) != hipSuccess) {
    m->hflag = nullptr;
    qi21_model_destroy(m);
    return fail(QI21_ENOMEM, "pinned host flag");
  }
  hipError_t e = hipMemcpyAsync(m->img_in, img_in, H * 64 * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(m->proj_out, proj_out, H * 64 * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    qi21_model_destroy(m);
    return fail(QI21_EDEVICE, "model upload: %s", hipGetErrorString(e));
  }
  *out = m;
  return QI21_OK;
}

int qi21_model_set_block(qi21_model* m, int layer, int w_dtype, const void* const* w, const float* norm_q,
                         const float* norm_k, void* stream) {
  g_err.clear();
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (layer < 0 || layer >= m->nb) return fail(QI21_EINVAL, "layer %d of %d", layer, m->nb);
  if (w_dtype < QI21_F32 || w_dtype > QI21_F16) return fail(QI21_EINVAL, "weight dtype %d", w_dtype);
  if (!w || !norm_q || !norm_k) return fail(QI21_EINVAL, "weight pointers are NULL");
  for (int i = 0; i < 7; ++i)
    if (!w[i]) return fail(QI21_EINVAL, "weight %d is NULL", i);
  hipStream_t s = (hipStream_t)stream;
  const int H = m->g.hidden, I = m->g.inter;
  // qkv plane rows: q [0, H), k [H, 2H), v [2H, 3H)
  for (int i = 0; i < 3; ++i) HIP_OK(qi21::launch_plane(w_dtype, w[i], H, H, m->wqkv[layer], H, 0, i * H, s));
  HIP_OK(qi21::launch_plane(w_dtype, w[3], H, H, m->wo[layer], H, 0, 0, s));
  // gate/up interleaved by 32 rows: plane rows 64j + r = gate 32j + r, 64j + 32 + r = up 32j + r;
  // lo8: both FFN planes in the lo8 row form, their fp8 residual bytes and
  // per-row scales derived from the f16 values
  const bool lo8 = m->o.ffn_mode == QI21_FFN_LO8, lo4 = m->o.ffn_mode == QI21_FFN_LO4;
  const int lo = lo8 ? 8 : lo4 ? 4 : 0;
  const int ld13 = lo8 ? 3 * H / 2 : lo4 ? 5 * H / 4 : H, ld2 = lo8 ? 3 * I / 2 : lo4 ? 5 * I / 4 : I;
  HIP_OK(qi21::launch_plane(w_dtype, w[4], I, H, m->w13[layer], 32, 64, 0, s, ld13, lo));
  HIP_OK(qi21::launch_plane(w_dtype, w[5], I, H, m->w13[layer], 32, 64, 32, s, ld13, lo));
  HIP_OK(qi21::launch_plane(w_dtype, w[6], H, I, m->w2[layer], H, 0, 0, s, ld2, lo));
  if (lo8) {
    HIP_OK(qi21::launch_plane8(2 * I, H, m->w13[layer], ld13, m->w13s[layer], s));
    HIP_OK(qi21::launch_plane8(H, I, m->w2[layer], ld2, m->w2s[layer], s));
  }
  if (lo4) {
    HIP_OK(qi21::launch_plane4(2 * I, H, m->w13[layer], ld13, m->w13s[layer], s));
    HIP_OK(qi21::launch_plane4(H, I, m->w2[layer], ld2, m->w2s[layer], s));
  }
  // the q norm weights carry the softmax's log2(e) / sqrt(128), so every q
  // the block produces is in the base-2 units the attention kernels take
  HIP_OK(qi21::launch_scale(128, norm_q, (float)(1.4426950408889634 / 11.313708498984761), m->nq[layer], s));
  HIP_OK(hipMemcpyAsync(m->nk[layer], norm_k, 128 * 4, hipMemcpyDeviceToDevice, s));
  int rc = sync_stream(s);
  if (rc) return rc;
  m->set[layer] = 1;
  return QI21_OK;
}

int qi21_prefill(qi21_model* m, uint64_t key, int lp, int n, const float* x, const float* rope_p_cos,
                 const float* rope_p_sin, const float* rope_t_cos, const float* rope_t_sin, const uint32_t* vis,
                 const float* mods0, void* stream) {
  g_err.clear();
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (lp < 1 || n < 1 || lp > (1 << 20) || n > (1 << 20)) return fail(QI21_EINVAL, "lp %d, n %d", lp, n);
  if (!x || !rope_p_cos || !rope_p_sin || !rope_t_cos || !rope_t_sin || !vis || !mods0)
    return fail(QI21_EINVAL, "prefill arguments include NULL");
  for (int l = 0; l < m->nb; ++l)
    if (!m->set[l]) return fail(QI21_EINVAL, "block %d has no weights", l);
  hipStream_t s = (hipStream_t)stream;
  // the mask the kernel walks: non-decreasing, each row sees >= 1 key
  std::vector<uint32_t> hv(lp);
  HIP_OK(hipMemcpyAsync(hv.data(), vis, (size_t)lp * 4, hipMemcpyDeviceToHost, s));
  int rc = sync_stream(s);
  if (rc) return rc;
  for (int i = 0; i < lp; ++i) {
    if (hv[i] < 1 || hv[i] > (uint32_t)lp)
      return fail(QI21_EINVAL, "vis[%d] = %u is outside [1, %d]", i, hv[i], lp);
    if (i && hv[i] < hv[i - 1]) return fail(QI21_EINVAL, "vis is not non-decreasing at row %d", i);
  }
  // replace the key, evict the oldest past max_programs
  for (auto it = m->progs.begin(); it != m->progs.end(); ++it)
    if (it->key == key) {
      free_prog(m, *it);
      m->progs.erase(it);
      break;
    }
  while ((int)m->progs.size() >= m->o.max_programs) {
    free_prog(m, m->progs.front());
    m->progs.pop_front();
  }
  rc = ensure_acts(m, std::max(lp, n), s);
  if (rc) return rc;
  const size_t H = m->g.hidden;
  Prog p;
  p.key = key;
  p.lp = lp;
  p.n = n;
  p.ldc = (int)round_up((size_t)lp, 64);
  bool ok = true;
  for (int l = 0; l < m->nb && ok; ++l) {
    f16* k = (f16*)dalloc(m, (size_t)lp * H * 2);
    f16* v = (f16*)dalloc(m, H * p.ldc * 2);
    if (k) p.kc.push_back(k);
    if (v) p.vtc.push_back(v);
    ok = k && v;
    if (!ok) {
      if (k && !v) { dfree(m, k, (size_t)lp * H * 2); p.kc.pop_back(); }
      if (v && !k) { dfree(m, v, H * p.ldc * 2); p.vtc.pop_back(); }
    }
  }
  ok = ok && (p.rc = (float*)dalloc(m, (size_t)n * 64 * 4)) && (p.rs = (float*)dalloc(m, (size_t)n * 64 * 4)) &&
       (p.rcs = (float*)dalloc(m, (size_t)n * 128 * 4));
  if (!ok) {
    free_prog(m, p);
    return fail(QI21_ENOMEM, "prefix cache of %d rows x %d blocks did not fit", lp, m->nb);
  }
  for (auto* v : p.vtc) HIP_OK(qi21::launch_fill32(v, 0u, H * p.ldc / 2, s));
  HIP_OK(hipMemcpyAsync(p.rc, rope_t_cos, (size_t)n * 64 * 4, hipMemcpyDeviceToDevice, s));
  HIP_OK(hipMemcpyAsync(p.rs, rope_t_sin, (size_t)n * 64 * 4, hipMemcpyDeviceToDevice, s));
  HIP_OK(qi21::launch_rope_pack(n, rope_t_cos, rope_t_sin, p.rcs, s));
  // the prefix pass
  Acts& a = m->acts;
  const Guard gd = guards(m);
  HIP_OK(qi21::launch_mods((int)H, mods0, a.mods, s));
  HIP_OK(hipMemcpyAsync(a.x, x, (size_t)lp * H * 4, hipMemcpyDeviceToDevice, s));
  HIP_OK(qi21::launch_rowop(lp, (int)H, 2, a.x, nullptr, a.xn, a.mods, 0, 0, m->g.eps, p2(-gd.attn), s));
  HIP_OK(qi21::launch_rope_pack(lp, rope_p_cos, rope_p_sin, a.rcs, s));
  std::vector<Seg> segs{Seg{0, lp, nullptr, rope_p_cos, rope_p_sin, a.rcs}};
  rc = run_blocks(m, lp, segs, &p, vis, s);
  if (rc == QI21_OK) rc = sync_stream(s);
  prof_collect(m);
  if (rc) {
    free_prog(m, p);
    return rc;
  }
  m->progs.push_back(std::move(p));
  return QI21_OK;
}

int qi21_step_batch(qi21_model* m, int nprog, const uint64_t* keys, const float* const* xtok, const float* mods,
                    const float* fs, float* const* out, void* stream) {
  g_err.clear();
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (nprog < 1 || nprog > 64 || !keys || !xtok || !out || !mods || !fs)
    return fail(QI21_EINVAL, "step arguments include NULL or nprog %d", nprog);
  // each program's rows start at a multiple of 64 of the shared
  // activations, so its V^T columns stay 16-byte aligned for the attention
  // kernel.  The gap rows between programs are zeroed in x and in the
  // attention output each call, so they stay exactly zero through every
  // block; the attention kernel reads their V^T columns (with P = 0) as the
  // padding of the program before, so they must be finite even after a
  // refused non-finite step left anything behind in the activations.
  std::vector<Prog*> ps(nprog);
  std::vector<int> start(nprog);
  int rows = 0;
  for (int i = 0; i < nprog; ++i) {
    ps[i] = find_prog(m, keys[i]);
    if (!ps[i]) return fail(QI21_ENOKEY, "no program for key %llu", (unsigned long long)keys[i]);
    if (!xtok[i] || !out[i]) return fail(QI21_EINVAL, "xtok / out %d is NULL", i);
    for (int j = 0; j < i; ++j)
      if (ps[j] == ps[i]) return fail(QI21_EINVAL, "key %llu appears twice", (unsigned long long)keys[i]);
    start[i] = (int)round_up((size_t)rows, 64);
    rows = start[i] + ps[i]->n;
  }
  hipStream_t s = (hipStream_t)stream;
  int rc = ensure_acts(m, rows, s);
  if (rc) return rc;
  const int H = m->g.hidden;
  Acts& a = m->acts;
  const Guard gd = guards(m);
  std::vector<Seg> segs;
  {
    Scope sc(m, C_IO, s);
    HIP_OK(qi21::launch_fill32(m->dflag, 0u, 1, s));
    HIP_OK(qi21::launch_mods(H, mods, a.mods, s));
    for (int i = 0; i < nprog; ++i) {
      segs.push_back(Seg{start[i], ps[i]->n, ps[i], ps[i]->rc, ps[i]->rs, ps[i]->rcs});
      HIP_OK(qi21::launch_embed(ps[i]->n, H, xtok[i], m->img_in, a.x + (size_t)start[i] * H, s));
      if (i > 0) {
        const size_t g0 = (size_t)start[i - 1] + ps[i - 1]->n, gn = (size_t)start[i] - g0;
        HIP_OK(qi21::launch_fill32(a.x + g0 * H, 0u, gn * H, s));
        HIP_OK(qi21::launch_fill32(a.att + g0 * H, 0u, gn * H / 2, s));
      }
    }
  }
  {
    Scope sc(m, C_ROW, s);
    HIP_OK(qi21::launch_rowop(rows, H, 2, a.x, nullptr, a.xn, a.mods, 0, 0, m->g.eps, p2(-gd.attn), s));
  }
  rc = run_blocks(m, rows, segs, nullptr, nullptr, s);
  if (rc) {
    (void)hipStreamSynchronize(s);
    prof_collect(m);
    return rc;
  }
  {
    Scope sc(m, C_IO, s);
    HIP_OK(qi21::launch_final(rows, H, a.x, fs, m->proj_out, m->g.eps, a.out, m->dflag, s));
    for (const Seg& sg : segs)
      HIP_OK(qi21::launch_commit(sg.rows * 64, a.out + (size_t)sg.row0 * 64,
                                 out[&sg - segs.data()], m->dflag, s));
    HIP_OK(hipMemcpyAsync(m->hflag, m->dflag, sizeof(int), hipMemcpyDeviceToHost, s));
  }
  rc = sync_stream(s);
  prof_collect(m);
  if (rc) return rc;
  if (*m->hflag) return fail(QI21_ENONFINITE, "the step produced a non-finite velocity (a range guard overflowed?)");
  return QI21_OK;
}

int qi21_step(qi21_model* m, uint64_t key, const float* xtok, const float* mods, const float* fs, float* out,
              void* stream) {
  return qi21_step_batch(m, 1, &key, &xtok, mods, fs, &out, stream);
}

int qi21_model_set_time(qi21_model* m, int w_dtype, const void* t_lin1, const void* t_lin2, const void* modulation,
                        const void* norm_out, void* stream) {
  g_err.clear();
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (w_dtype < QI21_F32 || w_dtype > QI21_F16) return fail(QI21_EINVAL, "w_dtype %d", w_dtype);
  const void* src[4] = {t_lin1, t_lin2, modulation, norm_out};
  for (int i = 0; i < 4; ++i)
    if (!src[i]) return fail(QI21_EINVAL, "time weight %d is NULL", i);
  hipStream_t s = (hipStream_t)stream;
  const size_t H = m->g.hidden;
  if (!m->tw[0]) {
    for (int i = 0; i < 4; ++i) m->tw[i] = (float*)dalloc(m, time_floats(m->g, i) * 4);
    m->twork = (float*)dalloc(m, (256 + 2 * H) * 4);
    m->tmods = (float*)dalloc(m, 4 * H * 4);
    m->tfs = (float*)dalloc(m, H * 4);
    if (!m->tw[0] || !m->tw[1] || !m->tw[2] || !m->tw[3] || !m->twork || !m->tmods || !m->tfs) {
      free_time(m);
      return fail(QI21_ENOMEM, "time-path weights did not fit");
    }
  }
  for (int i = 0; i < 4; ++i) HIP_OK(qi21::launch_to_f32(w_dtype, src[i], time_floats(m->g, i), m->tw[i], s));
  return sync_stream(s);
}

int qi21_time_mods(qi21_model* m, float t, float* mods, float* fs, void* stream) {
  g_err.clear();
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (!m->tw[0]) return fail(QI21_EINVAL, "no time-path weights (qi21_model_set_time)");
  if (!mods || !fs) return fail(QI21_EINVAL, "mods / fs is NULL");
  if (!std::isfinite(t)) return fail(QI21_EINVAL, "time is not finite");
  HIP_OK(qi21::launch_time_mods(m->g.hidden, t, m->tw[0], m->tw[1], m->tw[2], m->tw[3], m->twork, mods, fs,
                                (hipStream_t)stream));
  return QI21_OK;
}

int qi21_step_t(qi21_model* m, uint64_t key, const float* xtok, float t, float* out, void* stream) {
  int rc = qi21_time_mods(m, t, m ? m->tmods : nullptr, m ? m->tfs : nullptr, stream);
  if (rc) return rc;
  return qi21_step(m, key, xtok, m->tmods, m->tfs, out, stream);
}

int qi21_sample(qi21_model* m, uint64_t key, float* x, int nsteps, const float* t, void* stream) {
  g_err.clear();
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (nsteps < 0 || (nsteps > 0 && (!t || !x))) return fail(QI21_EINVAL, "sample: nsteps %d, t or x NULL", nsteps);
  if (!m->tw[0]) return fail(QI21_EINVAL, "no time-path weights (qi21_model_set_time)");
  Prog* p = find_prog(m, key);
  if (!p) return fail(QI21_ENOKEY, "no program for key %llu", (unsigned long long)key);
  for (int k = 0; k <= nsteps; ++k)
    if (!std::isfinite(t[k])) return fail(QI21_EINVAL, "time %d is not finite", k);
  if (nsteps == 0) return QI21_OK;
  const size_t nv = (size_t)p->n * 64;
  float* v = (float*)dalloc(m, nv * 4);
  if (!v) return fail(QI21_ENOMEM, "sampler velocity buffer");
  int rc = QI21_OK;
  hipStream_t s = (hipStream_t)stream;
  for (int k = 0; k < nsteps && rc == QI21_OK; ++k) {
    rc = qi21_step_t(m, key, x, t[k], v, stream);  // synchronises; x is untouched on failure
    if (rc == QI21_OK) {
      hipError_t e = qi21::launch_axpy((int)nv, t[k + 1] - t[k], v, x, s);
      if (e != hipSuccess) rc = fail(QI21_EDEVICE, "sampler update: %s", hipGetErrorString(e));
    }
  }
  if (rc == QI21_OK) rc = sync_stream(s);
  (void)hipStreamSynchronize(s);
  dfree(m, v, nv * 4);
  return rc;
}

int qi21_model_set_txt_in(qi21_model* m, int context_in, int w_dtype, const float* txt_norm, const void* txt_in1,
                          const void* txt_in2, void* stream) {
  g_err.clear();
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (context_in < 64 || context_in % 64 || context_in > 8192)
    return fail(QI21_EINVAL, "context_in %d (a multiple of 64, at most 8192)", context_in);
  if (w_dtype < QI21_F32 || w_dtype > QI21_F16) return fail(QI21_EINVAL, "w_dtype %d", w_dtype);
  if (!txt_norm || !txt_in1 || !txt_in2) return fail(QI21_EINVAL, "txt_in weight is NULL");
  hipStream_t s = (hipStream_t)stream;
  const size_t H = m->g.hidden, c = context_in;
  if (m->txt_cin != context_in) {
    free_txt(m);
    m->txt_cin = context_in;
    m->txt_norm = (float*)dalloc(m, c * 4);
    m->txt_w1 = (f16*)dalloc(m, H * c * 2);
    m->txt_w2 = (f16*)dalloc(m, H * H * 2);
    if (!m->txt_norm || !m->txt_w1 || !m->txt_w2) {
      free_txt(m);
      return fail(QI21_ENOMEM, "txt_in weights did not fit");
    }
  }
  HIP_OK(hipMemcpyAsync(m->txt_norm, txt_norm, c * 4, hipMemcpyDeviceToDevice, s));
  HIP_OK(qi21::launch_plane(w_dtype, txt_in1, (int)H, (int)c, m->txt_w1, (int)H, 0, 0, s));
  HIP_OK(qi21::launch_plane(w_dtype, txt_in2, (int)H, (int)H, m->txt_w2, (int)H, 0, 0, s));
  return sync_stream(s);
}

int qi21_txt_in(qi21_model* m, int n, const float* feats, float* out, void* stream) {
  g_err.clear();
  int rc = txt_in_check(m, n, feats, out);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int H = m->g.hidden, c = m->txt_cin;
  if (m->txt_cap < n) {
    HIP_OK(hipStreamSynchronize(s));  // earlier calls may still use the buffers
    free_txt_rows(m);
    const int cap = (int)round_up((size_t)n, 256);
    m->txt_xn = (f16*)dalloc(m, (size_t)cap * c * 2);
    m->txt_h = (f16*)dalloc(m, (size_t)cap * H * 2);
    if (!m->txt_xn || !m->txt_h) {
      free_txt_rows(m);
      return fail(QI21_ENOMEM, "txt_in rows for %d rows", n);
    }
    m->txt_cap = cap;
  }
  return txt_in_run(m, n, feats, out, m->txt_xn, m->txt_h, s);
}

int qi21_release_key(qi21_model* m, uint64_t key) {
  g_err.clear();
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  for (auto it = m->progs.begin(); it != m->progs.end(); ++it)
    if (it->key == key) {
      (void)hipDeviceSynchronize();
      free_prog(m, *it);
      m->progs.erase(it);
      return QI21_OK;
    }
  return fail(QI21_ENOKEY, "no program for key %llu", (unsigned long long)key);
}

int qi21_set_profile(qi21_model* m, int class_mask) {
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  m->o.profile = class_mask;
  return QI21_OK;
}

int qi21_set_profile_every(qi21_model* m, int every) {
  if (!m) return fail(QI21_EINVAL, "model is NULL");
  if (every < 1) return fail(QI21_EINVAL, "profile sampling every %d (>= 1)", every);
  m->prof.every = every;
  for (int64_t& c : m->prof.seen) c = 0;
  return QI21_OK;
}

int qi21_profile_read(qi21_model* m, double* ms, int64_t* launches) {
  if (!m || !ms || !launches) return fail(QI21_EINVAL, "NULL argument");
  for (int c = 0; c < NCLASS; ++c) {
    ms[c] = m->prof.ms[c];
    launches[c] = m->prof.n[c];
    m->prof.ms[c] = 0.0;
    m->prof.n[c] = 0;
  }
  return QI21_OK;
}

// ───────────────────────────── single-kernel entry points ─────────────────────────────

namespace {
// shared checks of the two GEMM entry points; ka = the columns of A read
int op_gemm(int epi, int M, int N, int K, int ka, const void* A, int lda, const void* W, void* out, int ldo,
            void* out2, int ld2, float oscale, float inscale, int tile, void* stream) {
  if (epi < QI21_EPI_F16 || epi > QI21_EPI_SWIGLU2) return fail(QI21_EINVAL, "epilogue %d", epi);
  if (M < 1 || N < 128 || K < 64 || N % 128 || K % 64 || lda % 8 || lda < ka || ldo % 4)
    return fail(QI21_EINVAL, "gemm M %d N %d K %d lda %d ldo %d (need N %% 128, K %% 64, lda %% 8, lda >= %d, ldo %% 4)",
                M, N, K, lda, ldo, ka);
  if (!A || !W || !out) return fail(QI21_EINVAL, "gemm pointer is NULL");
  const int ocols = epi == QI21_EPI_SWIGLU ? N / 2 : epi == QI21_EPI_QKV ? 2 * N / 3 : N;
  if (ldo < ocols) return fail(QI21_EINVAL, "ldo %d < %d output columns", ldo, ocols);
  // f16 rows of the row-layout epilogues are written in 16-byte vectors
  if (epi != QI21_EPI_F32 && epi != QI21_EPI_QKV && ldo % 8)
    return fail(QI21_EINVAL, "ldo %d: f16 output rows need ldo %% 8 == 0", ldo);
  if (epi == QI21_EPI_QKV && ((N / 3) % 128 || N % 3 || !out2 || ld2 % 4 || ld2 < M))
    return fail(QI21_EINVAL, "qkv epilogue needs N/3 %% 128 == 0, out2, ld2 %% 4 == 0, ld2 >= M");
  if (tile < -1 || tile > 2 || (tile != 1 && tile != -1 && N % 256)) return fail(QI21_EINVAL, "tile %d for N %d", tile, N);
  qi21::GemmArgs a = gemm_args(M, N, ka, (const f16*)A, lda, (const f16*)W, out, ldo, oscale, inscale, (f16*)out2, ld2);
  a.kw = K;
  HIP_OK(qi21::launch_gemm(epi, a, tile, (hipStream_t)stream));
  return QI21_OK;
}
}  // namespace

int qi21_op_gemm(int epi, int M, int N, int K, const void* A, int lda, const void* W, void* out, int ldo, void* out2,
                 int ld2, float oscale, float inscale, int tile, void* stream) {
  g_err.clear();
  return op_gemm(epi, M, N, K, K, A, lda, W, out, ldo, out2, ld2, oscale, inscale, tile, stream);
}

int qi21_op_gemm_pair(int epi, int M, int N, int K, const void* A, int lda, const void* W, void* out, int ldo,
                      float oscale, float inscale, int tile, void* stream) {
  g_err.clear();
  if (epi == QI21_EPI_QKV) return fail(QI21_EINVAL, "the pair GEMM has no qkv epilogue");
  return op_gemm(epi, M, N, K, 2 * K, A, lda, W, out, ldo, nullptr, 0, oscale, inscale, tile, stream);
}

int qi21_op_gemm_resid(int M, int N, int K, int kw, const void* A, int lda, const void* W, float* x, int ldx,
                       const float* gate, float oscale, int tile, void* stream) {
  g_err.clear();
  if (kw < 64 || kw % 64 || (K != kw && K != 2 * kw)) return fail(QI21_EINVAL, "resid gemm K %d kw %d", K, kw);
  if (!gate) return fail(QI21_EINVAL, "resid gemm gate is NULL");
  if (M < 1 || N < 128 || N % 128 || lda % 8 || lda < K || ldx % 4 || ldx < N)
    return fail(QI21_EINVAL, "resid gemm M %d N %d lda %d ldx %d", M, N, lda, ldx);
  if (!A || !W || !x) return fail(QI21_EINVAL, "resid gemm pointer is NULL");
  if (tile < -1 || tile > 2 || (tile != 1 && tile != -1 && N % 256)) return fail(QI21_EINVAL, "tile %d for N %d", tile, N);
  qi21::GemmArgs a = gemm_args(M, N, K, (const f16*)A, lda, (const f16*)W, x, ldx, oscale);
  a.kw = kw;
  a.gate = gate;
  HIP_OK(qi21::launch_gemm(qi21::EPI_RESID, a, tile, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_gemm_split(int M, int N, int K, int kw, const void* A, int lda, const void* W, float* part, int ksplit,
                       float oscale, int tile, void* stream) {
  g_err.clear();
  if (ksplit < 1 || ksplit > 8) return fail(QI21_EINVAL, "split gemm ksplit %d (1..8)", ksplit);
  if (kw < 64 || kw % 64 || (K != kw && K != 2 * kw) || K % (64 * ksplit))
    return fail(QI21_EINVAL, "split gemm K %d kw %d ksplit %d", K, kw, ksplit);
  if (M < 1 || N < 256 || N % 256 || lda % 8 || lda < K) return fail(QI21_EINVAL, "split gemm M %d N %d lda %d", M, N, lda);
  if (!A || !W || !part) return fail(QI21_EINVAL, "split gemm pointer is NULL");
  if (tile == -1) tile = 0;
  if (tile != 0 && tile != 2) return fail(QI21_EINVAL, "split gemm tile %d (0 or 2)", tile);
  qi21::GemmArgs a = gemm_args(M, N, K, (const f16*)A, lda, (const f16*)W, part, N, oscale);
  a.kw = kw;
  a.ksplit = ksplit;
  a.pstride = (size_t)M * N;
  HIP_OK(qi21::launch_gemm(qi21::EPI_F32, a, tile, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_rope_pack(int n, const float* cos, const float* sin, float* out, void* stream) {
  g_err.clear();
  if (n < 1) return fail(QI21_EINVAL, "rope pack n %d", n);
  if (!cos || !sin || !out) return fail(QI21_EINVAL, "rope pack pointer NULL");
  HIP_OK(qi21::launch_rope_pack(n, cos, sin, out, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_qk_gemm(int M, int H, const void* A, int lda, const void* W, void* q_out, int ldq, void* k_out, int ldk,
                    const float* norm_q, const float* norm_k, const float* rope, float eps, int tile, void* stream) {
  g_err.clear();
  if (M < 1 || H < 128 || H % 128 || lda % 8 || lda < H || ldq % 8 || ldk % 8 || ldq < H || ldk < H)
    return fail(QI21_EINVAL, "qk gemm M %d H %d lda %d ldq %d ldk %d", M, H, lda, ldq, ldk);
  if (!A || !W || !q_out || !k_out || !norm_q || !norm_k || !rope) return fail(QI21_EINVAL, "qk gemm pointer NULL");
  if (tile == -1) tile = 0;
  if (tile != 0 && tile != 2) return fail(QI21_EINVAL, "qk gemm tile %d (0 or 2)", tile);
  qi21::GemmArgs a = gemm_args(M, 2 * H, H, (const f16*)A, lda, (const f16*)W, q_out, ldq, 1.0f);
  a.nq = norm_q;
  a.nk = norm_k;
  a.rope = rope;
  a.eps = eps;
  a.kout = (f16*)k_out;
  a.ldk = ldk;
  HIP_OK(qi21::launch_gemm(qi21::EPI_QKROPE, a, tile, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_vt_gemm(int H, int nkeys, int K, const void* Wv, int lda, const void* X, void* out, int ldo, float oscale,
                    int tile, void* stream) {
  g_err.clear();
  if (H < 1 || nkeys < 1 || K < 64 || K % 64 || lda % 8 || lda < K || ldo % 8 || (size_t)ldo < round_up(nkeys, 16))
    return fail(QI21_EINVAL, "vt gemm H %d nkeys %d K %d lda %d ldo %d", H, nkeys, K, lda, ldo);
  if (!Wv || !X || !out) return fail(QI21_EINVAL, "vt gemm pointer NULL");
  if (tile == -1) tile = 0;
  if (tile != 0 && tile != 2) return fail(QI21_EINVAL, "vt gemm tile %d (0 or 2)", tile);
  qi21::GemmArgs a = gemm_args(H, (int)round_up(nkeys, 256), K, (const f16*)Wv, lda, (const f16*)X, out, ldo, oscale);
  a.nvalid = nkeys;
  HIP_OK(qi21::launch_gemm(qi21::EPI_VT, a, tile, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_flash(int nq, int heads, const void* q, int ldq, const void* k1, int ldk1, const void* vt1, int ldvt1,
                  int n1, const void* k2, int ldk2, const void* vt2, int ldvt2, int n2, const uint32_t* vis, void* out,
                  int ldo, float oscale, void* stream) {
  g_err.clear();
  if (nq < 1 || heads < 1 || n1 < 0 || n2 < 0 || n1 + n2 < 1) return fail(QI21_EINVAL, "flash sizes");
  if (!q || !out || (n1 && (!k1 || !vt1)) || (n2 && (!k2 || !vt2))) return fail(QI21_EINVAL, "flash pointer NULL");
  if (ldq % 8 || ldo % 4 || ldq < heads * 128 || ldo < heads * 128) return fail(QI21_EINVAL, "flash ldq / ldo");
  if (n1 && (ldk1 % 8 || ldvt1 % 8 || ldk1 < heads * 128 || (size_t)ldvt1 < round_up(n1, 64)))
    return fail(QI21_EINVAL, "flash source 1 leading dimensions");
  if (n2 && (ldk2 % 8 || ldvt2 % 8 || ldk2 < heads * 128 || (size_t)ldvt2 < round_up(n2, 64)))
    return fail(QI21_EINVAL, "flash source 2 leading dimensions");
  qi21::FlashArgs f{};
  f.q = (const f16*)q;
  f.ldq = ldq;
  f.nq = nq;
  f.heads = heads;
  f.k1 = (const f16*)k1;
  f.ldk1 = ldk1;
  f.vt1 = (const f16*)vt1;
  f.ldvt1 = ldvt1;
  f.n1 = n1;
  f.k2 = (const f16*)k2;
  f.ldk2 = ldk2;
  f.vt2 = (const f16*)vt2;
  f.ldvt2 = ldvt2;
  f.n2 = n2;
  f.vis = vis;
  f.out = (f16*)out;
  f.ldo = ldo;
  f.oscale = oscale;
  HIP_OK(qi21::launch_flash(f, (hipStream_t)stream));
  return QI21_OK;
}

namespace {
// shared checks of the row-op entry points; fmt: QI21_FFN_LO8 / LO4 for
// the residual FFN-input forms, 0 for the f16 forms
int op_rowop(int rows, int h, int mode, float* x, const float* y, int nparts, size_t pstride, void* xn, int ldxn,
             uint8_t* xsc, const float* mods, int g_off, int s_off, float eps, float oscale, void* stream, int fmt) {
  if (nparts < 1 || nparts > 8 || (nparts > 1 && pstride < (size_t)rows * h))
    return fail(QI21_EINVAL, "rowop nparts %d pstride %zu", nparts, pstride);
  const bool lo = fmt == QI21_FFN_LO8 || fmt == QI21_FFN_LO4;
  if (fmt != 0 && !lo) return fail(QI21_EINVAL, "rowop format %d (QI21_FFN_LO8 or QI21_FFN_LO4)", fmt);
  const bool mode_ok = lo ? (mode == 2 || mode == 3) : (mode >= 1 && mode <= 7 && mode != 4 && mode != 5);
  if (rows < 1 || h < 4 || h % 4 || h > 8192 || !mode_ok || g_off % 4 || s_off % 4 || g_off < 0 || s_off < 0)
    return fail(QI21_EINVAL, "rowop rows %d h %d mode %d", rows, h, mode);
  if (!x || !mods || ((mode & 1) && !y) || ((mode & 2) && !xn) || (lo && !xsc))
    return fail(QI21_EINVAL, "rowop pointer NULL");
  const int hm = fmt == QI21_FFN_LO4 ? 256 : 128;
  if (lo && h % hm) return fail(QI21_EINVAL, "rowop %s h %d (a multiple of %d)", fmt == QI21_FFN_LO8 ? "lo8" : "lo4", h, hm);
  // the row stride xn needs: h, 2h for the pair form, 1.5h (lo8) or 1.25h (lo4), in halves
  const long need = fmt == QI21_FFN_LO8 ? 3L * h / 2 : fmt == QI21_FFN_LO4 ? 5L * h / 4 : (mode & 4) ? 2L * h : h;
  if ((mode & 2) && (ldxn < need || ldxn % 4))
    return fail(QI21_EINVAL, "rowop ldxn %d (at least %ld halves for mode %d, a multiple of 4)", ldxn, need, mode);
  const int bits = fmt == QI21_FFN_LO8 ? 8 : fmt == QI21_FFN_LO4 ? 16 : 0;
  HIP_OK(qi21::launch_rowop(rows, h, mode | bits, x, y, (f16*)xn, mods, g_off, s_off, eps, oscale, (hipStream_t)stream,
                            nparts, pstride, xsc, (mode & 2) ? ldxn : h));
  return QI21_OK;
}
}  // namespace

int qi21_op_rowop(int rows, int h, int mode, float* x, const float* y, void* xn, int ldxn, const float* mods,
                  int g_off, int s_off, float eps, float oscale, void* stream) {
  g_err.clear();
  return op_rowop(rows, h, mode, x, y, 1, 0, xn, ldxn, nullptr, mods, g_off, s_off, eps, oscale, stream, 0);
}

int qi21_op_rowop_parts(int rows, int h, int mode, float* x, const float* y, int nparts, size_t pstride, void* xn,
                        int ldxn, const float* mods, int g_off, int s_off, float eps, float oscale, void* stream) {
  g_err.clear();
  return op_rowop(rows, h, mode, x, y, nparts, pstride, xn, ldxn, nullptr, mods, g_off, s_off, eps, oscale, stream, 0);
}

int qi21_op_rowop_lo(int fmt, int rows, int h, int mode, float* x, const float* y, int nparts, size_t pstride,
                     void* xn, int ldxn, uint8_t* xsc, const float* mods, int g_off, int s_off, float eps,
                     float oscale, void* stream) {
  g_err.clear();
  if (fmt != QI21_FFN_LO8 && fmt != QI21_FFN_LO4) return fail(QI21_EINVAL, "rowop format %d", fmt);
  return op_rowop(rows, h, mode, x, y, nparts, pstride, xn, ldxn, xsc, mods, g_off, s_off, eps, oscale, stream, fmt);
}

int qi21_op_gemm_lo(int fmt, int epi, int M, int N, int K, const void* A, int lda, const uint8_t* asc, const void* W,
                    int ldw, const uint8_t* wsc, void* out, int ldo, const float* gate, uint8_t* osc, int ksplit,
                    float oscale, float inscale, void* stream) {
  g_err.clear();
  const bool l8 = fmt == QI21_FFN_LO8;
  if (!l8 && fmt != QI21_FFN_LO4) return fail(QI21_EINVAL, "gemm format %d (QI21_FFN_LO8 or QI21_FFN_LO4)", fmt);
  const int sw = l8 ? QI21_EPI_SWIGLU8 : QI21_EPI_SWIGLU4;
  if (epi != QI21_EPI_F32 && epi != QI21_EPI_RESID && epi != sw)
    return fail(QI21_EINVAL, "residual gemm epilogue %d (F32, RESID or the format's SWIGLU)", epi);
  const int g = l8 ? 128 : 256;                    // columns per group
  const long krow = l8 ? 3L * K / 2 : 5L * K / 4;  // halves per row
  if (M < 1 || N < 256 || N % 256 || K < g || K % g || lda % 8 || ldw % 8 || lda < krow || ldw < krow)
    return fail(QI21_EINVAL,
                "residual gemm M %d N %d K %d lda %d ldw %d (need N %% 256, K %% %d, lda and ldw >= %ld and %% 8)", M, N,
                K, lda, ldw, g, krow);
  if (!A || !W || !asc || !wsc || !out) return fail(QI21_EINVAL, "residual gemm pointer is NULL");
  if (ksplit < 1 || ksplit > 8 || (K / g) % ksplit || (ksplit > 1 && epi != QI21_EPI_F32))
    return fail(QI21_EINVAL, "residual gemm ksplit %d (1..8, dividing K / %d; F32 only)", ksplit, g);
  if (epi == QI21_EPI_RESID && (!gate || ldo < N || ldo % 4)) return fail(QI21_EINVAL, "residual gemm resid gate / ldo %d", ldo);
  if (epi == QI21_EPI_F32 && (ldo < N || ldo % 4 || (ksplit > 1 && ldo != N)))
    return fail(QI21_EINVAL, "residual gemm f32 ldo %d (>= N, %% 4; = N when split)", ldo);
  const long hrow = l8 ? 3L * N / 4 : 5L * N / 8;  // halves of an output row of N/2 columns
  if (epi == sw && (!osc || ldo < hrow || ldo % 8 || (N / 2) % g))
    return fail(QI21_EINVAL, "residual gemm swiglu ldo %d (>= %ld, %% 8), osc, N / 2 %% %d", ldo, hrow, g);
  qi21::GemmArgs a = gemm_args(M, N, (int)krow, (const f16*)A, lda, (const f16*)W, out, ldo, oscale, inscale);
  a.ldw = ldw;
  a.lo = l8 ? 8 : 4;
  a.asc = asc;
  a.lds = l8 ? K / 64 : K / 32;
  a.wsc = wsc;
  a.ldws = l8 ? 0 : K / 32;
  a.gate = gate;
  a.osc = osc;
  a.ksplit = ksplit;
  a.pstride = (size_t)M * N;
  HIP_OK(qi21::launch_gemm(epi, a, 0, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_plane_lo(int fmt, int src_dtype, const void* src, int rows, int cols, void* dst, int ld, int group,
                     int gstride, int goff, void* stream) {
  g_err.clear();
  const bool l8 = fmt == QI21_FFN_LO8;
  if (!l8 && fmt != QI21_FFN_LO4) return fail(QI21_EINVAL, "plane format %d", fmt);
  const int g = l8 ? 128 : 256;
  const long need = l8 ? 3L * cols / 2 : 5L * cols / 4;
  if (src_dtype < QI21_F32 || src_dtype > QI21_F16 || rows < 1 || cols < g || cols % g || ld < need || ld % 4 ||
      group < 1 || gstride < 0 || goff < 0 || !src || !dst)
    return fail(QI21_EINVAL, "residual plane arguments (cols %% %d, ld >= %ld and %% 4)", g, need);
  HIP_OK(qi21::launch_plane(src_dtype, src, rows, cols, (f16*)dst, group, gstride, goff, (hipStream_t)stream, ld,
                            l8 ? 8 : 4));
  return QI21_OK;
}

int qi21_op_plane_lo_fill(int fmt, int rows, int cols, void* plane, int ld, uint8_t* sc, void* stream) {
  g_err.clear();
  const bool l8 = fmt == QI21_FFN_LO8;
  if (!l8 && fmt != QI21_FFN_LO4) return fail(QI21_EINVAL, "plane format %d", fmt);
  const int g = l8 ? 128 : 256;
  const long need = l8 ? 3L * cols / 2 : 5L * cols / 4;
  if (rows < 1 || cols < g || cols % g || ld < need || ld % 4 || !plane || !sc)
    return fail(QI21_EINVAL, "residual plane fill rows %d cols %d ld %d", rows, cols, ld);
  if (l8)
    HIP_OK(qi21::launch_plane8(rows, cols, (f16*)plane, ld, sc, (hipStream_t)stream));
  else
    HIP_OK(qi21::launch_plane4(rows, cols, (f16*)plane, ld, sc, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_qkrope(int rows, int heads, void* panel, int ldp, const float* norm_q, const float* norm_k,
                   const float* cos, const float* sin, float eps, void* kdst, int ldk, void* stream) {
  g_err.clear();
  if (rows < 1 || heads < 1 || ldp < 2 * heads * 128 || ldp % 2 || (kdst && (ldk < heads * 128 || ldk % 2)))
    return fail(QI21_EINVAL, "qkrope rows %d heads %d ldp %d", rows, heads, ldp);
  if (!panel || !norm_q || !norm_k || !cos || !sin) return fail(QI21_EINVAL, "qkrope pointer NULL");
  HIP_OK(qi21::launch_qkrope(rows, heads, (f16*)panel, ldp, norm_q, norm_k, cos, sin, eps, (f16*)kdst, ldk,
                             (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_embed(int rows, int h, const float* tok, const float* img_in, float* x, void* stream) {
  g_err.clear();
  if (rows < 1 || h < 64 || h % 64 || !tok || !img_in || !x) return fail(QI21_EINVAL, "embed rows %d h %d", rows, h);
  HIP_OK(qi21::launch_embed(rows, h, tok, img_in, x, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_final(int rows, int h, const float* x, const float* fs, const float* proj_out, float eps, float* out,
                  int* flag, void* stream) {
  g_err.clear();
  if (rows < 1 || h < 256 || h % 256 || !x || !fs || !proj_out || !out || !flag)
    return fail(QI21_EINVAL, "final rows %d h %d", rows, h);
  HIP_OK(qi21::launch_final(rows, h, x, fs, proj_out, eps, out, flag, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_mods(int h, const float* mods, float* mods_dev, void* stream) {
  g_err.clear();
  if (h < 1 || h > 65536 || !mods || !mods_dev) return fail(QI21_EINVAL, "mods h %d", h);
  HIP_OK(qi21::launch_mods(h, mods, mods_dev, (hipStream_t)stream));
  return QI21_OK;
}

int qi21_op_plane(int src_dtype, const void* src, int rows, int cols, void* dst, int group, int gstride, int goff,
                  void* stream) {
  g_err.clear();
  if (src_dtype < QI21_F32 || src_dtype > QI21_F16 || rows < 1 || cols < 1 || group < 1 || gstride < 0 || goff < 0 ||
      !src || !dst)
    return fail(QI21_EINVAL, "plane arguments");
  HIP_OK(qi21::launch_plane(src_dtype, src, rows, cols, (f16*)dst, group, gstride, goff, (hipStream_t)stream));
  return QI21_OK;
}

}  // extern "C"
