// Host-only checks of the qi21 library's host logic (layout helpers, the
// model's creation, refusal and allocation-failure paths, the op entry
// points' shape validation, the launch-shape choices), built with address
// and undefined-behaviour sanitizers and linked against stand-ins for the
// device launchers.  Every call here must finish before any device work:
// a refused shape, a failed allocation, a null argument.  Exit status 0
// when every check holds; a sanitizer report ends the run with an error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "qi21.h"
#include "qi21_ops.h"
#include "qi21_internal.h"

namespace {

int g_fail = 0, g_checks = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      ++g_fail;                                                              \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
    }                                                                        \
  } while (0)

// a status and a non-empty explanation
void expect(int rc, int want, const char* what) {
  ++g_checks;
  const char* e = qi21_last_error();
  if (rc != want || !e || !*e) {
    ++g_fail;
    std::fprintf(stderr, "%s: status %d (want %d), error '%s'\n", what, rc, want, e ? e : "(null)");
  }
}

// made-up, never dereferenced device addresses
void* fake(int i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(0x7e0000000000ull + (uint64_t)i * 0x100000)); }

void layout_checks() {
  // the text + image layout of the step: 18 text rows, a 16 x 16 target
  const qi21_seg a[2] = {{0, 18, 0}, {1, 16, 16}};
  int32_t lp = -1, n = -1;
  CHECK(qi21_layout_sizes(a, 2, &lp, &n) == QI21_OK && lp == 18 && n == 256);
  CHECK(qi21_last_error()[0] == 0);
  // a condition image between two text runs, then the target
  const qi21_seg b[4] = {{0, 5, 0}, {1, 3, 4}, {0, 2, 0}, {1, 9, 7}};
  CHECK(qi21_layout_sizes(b, 4, &lp, &n) == QI21_OK && lp == 19 && n == 63);
  const int32_t axes[3] = {16, 56, 56};
  const int total = lp + n;
  std::vector<int64_t> pos((size_t)total * 3, -7);
  std::vector<uint32_t> vis(lp, 0);
  std::vector<float> cp((size_t)lp * 64), sp((size_t)lp * 64), ct((size_t)n * 64), st((size_t)n * 64);
  CHECK(qi21_layout_tables(b, 4, axes, 10000.f, pos.data(), vis.data(), cp.data(), sp.data(), ct.data(), st.data()) ==
        QI21_OK);
  for (int i = 1; i < lp; ++i) CHECK(vis[i] >= vis[i - 1] && vis[i] >= 1 && (int)vis[i] <= lp);
  CHECK(vis[0] == 1 && vis[4] == 5);      // text rows see themselves and what came before
  CHECK(vis[5] == 17 && vis[16] == 17);   // the condition image sees to its own end
  for (size_t i = 0; i < pos.size(); ++i) CHECK(pos[i] != -7);
  // position 0 has angle 0 on every axis
  bool unit = true;
  for (int c = 0; c < 64; ++c) unit = unit && cp[c] == 1.f && sp[c] == 0.f;
  CHECK(unit);
  // any subset of the outputs
  CHECK(qi21_layout_tables(b, 4, axes, 10000.f, nullptr, vis.data(), nullptr, nullptr, nullptr, nullptr) == QI21_OK);
  CHECK(qi21_layout_tables(b, 4, axes, 10000.f, pos.data(), nullptr, nullptr, nullptr, ct.data(), st.data()) == QI21_OK);

  const qi21_seg text_last[2] = {{1, 2, 2}, {0, 3, 0}};
  const qi21_seg empty_img[2] = {{0, 3, 0}, {1, 0, 5}};
  const qi21_seg neg[2] = {{0, -3, 0}, {1, 2, 2}};
  const qi21_seg huge[2] = {{0, 4, 0}, {1, 1 << 20, 1 << 20}};
  const qi21_seg bad_kind[2] = {{7, 3, 0}, {1, 2, 2}};
  const qi21_seg only_img[1] = {{1, 4, 4}};
  expect(qi21_layout_sizes(nullptr, 2, &lp, &n), QI21_EINVAL, "null segments");
  expect(qi21_layout_sizes(a, 0, &lp, &n), QI21_EINVAL, "no segments");
  expect(qi21_layout_sizes(text_last, 2, &lp, &n), QI21_EINVAL, "text last");
  expect(qi21_layout_sizes(empty_img, 2, &lp, &n), QI21_EINVAL, "empty target image");
  expect(qi21_layout_sizes(neg, 2, &lp, &n), QI21_EINVAL, "negative run");
  expect(qi21_layout_sizes(huge, 2, &lp, &n), QI21_EINVAL, "target past int32");
  expect(qi21_layout_sizes(bad_kind, 2, &lp, &n), QI21_EINVAL, "unknown run kind");
  expect(qi21_layout_sizes(only_img, 1, &lp, &n), QI21_EINVAL, "empty prefix");
  const int32_t odd[3] = {15, 57, 56}, zero[3] = {0, 64, 64};
  expect(qi21_layout_tables(a, 2, odd, 10000.f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), QI21_EINVAL,
         "odd axis");
  expect(qi21_layout_tables(a, 2, zero, 10000.f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), QI21_EINVAL,
         "empty axis");
  expect(qi21_layout_tables(a, 2, nullptr, 10000.f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), QI21_EINVAL,
         "no axes");
  // a narrower head: the tables are [rows][sum of axes / 2]
  const int32_t narrow[3] = {8, 28, 28};
  std::vector<float> cn((size_t)18 * 32), sn((size_t)18 * 32);
  CHECK(qi21_layout_tables(a, 2, narrow, 10000.f, nullptr, nullptr, cn.data(), sn.data(), nullptr, nullptr) == QI21_OK);
}

qi21_geom geom(int hidden = 256, int heads = 2, int inter = 768) {
  qi21_geom g{};
  g.hidden = hidden;
  g.heads = heads;
  g.head_dim = 128;
  g.inter = inter;
  g.in_ch = 64;
  g.eps = 1e-6f;
  return g;
}

// An allocator hook that hands out made-up addresses and refuses request
// number fail_at; it records every block so that none may be lost or freed
// twice.
struct Pool {
  int fail_at = -1, calls = 0;
  std::vector<std::pair<void*, size_t>> live;
  int bad_frees = 0;
};

void* pool_alloc(size_t bytes, void* ctx) {
  Pool* p = static_cast<Pool*>(ctx);
  const int i = p->calls++;
  if (i == p->fail_at) return nullptr;
  void* a = fake(1000 + i);
  p->live.push_back({a, bytes});
  return a;
}

void pool_free(void* ptr, void* ctx) {
  Pool* p = static_cast<Pool*>(ctx);
  for (size_t i = 0; i < p->live.size(); ++i)
    if (p->live[i].first == ptr) {
      p->live.erase(p->live.begin() + (long)i);
      return;
    }
  ++p->bad_frees;
}

void model_checks() {
  qi21_model* m = reinterpret_cast<qi21_model*>(fake(1));
  const qi21_geom g = geom();
  expect(qi21_model_create(&g, nullptr, 2, (float*)fake(2), (float*)fake(3), nullptr, nullptr), QI21_EINVAL,
         "null out");
  expect(qi21_model_create(nullptr, nullptr, 2, (float*)fake(2), (float*)fake(3), nullptr, &m), QI21_EINVAL,
         "null geometry");
  CHECK(m == nullptr);  // out is cleared before anything else is looked at
  const qi21_geom bad[5] = {geom(256, 3), geom(256, 2, 100), geom(16384, 128), geom(0, 0, 768), geom(-256, -2, 768)};
  for (const auto& b : bad) {
    const int rc = qi21_model_create(&b, nullptr, 2, (float*)fake(2), (float*)fake(3), nullptr, &m);
    CHECK(rc == QI21_EUNSUPPORTED || rc == QI21_EINVAL);
    CHECK(m == nullptr && qi21_last_error()[0] != 0);
  }
  expect(qi21_model_create(&g, nullptr, 0, (float*)fake(2), (float*)fake(3), nullptr, &m), QI21_EINVAL, "no blocks");
  expect(qi21_model_create(&g, nullptr, 2, nullptr, (float*)fake(3), nullptr, &m), QI21_EINVAL, "null img_in");

  qi21_options o;
  qi21_default_options(&o);
  Pool half;
  o.alloc = pool_alloc;
  o.alloc_ctx = &half;
  expect(qi21_model_create(&g, &o, 2, (float*)fake(2), (float*)fake(3), nullptr, &m), QI21_EINVAL, "alloc, no free");
  CHECK(half.calls == 0);
  o.ffn_mode = 9;
  o.free = pool_free;
  expect(qi21_model_create(&g, &o, 2, (float*)fake(2), (float*)fake(3), nullptr, &m), QI21_EINVAL, "ffn_mode 9");

  // every request of qi21_model_create refused in turn, for each FFN form:
  // ENOMEM, nothing asked after the refusal, every earlier block handed back
  const int modes[4] = {QI21_FFN_F16, QI21_FFN_PAIR, QI21_FFN_LO8, QI21_FFN_LO4};
  for (int mode : modes) {
    const int nb = 3;
    const int per_block = 6 + ((mode == QI21_FFN_LO8 || mode == QI21_FFN_LO4) ? 2 : 0);
    const int total = nb * per_block + 3;
    for (int k = 0; k < total; ++k) {
      Pool p;
      p.fail_at = k;
      qi21_default_options(&o);
      o.ffn_mode = mode;
      o.alloc = pool_alloc;
      o.free = pool_free;
      o.alloc_ctx = &p;
      m = nullptr;
      const int rc = qi21_model_create(&g, &o, nb, (float*)fake(2), (float*)fake(3), nullptr, &m);
      ++g_checks;
      if (rc != QI21_ENOMEM || m != nullptr || p.calls != k + 1 || !p.live.empty() || p.bad_frees ||
          !std::strstr(qi21_last_error(), "did not fit")) {
        ++g_fail;
        std::fprintf(stderr, "ffn_mode %d, request %d refused: status %d, %d requests, %zu blocks kept, %d bad frees, '%s'\n",
                     mode, k, rc, p.calls, p.live.size(), p.bad_frees, qi21_last_error());
      }
    }
  }

  // null-model calls
  float* f = (float*)fake(5);
  uint64_t key = 1;
  const float* xs[1] = {f};
  float* outs[1] = {f};
  expect(qi21_model_set_block(nullptr, 0, QI21_F32, nullptr, f, f, nullptr), QI21_EINVAL, "set_block null model");
  expect(qi21_prefill(nullptr, 1, 4, 4, f, f, f, f, f, (uint32_t*)fake(6), f, nullptr), QI21_EINVAL, "prefill null model");
  expect(qi21_step(nullptr, 1, f, f, f, f, nullptr), QI21_EINVAL, "step null model");
  expect(qi21_step_batch(nullptr, 1, &key, xs, f, f, outs, nullptr), QI21_EINVAL, "step_batch null model");
  expect(qi21_txt_in(nullptr, 4, f, f, nullptr), QI21_EINVAL, "txt_in null model");
  expect(qi21_time_mods(nullptr, 0.5f, f, f, nullptr), QI21_EINVAL, "time_mods null model");
  expect(qi21_sample(nullptr, 1, f, 2, f, nullptr), QI21_EINVAL, "sample null model");
  double ms[8];
  int64_t launches[8];
  expect(qi21_profile_read(nullptr, ms, launches), QI21_EINVAL, "profile_read null model");
  CHECK(qi21_release_key(nullptr, 1) != QI21_OK);
  CHECK(qi21_model_bytes(nullptr) == 0);
  qi21_model_destroy(nullptr);
}

void op_checks() {
  void* p = fake(7);
  float* f = (float*)fake(8);
  uint8_t* b = (uint8_t*)fake(9);
  expect(qi21_op_gemm(0, 16, 100, 64, p, 64, p, p, 100, nullptr, 0, 1.f, 1.f, -1, nullptr), QI21_EINVAL, "gemm N % 128");
  expect(qi21_op_gemm(0, 16, 128, 60, p, 64, p, p, 128, nullptr, 0, 1.f, 1.f, -1, nullptr), QI21_EINVAL, "gemm K % 64");
  expect(qi21_op_gemm(0, 16, 128, 64, p, 60, p, p, 128, nullptr, 0, 1.f, 1.f, -1, nullptr), QI21_EINVAL, "gemm lda");
  expect(qi21_op_gemm(3, 16, 384, 64, p, 64, p, p, 256, nullptr, 0, 1.f, 1.f, -1, nullptr), QI21_EINVAL, "qkv no out2");
  expect(qi21_op_gemm(5, 16, 128, 64, p, 64, p, p, 128, nullptr, 0, 1.f, 1.f, -1, nullptr), QI21_EINVAL, "epilogue 5");
  expect(qi21_op_gemm(0, -1, 128, 64, p, 64, p, p, 128, nullptr, 0, 1.f, 1.f, -1, nullptr), QI21_EINVAL, "gemm M < 0");
  expect(qi21_op_gemm_pair(1, 16, 128, 64, p, 100, p, p, 128, 1.f, 1.f, -1, nullptr), QI21_EINVAL, "pair lda");
  expect(qi21_op_gemm_split(16, 256, 192, 192, p, 192, p, f, 2, 1.f, -1, nullptr), QI21_EINVAL, "split K");
  expect(qi21_op_gemm_split(16, 256, 256, 256, p, 256, p, f, 9, 1.f, -1, nullptr), QI21_EINVAL, "split 9");
  expect(qi21_op_gemm_resid(16, 128, 64, 64, p, 64, p, nullptr, 128, f, 1.f, -1, nullptr), QI21_EINVAL, "resid no x");
  expect(qi21_op_qk_gemm(16, 200, p, 256, p, p, 256, p, 256, f, f, f, 1e-6f, -1, nullptr), QI21_EINVAL, "qk H % 128");
  expect(qi21_op_rope_pack(0, f, f, f, nullptr), QI21_EINVAL, "rope_pack n 0");
  expect(qi21_op_vt_gemm(256, 100, 256, p, 256, p, p, 100, 1.f, -1, nullptr), QI21_EINVAL, "vt ldo");
  expect(qi21_op_flash(0, 1, p, 128, p, 128, p, 64, 10, nullptr, 0, nullptr, 0, 0, nullptr, p, 128, 1.f, nullptr),
         QI21_EINVAL, "flash no queries");
  expect(qi21_op_flash(4, 1, p, 128, p, 128, p, 32, 40, nullptr, 0, nullptr, 0, 0, nullptr, p, 128, 1.f, nullptr),
         QI21_EINVAL, "flash ldvt");
  expect(qi21_op_rowop(4, 4098, 2, f, f, p, 4100, f, 0, 0, 1e-6f, 1.f, nullptr), QI21_EINVAL, "rowop h");
  expect(qi21_op_rowop(4, 256, 6, f, f, p, 256, f, 0, 0, 1e-6f, 1.f, nullptr), QI21_EINVAL, "rowop pair ldxn");
  expect(qi21_op_rowop_parts(4, 256, 3, f, f, 0, 1024, p, 256, f, 0, 0, 1e-6f, 1.f, nullptr), QI21_EINVAL,
         "rowop 0 parts");
  expect(qi21_op_rowop_lo(QI21_FFN_LO4, 4, 512, 2, f, f, 1, 0, p, 636, b, f, 0, 0, 1e-6f, 1.f, nullptr), QI21_EINVAL,
         "rowop_lo ldxn");
  expect(qi21_op_rowop_lo(5, 4, 512, 2, f, f, 1, 0, p, 1024, b, f, 0, 0, 1e-6f, 1.f, nullptr), QI21_EINVAL,
         "rowop_lo format");
  expect(qi21_op_gemm_lo(QI21_FFN_LO8, 1, 16, 256, 192, p, 288, b, p, 288, b, p, 256, nullptr, nullptr, 1, 1.f, 1.f,
                         nullptr),
         QI21_EINVAL, "gemm_lo K % 128");
  expect(qi21_op_gemm_lo(QI21_FFN_LO4, 10, 16, 512, 512, p, 640, b, p, 640, b, p, 312, nullptr, b, 1, 1.f, 1.f, nullptr),
         QI21_EINVAL, "gemm_lo ldo");
  expect(qi21_op_plane_lo(QI21_FFN_LO4, QI21_F32, p, 16, 512, p, 636, 16, 0, 0, nullptr), QI21_EINVAL, "plane_lo ld");
  expect(qi21_op_plane_lo_fill(QI21_FFN_LO8, 16, 256, p, 384, nullptr, nullptr), QI21_EINVAL, "plane_lo_fill sc");
  expect(qi21_op_qkrope(4, 2, p, 256, f, f, f, f, 1e-6f, nullptr, 0, nullptr), QI21_EINVAL, "qkrope ldp");
  expect(qi21_op_embed(4, 100, f, f, f, nullptr), QI21_EINVAL, "embed h");
  expect(qi21_op_final(4, 100, f, f, f, 1e-6f, f, (int*)p, nullptr), QI21_EINVAL, "final h");
  expect(qi21_op_mods(0, f, f, nullptr), QI21_EINVAL, "mods h 0");
  expect(qi21_op_mods(1 << 30, f, f, nullptr), QI21_EINVAL, "mods h past the bound");
  expect(qi21_op_plane(QI21_F32, p, 0, 64, p, 16, 0, 0, nullptr), QI21_EINVAL, "plane rows");
}

void tile_checks() {
  // no device here: both choices assume 256 CUs
  CHECK(qi21::gemm_pick_tile(4096, 128 * 3, 256) == 1);   // N % 256: only the 128 x 128 tile
  CHECK(qi21::gemm_pick_tile(4096, 9216, 3072) == 0);     // many 256 x 256 tiles
  CHECK(qi21::gemm_pick_tile(1024, 3072, 3072) == 1);     // 48 tiles: the smaller tile fills more
  CHECK(qi21::gemm_split_count(1024, 3072, 8192, 4) == 4);
  CHECK(qi21::gemm_split_count(256, 3072, 8192, 4) == 1);  // too few rows
  CHECK(qi21::gemm_split_count(4096, 9216, 3072, 4) == 1);
  CHECK(qi21::gemm_split_count(1024, 3072, 64 * 3, 4) == 3);  // the largest divisor of K / 64 within the bound
}

void thread_checks() {
  // the last error belongs to the calling thread
  int32_t lp, n;
  const qi21_seg a[2] = {{0, 18, 0}, {1, 16, 16}};
  CHECK(qi21_layout_sizes(nullptr, 2, &lp, &n) == QI21_EINVAL && qi21_last_error()[0] != 0);
  std::string other = "unset";
  std::thread t([&] {
    other = qi21_last_error();
    CHECK(qi21_layout_sizes(a, 2, &lp, &n) == QI21_OK);
  });
  t.join();
  CHECK(other.empty());
  CHECK(qi21_last_error()[0] != 0);
}

}  // namespace

int main() {
  layout_checks();
  model_checks();
  op_checks();
  tile_checks();
  thread_checks();
  std::printf("host checks: %d of %d held\n", g_checks - g_fail, g_checks);
  return g_fail ? 1 : 0;
}
