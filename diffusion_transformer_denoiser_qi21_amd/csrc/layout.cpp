// Layout helpers of the qi21 C ABI (host only): prefix / target sizes,
// RoPE positions, the prefix's block-causal visibility and the RoPE tables.
//
// Following [QI] (docs.rs cortiq-engine 0.8.4,
// src/cortiq_engine/qwen_image21.rs), items `Qi21Layout`, `prefill` and
// `rope_tables`.  Each row gets a (frame, row, col) position from a running
// counter p: a text row takes (p, p, p) and bumps p by one; an image of
// h x w tokens puts all its tokens on frame p, with the grid shifted so
// that row r sits at r - (h - h/2) and column c at c - (w - w/2) (integer
// division), after which p grows by max(h, w).  In a prefill, text row i
// attends to keys 0..i and an image row to every key up to the last row of
// its own image.  The tables use float32 frequencies 1/theta^(2i/d) for
// each axis of width d and a float32 angle, with the axes laid out frame,
// row, col.
#include <cmath>
#include <vector>

#include "../../include/qi21.h"
#include "status.h"

namespace {
int64_t seg_len(const qi21_seg& s) { return s.kind == 0 ? (int64_t)s.h : (int64_t)s.h * s.w; }

int refuse(const char* why) {
  qi21::set_error_text(why);
  return QI21_EINVAL;
}
}  // namespace

extern "C" {

int qi21_layout_sizes(const qi21_seg* segs, int nseg, int32_t* lp, int32_t* n) {
  qi21::set_error_text("");
  if (!segs || nseg < 2) return refuse("layout: a prefix run and the target image are needed (segs NULL or nseg < 2)");
  int64_t total = 0;
  for (int i = 0; i < nseg; ++i) {
    const qi21_seg& s = segs[i];
    if ((s.kind != 0 && s.kind != 1) || s.h < 0 || (s.kind == 1 && s.w < 0))
      return refuse("layout: a run has an unknown kind or a negative size");
    total += seg_len(s);
    if (total > (1 << 24)) return refuse("layout: more than 2^24 rows");
  }
  const qi21_seg& t = segs[nseg - 1];
  if (t.kind != 1 || t.h <= 0 || t.w <= 0) return refuse("layout: the final run must be a non-empty image");
  const int64_t nt = seg_len(t);
  if (total - nt <= 0) return refuse("layout: the prefix has no rows");
  if (lp) *lp = (int32_t)(total - nt);
  if (n) *n = (int32_t)nt;
  return QI21_OK;
}

int qi21_layout_tables(const qi21_seg* segs, int nseg, const int32_t* axes, float theta, int64_t* pos,
                       uint32_t* vis, float* cos_p, float* sin_p, float* cos_t, float* sin_t) {
  int32_t lp = 0, n = 0;
  const int rc = qi21_layout_sizes(segs, nseg, &lp, &n);
  if (rc != QI21_OK) return rc;
  if (!axes) return refuse("layout tables: axes is NULL");
  int hd = 0;
  for (int a = 0; a < 3; ++a) {
    if (axes[a] <= 0 || axes[a] % 2) return refuse("layout tables: every axis width must be positive and even");
    hd += axes[a];
  }
  const int half = hd / 2;
  const int total = lp + n;
  std::vector<int64_t> P((size_t)total * 3);
  std::vector<int> block((size_t)total, -1);
  int64_t p = 0;
  int r = 0, id = 0;
  for (int i = 0; i < nseg; ++i) {
    const qi21_seg& s = segs[i];
    if (s.kind == 0) {
      for (int j = 0; j < s.h; ++j, ++r) {
        P[3 * r] = P[3 * r + 1] = P[3 * r + 2] = p;
        ++p;
      }
    } else {
      const int64_t h = s.h, w = s.w;
      for (int64_t y = 0; y < h; ++y)
        for (int64_t x = 0; x < w; ++x, ++r) {
          P[3 * r] = p;
          P[3 * r + 1] = y - (h - h / 2);
          P[3 * r + 2] = x - (w - w / 2);
          block[r] = id;
        }
      ++id;
      p += h > w ? h : w;
    }
  }
  if (pos)
    for (size_t i = 0; i < P.size(); ++i) pos[i] = P[i];
  if (vis) {
    for (int i = 0; i < lp; ++i) {
      int e = i + 1;
      if (block[i] >= 0)
        while (e < lp && block[e] == block[i]) ++e;
      vis[i] = (uint32_t)e;
    }
  }
  // per-column frequency and axis
  std::vector<float> freq(half);
  std::vector<int> axis(half);
  int j = 0;
  for (int a = 0; a < 3; ++a)
    for (int i = 0; i < axes[a] / 2; ++i, ++j) {
      freq[j] = 1.0f / std::pow(theta, (float)(2 * i) / (float)axes[a]);
      axis[j] = a;
    }
  auto fill = [&](int row0, int rows, float* c, float* s) {
    if (!c && !s) return;
    for (int rr = 0; rr < rows; ++rr)
      for (int k = 0; k < half; ++k) {
        const float ang = (float)P[3 * (size_t)(row0 + rr) + axis[k]] * freq[k];
        if (c) c[(size_t)rr * half + k] = std::cos(ang);
        if (s) s[(size_t)rr * half + k] = std::sin(ang);
      }
  };
  fill(0, lp, cos_p, sin_p);
  fill(lp, n, cos_t, sin_t);
  return QI21_OK;
}

}  // extern "C"
