"""CPU oracle of the Qwen-Image-2.1 single-stream denoiser step.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, and it shares no code with the GPU library: no kernels, headers,
tables or helpers.  It is the plain, slow definition that the GPU path is
checked against.

Sources, cited below by short name and item:

  [QI]  docs.rs, cortiq-engine 0.8.4, ``src/cortiq_engine/qwen_image21.rs``:
        the CPU reference of the denoiser (module doc "Semantics" and
        "Precision", ``Qi21Layout``, ``rope_tables``, ``layer_norm_into``,
        ``rms_norm_inplace``, ``softmax_prefix``, ``lin``, ``silu``,
        ``norm_mod``, ``gated_add``, ``qk_norm_rope``, ``attention``,
        ``block_cpu``, ``prefill``, ``step_cpu``, ``target_rope``).
  [WG]  docs.rs, cortiq-engine 0.8.3, ``src/gpu_wgpu/qi21.rs``: the device
        path (``mods_dev``, the ``qi_rowop`` kernel, ``dims``).

Precision ([QI] module doc, "Precision"): float32 activations; float64 sums
inside every norm and in the softmax denominator; the projections are
float32-accumulated GEMMs (numpy's float32 ``matmul``).  Passing
``dt=np.float64`` runs the same steps with float64 activations and GEMMs,
which bounds the float32 oracle's own rounding error.

The oracle has no range guards (the device path's power-of-two scalings of
its float16 sites are exact in exact arithmetic, [WG] module doc).

``storage="f16"`` additionally rounds, to IEEE binary16, every activation
the device design stores in float16 ([WG] module doc and ``Acts``: the
attention input, the q|k|v panel, the normalised and rotated q and k, the
unnormalised softmax weights P, the attention output, the FFN input and the
SwiGLU hidden), keeping everything else as above.  It computes what the
device design computes up to accumulation order, which separates the
design's own storage error from the kernels' arithmetic.

Parity status: every function here is pinned by a CPU test (worked values
printed on the pages, closed forms, invariants or brute force).  The
absolute values of the full-size output have no printed counterpart on the
pages; they rest on those pins plus the joint-recompute identity.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

F32 = np.float32
F64 = np.float64


# ───────────────────────────── layout ─────────────────────────────


def _seg_len(s) -> int:
    return int(s[1]) if s[0] == "text" else int(s[1]) * int(s[2])


class Layout:
    """Runs of the joint sequence, prefix first, target image last ([QI] ``Qi21Layout``).

    A run is ``("text", n)`` or ``("image", h, w)`` (h x w latent tokens in
    raster order).
    """

    def __init__(self, segs: Sequence[tuple]):
        self.segs = [tuple(s) for s in segs]

    @property
    def total(self) -> int:
        return sum(_seg_len(s) for s in self.segs)

    @property
    def target_len(self) -> int:
        return _seg_len(self.segs[-1])

    @property
    def prefix_len(self) -> int:
        return self.total - self.target_len

    def validate(self) -> None:
        """The last run is a non-empty image, and the prefix is not empty ([QI] ``validate``)."""
        last = self.segs[-1] if self.segs else None
        if last is None or last[0] != "image" or last[1] <= 0 or last[2] <= 0:
            raise ValueError("invalid layout: its last run has to be an image of at least one row and one column")
        if self.prefix_len == 0:
            raise ValueError("the prompt prefix is empty")

    def block_ids(self) -> List[int]:
        """Per row: the image block's ordinal, or -1 on a text row ([QI] ``block_ids``)."""
        out: List[int] = []
        nxt = 0
        for s in self.segs:
            if s[0] == "text":
                out += [-1] * s[1]
            else:
                out += [nxt] * (s[1] * s[2])
                nxt += 1
        return out

    def positions(self) -> np.ndarray:
        """(frame, row, col) RoPE position of every row, int64 ``[total, 3]`` ([QI] ``positions``).

        A text row sits at (p, p, p) and advances p by one.  An image block
        keeps the frame at p, centres its grid with integer halving
        (row r maps to r - (h - h//2), col c to c - (w - w//2)), and then
        advances p by max(h, w).
        """
        out = []
        p = 0
        for s in self.segs:
            if s[0] == "text":
                for _ in range(s[1]):
                    out.append((p, p, p))
                    p += 1
            else:
                h, w = int(s[1]), int(s[2])
                for r in range(h):
                    for c in range(w):
                        out.append((p, r - (h - h // 2), c - (w - w // 2)))
                p += max(h, w)
        return np.asarray(out, dtype=np.int64).reshape(-1, 3)


def prefix_visibility(layout: Layout) -> np.ndarray:
    """Keys each prefix row sees, as a count of leading keys ([QI] ``prefill``, ``end``).

    The block-causal mask of [QI] module doc: a text row i sees keys
    [0, i+1); an image row sees up to the end of its own image block.
    """
    ids = layout.block_ids()
    lp = layout.prefix_len
    end = np.zeros(lp, dtype=np.int64)
    for i in range(lp):
        if ids[i] < 0:
            end[i] = i + 1
        else:
            e = i + 1
            while e < lp and ids[e] == ids[i]:
                e += 1
            end[i] = e
    return end


def rope_tables(pos: np.ndarray, axes=(16, 56, 56), theta: float = 10000.0):
    """cos/sin ``[rows, sum(axes)/2]`` float32 ([QI] ``rope_tables``).

    Axis a with width d contributes d/2 frequencies 1/theta^(2i/d), computed
    in float32; the angle is float32(position) times the frequency in
    float32.  Columns run over the frame axis, then row, then column.
    """
    pos = np.asarray(pos, dtype=np.int64).reshape(-1, 3)
    freqs = []
    for d in axes:
        e = (np.arange(0, d // 2, dtype=F32) * F32(2)) / F32(d)
        freqs.append(F32(1.0) / np.power(F32(theta), e).astype(F32))
    cols = []
    for a, fr in enumerate(freqs):
        ang = pos[:, a].astype(F32)[:, None] * fr[None, :]
        cols.append(ang.astype(F32))
    ang = np.concatenate(cols, axis=1)
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


# ───────────────────────────── row helpers ─────────────────────────────


def store(a: np.ndarray, storage):
    """Round to the device's float16 storage when ``storage == "f16"`` ([WG] ``Acts``)."""
    if storage == "f16":
        return a.astype(np.float16).astype(a.dtype)
    return a



def layer_norm(x: np.ndarray, eps: float, dt=F32) -> np.ndarray:
    """Affine-free LayerNorm over the last axis, biased variance ([QI] ``layer_norm_into``).

    Mean and variance are float64 sums; the normalised value is rounded to
    the activation type.
    """
    x64 = x.astype(F64)
    n = x.shape[-1]
    mean = x64.sum(axis=-1, keepdims=True) / n
    d = x64 - mean
    var = (d * d).sum(axis=-1, keepdims=True) / n
    inv = 1.0 / np.sqrt(var + eps)
    return (d * inv).astype(dt)


def norm_mod(x: np.ndarray, scale: np.ndarray, eps: float, dt=F32) -> np.ndarray:
    """LN(x) * (1 + scale) ([QI] ``norm_mod``); ``scale`` is ``[H]`` or per row ``[rows, H]``."""
    one = dt(1.0)
    return (layer_norm(x, eps, dt) * (one + scale.astype(dt))).astype(dt)


def gated_add(x: np.ndarray, y: np.ndarray, gate_tanh: np.ndarray, dt=F32) -> np.ndarray:
    """x + tanh(gate) * y, the product rounded before the add ([QI] ``gated_add``)."""
    return (x + (gate_tanh.astype(dt) * y).astype(dt)).astype(dt)


def rms_norm(v: np.ndarray, w: np.ndarray, eps: float, dt=F32) -> np.ndarray:
    """Weighted RMSNorm over the last axis ([QI] ``rms_norm_inplace``).

    Mean of squares in float64; (x * inv) is rounded to the activation type
    and then multiplied by the weight.
    """
    v64 = v.astype(F64)
    ss = (v64 * v64).sum(axis=-1, keepdims=True) / v.shape[-1]
    inv = 1.0 / np.sqrt(ss + eps)
    return ((v64 * inv).astype(dt) * w.astype(dt)).astype(dt)


def softmax_prefix(scores: np.ndarray, valid: np.ndarray, dt=F32) -> np.ndarray:
    """Row softmax over each row's first ``valid[r]`` entries; the rest are 0 ([QI] ``softmax_prefix``).

    Row maximum and exponentials in the activation type, the denominator as
    a float64 sum, then a multiply by the rounded reciprocal.
    """
    rows, m = scores.shape
    valid = np.asarray(valid, dtype=np.int64).reshape(rows)
    live = np.arange(m)[None, :] < valid[:, None]
    neg = np.array(-np.inf, dtype=dt)
    mx = np.where(live, scores, neg).max(axis=1, keepdims=True)
    e = np.where(live, np.exp((scores - mx).astype(dt)).astype(dt), dt(0.0))
    den = e.astype(F64).sum(axis=1, keepdims=True)
    inv = (1.0 / den).astype(dt)
    return (e * inv).astype(dt)


def lin(x: np.ndarray, w: np.ndarray, dt=F32) -> np.ndarray:
    """y = x W^T with W stored ``[out, in]`` ([QI] ``lin``): one GEMM, accumulated in ``dt``."""
    return np.matmul(x.astype(dt), w.astype(dt).T).astype(dt)


def silu(v: np.ndarray, dt=F32) -> np.ndarray:
    """v / (1 + e^-v) ([QI] ``silu``)."""
    one = dt(1.0)
    return (v / (one + np.exp(-v).astype(dt))).astype(dt)


def split_mods(mods: np.ndarray, h: int, dt=F32):
    """[scale1 | gate1 | scale2 | gate2] -> (s1, tanh g1, s2, tanh g2) ([QI] ``block_cpu``; [WG] ``mods_dev``).

    The gates pass through tanh in the activation type; the scales are used
    as they are.  ``mods`` may be ``[4H]`` or per row ``[rows, 4H]``.
    """
    m = mods.astype(dt)
    s1, g1, s2, g2 = (m[..., i * h:(i + 1) * h] for i in range(4))
    return s1, np.tanh(g1).astype(dt), s2, np.tanh(g2).astype(dt)


def qk_norm_rope(a: np.ndarray, w: np.ndarray, cos: np.ndarray, sin: np.ndarray,
                 heads: int, hd: int, eps: float, dt=F32) -> np.ndarray:
    """Per (row, head): RMSNorm with ``w``, then rotate each interleaved pair ([QI] ``qk_norm_rope``).

    The pair (x[2j], x[2j+1]) with the row's (c, s) = (cos[j], sin[j])
    becomes (x[2j] c - x[2j+1] s, x[2j] s + x[2j+1] c).
    """
    n = a.shape[0]
    v = rms_norm(a.reshape(n, heads, hd), w, eps, dt)
    ev, od = v[..., 0::2], v[..., 1::2]
    c = cos.astype(dt)[:, None, :]
    s = sin.astype(dt)[:, None, :]
    out = np.empty_like(v)
    out[..., 0::2] = (ev * c).astype(dt) - (od * s).astype(dt)
    out[..., 1::2] = (ev * s).astype(dt) + (od * c).astype(dt)
    return out.reshape(n, heads * hd).astype(dt)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray,
              heads: int, hd: int, dt=F32, storage=None) -> np.ndarray:
    """Masked multi-head attention, all scores materialised ([QI] ``attention``).

    Per head: q scaled by 1/sqrt(hd), scores = q k^T (one GEMM), row i keeps
    its first ``visible[i]`` keys (``softmax_prefix``), output = P V.
    ``q`` is ``[n, heads*hd]``, ``k`` and ``v`` ``[m, heads*hd]``.
    With ``storage="f16"`` the unnormalised weights exp(s - max) are
    rounded to float16 before P V and their sum ([WG] ``qi_flash``: P in
    f16, the row sum of the same values).
    """
    n, m = q.shape[0], k.shape[0]
    scale = dt(1.0) / np.sqrt(dt(hd)).astype(dt)
    out = np.empty((n, heads * hd), dtype=dt)
    for h in range(heads):
        cs = slice(h * hd, (h + 1) * hd)
        qh = (q[:, cs].astype(dt) * scale).astype(dt)
        scores = np.matmul(qh, k[:, cs].astype(dt).T).astype(dt)
        if storage == "f16":
            live = np.arange(m)[None, :] < np.asarray(visible).reshape(n, 1)
            mx = np.where(live, scores, -np.inf).max(axis=1, keepdims=True)
            e = store(np.where(live, np.exp((scores - mx).astype(dt)), dt(0.0)).astype(dt), storage)
            den = e.astype(F64).sum(axis=1, keepdims=True)
            out[:, cs] = (np.matmul(e, v[:, cs].astype(dt)) / den).astype(dt)
        else:
            p = softmax_prefix(scores, visible, dt)
            out[:, cs] = np.matmul(p, v[:, cs].astype(dt)).astype(dt)
    return out


# ───────────────────────────── model pieces ─────────────────────────────


@dataclass
class Geometry:
    dim: int
    heads: int
    head_dim: int
    inter: int
    in_ch: int = 64
    eps: float = 1e-6
    axes: Tuple[int, int, int] = (16, 56, 56)
    theta: float = 10000.0


def block(blk: dict, x: np.ndarray, mods: np.ndarray, rope, kv_prefix, visible,
          g: Geometry, dt=F32, storage=None):
    """One single-stream block on the query rows ``x`` ([QI] ``block_cpu``; module doc "Semantics").

    x += tanh(g1) * O(attn(LN(x)(1+s1))), then x += tanh(g2) * down(silu(gate) * up)
    of LN(x)(1+s2).  ``kv_prefix`` = (K, V) of earlier rows that the
    queries also attend to, placed before the rows' own keys; ``visible[i]``
    counts the leading keys query i sees.  Returns (new x, (K, V) of the
    rows themselves, post norm and RoPE).
    """
    h = g.dim
    st = storage
    s1, g1t, s2, g2t = split_mods(mods, h, dt)
    xn = store(norm_mod(x, s1, g.eps, dt), st)
    q = store(lin(xn, blk["to_q"], dt), st)
    k = store(lin(xn, blk["to_k"], dt), st)
    v = store(lin(xn, blk["to_v"], dt), st)
    q = store(qk_norm_rope(q, blk["norm_q"], rope[0], rope[1], g.heads, g.head_dim, g.eps, dt), st)
    k = store(qk_norm_rope(k, blk["norm_k"], rope[0], rope[1], g.heads, g.head_dim, g.eps, dt), st)
    if kv_prefix is not None:
        ka = np.concatenate([kv_prefix[0].astype(dt), k], axis=0)
        va = np.concatenate([kv_prefix[1].astype(dt), v], axis=0)
    else:
        ka, va = k, v
    att = store(attention(q, ka, va, visible, g.heads, g.head_dim, dt, st), st)
    x = gated_add(x.astype(dt), lin(att, blk["to_out"], dt), g1t, dt)
    xn = store(norm_mod(x, s2, g.eps, dt), st)
    hid = store((silu(lin(xn, blk["gate"], dt), dt) * lin(xn, blk["up"], dt)).astype(dt), st)
    x = gated_add(x, lin(hid, blk["down"], dt), g2t, dt)
    return x, (k, v)


@dataclass
class Prefix:
    """Per-layer post-RoPE keys and values of a prompt prefix, plus its target RoPE ([QI] ``Qi21Prefix``)."""

    layout: Layout
    k: List[np.ndarray]
    v: List[np.ndarray]
    rope_t: Tuple[np.ndarray, np.ndarray]

    @property
    def lp(self) -> int:
        return self.layout.prefix_len


def target_rope(layout: Layout, g: Geometry):
    """RoPE tables of the target rows under this prefix's layout ([QI] ``target_rope``)."""
    pos = layout.positions()
    return rope_tables(pos[layout.prefix_len:], g.axes, g.theta)


def prefill(model, x: np.ndarray, layout: Layout, dt=F32, layers: Optional[int] = None,
            storage=None) -> Prefix:
    """Run the prefix rows through every block once, keeping K/V per layer ([QI] ``prefill``).

    ``x`` holds the prefix rows ``[lp, H]`` (already embedded); modulation is
    the t = 0 modulation ``model.mods0``; the mask is block-causal.
    """
    g = model.geom
    layout.validate()
    lp = layout.prefix_len
    if x.shape != (lp, g.dim):
        raise ValueError(f"prefix rows {x.shape}, the layout needs {(lp, g.dim)}")
    pos = layout.positions()
    rope_p = rope_tables(pos[:lp], g.axes, g.theta)
    vis = prefix_visibility(layout)
    ks, vs = [], []
    x = x.astype(dt)
    for l in range(model.layers if layers is None else layers):
        x, (k, v) = block(model.block(l), x, model.mods0, rope_p, None, vis, g, dt, storage)
        ks.append(k)
        vs.append(v)
    return Prefix(layout, ks, vs, target_rope(layout, g))


def embed_image(tok: np.ndarray, img_in: np.ndarray, dt=F32) -> np.ndarray:
    """img_in projection of the latent tokens, no bias ([QI] ``embed_image``)."""
    return lin(tok, img_in, dt)


def final_layer(x: np.ndarray, final_scale: np.ndarray, proj_out: np.ndarray, eps: float, dt=F32):
    """v = (LN(x)(1 + final_scale)) proj_out^T ([QI] ``step_cpu``; the final norm's eps is eps, [WG] ``dims``)."""
    return lin(norm_mod(x, final_scale, eps, dt), proj_out, dt)


def step(model, prefix: Prefix, tok: np.ndarray, mods: np.ndarray, final_scale: np.ndarray,
         dt=F32, layers: Optional[int] = None, storage=None) -> np.ndarray:
    """One denoiser call: tokens ``[n, 64]`` -> velocity ``[n, 64]`` ([QI] ``step_cpu``).

    Every target row sees all lp + n keys: the cached prefix, then the
    target rows themselves, rotated by the prefix's own target tables.
    """
    g = model.geom
    n = prefix.layout.target_len
    lp = prefix.lp
    x = embed_image(tok, model.img_in, dt)
    every = np.full(n, lp + n, dtype=np.int64)
    for l in range(model.layers if layers is None else layers):
        x, _ = block(model.block(l), x, mods, prefix.rope_t, (prefix.k[l], prefix.v[l]), every, g, dt, storage)
    return final_layer(x, final_scale, model.proj_out, g.eps, dt)


# ───────────────────────────── time path and sampler ─────────────────────────────


def timestep_embedding(t: float) -> np.ndarray:
    """Sinusoidal embedding of the model time t in [0, 1] ([QI] ``Qi21Dit::temb``).

    ts = 1000 t; frequency i = exp(-ln(10000) i / 128) for i < 128; the
    cosines of ts * frequency, then the sines.  Every step in float32, as on
    the host path.
    """
    half = 128
    ts = F32(1000.0) * F32(t)
    i = np.arange(half, dtype=F32)
    f = np.exp((-np.log(F32(10000.0))) * i / F32(half)).astype(F32)
    a = (ts * f).astype(F32)
    return np.concatenate([np.cos(a), np.sin(a)]).astype(F32)


def lin_row(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """One vector through a small bias-free projection ``w [out][in]`` with
    float64 accumulation, rounded to float32 ([QI] ``lin_row``)."""
    return (np.asarray(w, F64) @ np.asarray(x, F64)).astype(F32)


def time_mods(tw: dict, t: float):
    """The shared block modulation and the final-norm scale of one time
    ([QI] ``Qi21Dit::temb`` and ``Qi21Dit::mods``).

    temb = t_lin2 silu(t_lin1 e(t)); s = silu(temb); returns
    (modulation s [4 dim] = raw [s1|g1|s2|g2], norm_out s [dim] = final_scale).
    """
    e = timestep_embedding(t)
    h = silu(lin_row(tw["t_lin1"], e))
    s = silu(lin_row(tw["t_lin2"], h))
    return lin_row(tw["modulation"], s), lin_row(tw["norm_out"], s)


def sample(model, prefix: Prefix, tok: np.ndarray, schedule, storage=None) -> np.ndarray:
    """A flow-matching Euler sampler over the cached prefix ([WG] module doc:
    a 40-step ``imagine`` calls the step once per time).

    Reading (the pages give no schedule or update rule): for k < len - 1,
    v = step(x, mods(t_k)), x <- x + (t_{k+1} - t_k) v, with the difference
    taken in float32 between the float32 times.
    """
    x = np.asarray(tok, F32)
    tw = model.time()
    ts = np.asarray(schedule, F32)
    for k in range(len(ts) - 1):
        mods, fsc = time_mods(tw, float(ts[k]))
        v = step(model, prefix, x, mods, fsc, storage=storage)
        x = (x + (ts[k + 1] - ts[k]) * v).astype(F32)
    return x


# ───────────────────────────── txt_in front ─────────────────────────────


def gelu_tanh(v: np.ndarray) -> np.ndarray:
    """The tanh approximation of GELU, evaluated in float64 and rounded to
    float32 ([QI] ``gelu_tanh``)."""
    x = np.asarray(v, F64)
    return (0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x * x * x)))).astype(F32)


def embed_text(feats: np.ndarray, txt_norm: np.ndarray, txt_in1: np.ndarray, txt_in2: np.ndarray,
               eps: float) -> np.ndarray:
    """Text features ``[n, context_in]`` -> prefix rows ``[n, dim]`` ([QI] ``Qi21Dit::embed_text``).

    Per row: RMSNorm with a float64 sum of squares and a zero-centred
    weight, f32(v / sqrt(mean(v^2) + eps)) * (w + 1); then txt_in1, the tanh
    GELU, and txt_in2 (bias-free, float32-accumulated projections).
    """
    x = np.asarray(feats, F32)
    ms = (x.astype(F64) ** 2).sum(axis=1, keepdims=True) / x.shape[1]
    inv = 1.0 / np.sqrt(ms + eps)
    xn = ((x.astype(F64) * inv).astype(F32) * (np.asarray(txt_norm, F32) + F32(1.0))).astype(F32)
    h = gelu_tanh(lin(xn, txt_in1))
    return lin(h, txt_in2)


def joint_forward(model, x_prefix: np.ndarray, tok: np.ndarray, layout: Layout, mods: np.ndarray,
                  final_scale: np.ndarray, dt=F32, layers: Optional[int] = None):
    """The whole joint sequence [prefix; target] in one pass, no cache ([QI] module doc "Semantics").

    Prefix rows carry the t = 0 modulation and the block-causal mask; target
    rows carry the step's modulation and see every row.  Returns the target
    rows' velocity, the prefix rows after the last block, and every layer's
    (K, V) of all rows.  Used only to pin the cache: prefill + step must
    give the same target velocity.
    """
    g = model.geom
    lp, n = layout.prefix_len, layout.target_len
    pos = layout.positions()
    rope = rope_tables(pos, g.axes, g.theta)
    vis = np.concatenate([prefix_visibility(layout), np.full(n, lp + n, dtype=np.int64)])
    row_mods = np.concatenate([np.broadcast_to(model.mods0, (lp, 4 * g.dim)),
                               np.broadcast_to(mods, (n, 4 * g.dim))], axis=0)
    x = np.concatenate([x_prefix.astype(dt), embed_image(tok, model.img_in, dt)], axis=0)
    kv = []
    for l in range(model.layers if layers is None else layers):
        x, (k, v) = block(model.block(l), x, row_mods, rope, None, vis, g, dt)
        kv.append((k, v))
    out = final_layer(x[lp:], final_scale, model.proj_out, g.eps, dt)
    return out, x[:lp], kv
