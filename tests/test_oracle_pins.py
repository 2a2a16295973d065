"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: values
printed on the pages (``tests/golden/pages_examples.json``), closed forms,
brute force on tiny inputs, library special cases, or invariants of the
method (linearity, scale invariance, relative RoPE, causality, the cache
identity).  Each is chosen so that a plausible mistake (a dropped term, a
transposed operand, a swapped gate/up, a wrong RoPE pairing, a wrong mask)
fails at least one of them.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

from inputs import CONFIGS
from oracle import SynthModel, workload_inputs
from oracle import qi21_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")))
F64 = np.float64


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, F64) - np.asarray(b, F64)) / np.linalg.norm(np.asarray(b, F64)))


# ───────────────────────────── layout / RoPE ─────────────────────────────


def test_positions_worked_example_t2i():
    g = GOLD["positions_t2i"]
    lay = O.Layout(g["layout"])
    p = lay.positions()
    for r, want in g["rows"].items():
        assert list(p[int(r)]) == want
    assert lay.prefix_len == g["prefix_len"]
    assert lay.block_ids() == g["block_ids"]


def test_positions_text_after_image():
    g = GOLD["positions_text_after_image"]
    p = O.Layout(g["layout"]).positions()
    for r, f in g["frame_of_row"].items():
        assert p[int(r)][0] == f
    for r, want in g["rows"].items():
        assert list(p[int(r)]) == want


def test_rope_tables_unit_rotations_and_identity():
    g = GOLD["rope_unit_rotations"]
    lay = O.Layout(g["layout"])
    c, s = O.rope_tables(lay.positions(), tuple(g["axes"]), g["theta"])
    assert c.shape == (lay.total, g["columns_per_row"])
    assert np.all(np.abs(c.astype(F64) ** 2 + s.astype(F64) ** 2 - 1.0) < g["unit_tol"])
    assert np.all(np.abs(c[0] - 1.0) < g["identity_at_position_zero_tol"])


def test_rope_tables_hand_values():
    # Position (5, -1, 2): column 0 is the frame axis' first frequency (1),
    # column 1 its second (10000^(-2/16)), column 8 the row axis' first
    # frequency, column 36 the column axis' first, column 63 the column
    # axis' last (10000^(-54/56)).
    c, s = O.rope_tables(np.array([[5, -1, 2]]), (16, 56, 56), 10000.0)
    want = {0: 5.0, 1: 5.0 * 10000 ** (-2 / 16), 7: 5.0 * 10000 ** (-14 / 16), 8: -1.0,
            9: -1.0 * 10000 ** (-2 / 56), 36: 2.0, 63: 2.0 * 10000 ** (-54 / 56)}
    for col, ang in want.items():
        assert abs(c[0, col] - math.cos(ang)) < 2e-6, col
        assert abs(s[0, col] - math.sin(ang)) < 2e-6, col


def test_prefix_visibility_block_causal():
    lay = O.Layout([("text", 3), ("image", 2, 2), ("text", 2), ("image", 1, 1)])
    # text rows see up to themselves; the 2x2 image rows see to the end of
    # their block; the target block is not part of the prefix
    assert list(O.prefix_visibility(lay)) == [1, 2, 3, 7, 7, 7, 7, 8, 9]


def test_layout_validation():
    with pytest.raises(ValueError):
        O.Layout([("text", 3)]).validate()
    with pytest.raises(ValueError):
        O.Layout([("image", 2, 2)]).validate()
    with pytest.raises(ValueError):
        O.Layout([("text", 2), ("image", 0, 3)]).validate()


def test_mods_gate_chunks_tanh_worked_example():
    g = GOLD["mods_dev_gates_tanh"]
    h = g["h"]
    m = (np.arange(4 * h, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    d = np.concatenate(O.split_mods(m, h))
    for lo, hi in g["unchanged"]:
        assert np.array_equal(d[lo:hi], m[lo:hi])
    for i in g["tanh_of_input_at"]:
        assert abs(float(d[i]) - math.tanh(float(m[i]))) < 1e-7
    assert np.array_equal(d[3:6], np.tanh(m[3:6]))


# ───────────────────────────── norms / softmax / lin ─────────────────────────────


def test_layer_norm_closed_form():
    x = np.array([[1.0, 2.0, 3.0, 4.0]], dtype=np.float32)
    y = O.layer_norm(x, 1e-6)
    want = (np.array([1, 2, 3, 4]) - 2.5) / math.sqrt(1.25 + 1e-6)
    assert np.allclose(y[0], want, rtol=1e-6, atol=1e-7)
    r = np.random.default_rng(0).normal(3.0, 2.0, size=(8, 512)).astype(np.float32)
    y = O.layer_norm(r, 1e-6).astype(F64)
    assert np.all(np.abs(y.mean(1)) < 1e-6)
    assert np.all(np.abs(y.var(1) - 1.0) < 1e-5)
    # affine invariance: LN(a x + b) = LN(x)
    assert np.allclose(O.layer_norm(r * 3 + 7, 1e-6), O.layer_norm(r, 1e-6), atol=2e-5)


def test_norm_mod_scale_and_gated_add():
    r = np.random.default_rng(1).normal(size=(4, 64)).astype(np.float32)
    s = np.random.default_rng(2).normal(0, 0.1, size=64).astype(np.float32)
    y = O.norm_mod(r, s, 1e-6)
    assert np.allclose(y / (1 + s), O.layer_norm(r, 1e-6), rtol=1e-6, atol=1e-6)
    yy = np.ones_like(r)
    gt = np.full(64, 0.5, np.float32)
    assert np.array_equal(O.gated_add(r, yy, gt), r + np.float32(0.5))
    assert np.array_equal(O.gated_add(r, yy, np.zeros(64, np.float32)), r)


def test_rms_norm_closed_form():
    y = O.rms_norm(np.array([[3.0, 4.0]], np.float32), np.array([1.0, 2.0], np.float32), 0.0)
    rms = math.sqrt(12.5)
    assert np.allclose(y[0], [3 / rms, 2 * 4 / rms], rtol=1e-6)
    r = np.random.default_rng(3).normal(0, 5, size=(16, 128)).astype(np.float32)
    y = O.rms_norm(r, np.ones(128, np.float32), 1e-6).astype(F64)
    assert np.allclose(np.sqrt((y * y).mean(1)), 1.0, atol=1e-6)


def test_softmax_prefix_against_definition():
    rng = np.random.default_rng(4)
    s = rng.normal(0, 3, size=(6, 9)).astype(np.float32)
    valid = np.array([1, 2, 5, 9, 9, 3])
    p = O.softmax_prefix(s, valid)
    for r in range(6):
        v = valid[r]
        e = np.exp(s[r, :v].astype(F64) - s[r, :v].max())
        assert np.allclose(p[r, :v], e / e.sum(), rtol=1e-6, atol=1e-7)
        assert np.all(p[r, v:] == 0)
    assert p[0, 0] == 1.0


def test_lin_orientation_permutation():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(5, 7)).astype(np.float32)
    perm = rng.permutation(7)[:4]
    w = np.zeros((4, 7), np.float32)
    w[np.arange(4), perm] = 1.0
    assert np.array_equal(O.lin(x, w), x[:, perm])


def test_silu_values():
    v = np.array([0.0, 1.0, -2.0, 10.0], np.float32)
    want = [0.0, 1 / (1 + math.exp(-1)), -2 / (1 + math.exp(2)), 10 / (1 + math.exp(-10))]
    assert np.allclose(O.silu(v), want, rtol=1e-6)


# ───────────────────────────── qk norm + RoPE ─────────────────────────────


def test_qk_norm_rope_unit_vectors():
    hd, heads = 128, 2
    p = 3
    c, s = O.rope_tables(np.array([[p, p, p]]), (16, 56, 56), 10000.0)
    a = np.zeros((1, heads * hd), np.float32)
    a[0, 0] = 2.0          # head 0: e_0
    a[0, hd + 1] = 0.5     # head 1: e_1
    y = O.qk_norm_rope(a, np.ones(hd, np.float32), c, s, heads, hd, 0.0)
    r = math.sqrt(hd)      # RMSNorm of a one-hot vector
    assert np.allclose(y[0, :2], [r * math.cos(p), r * math.sin(p)], rtol=1e-5)
    assert np.allclose(y[0, hd:hd + 2], [-r * math.sin(p), r * math.cos(p)], rtol=1e-5)
    assert np.all(y[0, 2:hd] == 0) and np.all(y[0, hd + 2:] == 0)


def test_qk_rope_preserves_norm_and_weight_applies_before_rotation():
    rng = np.random.default_rng(6)
    hd, heads, n = 128, 3, 10
    pos = np.stack([np.arange(n), np.arange(n) - 4, np.arange(n) * 2], 1)
    c, s = O.rope_tables(pos, (16, 56, 56), 10000.0)
    a = rng.normal(size=(n, heads * hd)).astype(np.float32)
    w = (1 + rng.normal(0, 0.02, hd)).astype(np.float32)
    y = O.qk_norm_rope(a, w, c, s, heads, hd, 1e-6).reshape(n, heads, hd).astype(F64)
    z = O.rms_norm(a.reshape(n, heads, hd), w, 1e-6).astype(F64)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(z, axis=-1), rtol=1e-6)


# ───────────────────────────── attention ─────────────────────────────


def _brute_attention(q, k, v, vis, heads, hd):
    n, m = q.shape[0], k.shape[0]
    out = np.zeros((n, heads * hd))
    for h in range(heads):
        for i in range(n):
            sc = []
            for j in range(vis[i]):
                sc.append(sum(float(q[i, h * hd + d]) * float(k[j, h * hd + d]) for d in range(hd)) / math.sqrt(hd))
            mx = max(sc)
            e = [math.exp(t - mx) for t in sc]
            z = sum(e)
            for d in range(hd):
                out[i, h * hd + d] = sum(e[j] / z * float(v[j, h * hd + d]) for j in range(vis[i]))
    return out


def test_attention_brute_force_masked():
    rng = np.random.default_rng(7)
    heads, hd, n, m = 2, 8, 6, 9
    q, k, v = (rng.normal(size=(r, heads * hd)).astype(np.float32) for r in (n, m, m))
    vis = np.array([1, 3, 3, 6, 9, 9])
    want = _brute_attention(q, k, v, vis, heads, hd)
    assert _rel(O.attention(q, k, v, vis, heads, hd), want) < 1e-6
    assert _rel(O.attention(q, k, v, vis, heads, hd, dt=F64), want) < 1e-13


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    heads, hd, n, m = 2, 16, 4, 7
    q, k, v = (rng.normal(size=(r, heads * hd)).astype(np.float32) for r in (n, m, m))
    one = O.attention(q, k, v, np.ones(n, np.int64), heads, hd)
    assert np.allclose(one, np.broadcast_to(v[0], one.shape), atol=1e-7)
    ksame = np.broadcast_to(k[0], k.shape).copy()
    vis = np.array([2, 4, 7, 7])
    out = O.attention(q, ksame, v, vis, heads, hd)
    for i in range(n):
        assert np.allclose(out[i], v[:vis[i]].astype(F64).mean(0), atol=1e-6)


def test_attention_matches_torch_sdpa_f64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    heads, hd, n, m = 3, 32, 11, 15
    q, k, v = (rng.normal(size=(r, heads * hd)) for r in (n, m, m))
    vis = np.sort(rng.integers(1, m + 1, size=n))
    mask = torch.from_numpy(np.arange(m)[None, :] < vis[:, None])
    tq, tk, tv = (torch.from_numpy(a).reshape(a.shape[0], heads, hd).transpose(0, 1) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    ref = ref.transpose(0, 1).reshape(n, heads * hd).numpy()
    assert _rel(O.attention(q, k, v, vis, heads, hd, dt=F64), ref) < 1e-12


# ───────────────────────────── block / step ─────────────────────────────


@pytest.fixture(scope="module")
def tiny():
    w = CONFIGS["tiny"]
    return w, SynthModel(w.model), workload_inputs(w)


def _one_block(model, x, mods, overrides=None, dt=F64, kv=None, eps=None):
    g = model.geom if eps is None else dataclasses.replace(model.geom, eps=eps)
    n = x.shape[0]
    pos = np.stack([np.arange(n)] * 3, 1)
    rope = O.rope_tables(pos, g.axes, g.theta)
    blk = dict(model.block(0))
    blk.update(overrides or {})
    vis = np.full(n, n, np.int64) if kv is None else np.full(n, n + kv[0].shape[0], np.int64)
    return O.block(blk, x, mods, rope, kv, vis, g, dt)


def test_gate_zero_gives_identity_residual(tiny):
    w, model, d = tiny
    g = model.geom
    h = g.dim
    mods = d["mods"].copy()
    mods[h:2 * h] = 0.0
    mods[3 * h:] = 0.0
    lay = O.Layout(w.layout())
    pre = O.prefill(model, d["x_prefix"], lay)
    v = O.step(model, pre, d["tok"], mods, d["final_scale"])
    # closed form: both gates zero, so every block is the identity
    x = d["tok"].astype(F64) @ model.img_in.astype(F64).T
    mu = x.mean(1, keepdims=True)
    xn = (x - mu) / np.sqrt(((x - mu) ** 2).mean(1, keepdims=True) + g.eps)
    want = (xn * (1 + d["final_scale"].astype(F64))) @ model.proj_out.astype(F64).T
    assert _rel(v, want) < 1e-5


def test_ffn_branch_linear_in_up_and_down_not_gate(tiny):
    _, model, d = tiny
    g = model.geom
    h = g.dim
    x = d["x_prefix"][:8].astype(F64)
    mods = d["mods"].astype(F64).copy()
    mods[h:2 * h] = 0.0     # attention branch off
    mods[3 * h:] = 5.0      # FFN gate tanh(5)
    blk = model.block(0)
    base = _one_block(model, x, mods)[0] - x
    up2 = _one_block(model, x, mods, {"up": blk["up"] * 2})[0] - x
    down2 = _one_block(model, x, mods, {"down": blk["down"] * 2})[0] - x
    gate2 = _one_block(model, x, mods, {"gate": blk["gate"] * 2})[0] - x
    assert _rel(up2, 2 * base) < 1e-12
    assert _rel(down2, 2 * base) < 1e-12
    assert _rel(gate2, 2 * base) > 1e-3


def test_attention_branch_linear_in_v_and_o_invariant_in_q_k_scale(tiny):
    _, model, d = tiny
    g = model.geom
    h = g.dim
    x = d["x_prefix"][:8].astype(F64)
    mods = d["mods"].astype(F64).copy()
    mods[h:2 * h] = 5.0     # attention gate tanh(5)
    mods[3 * h:] = 0.0      # FFN branch off
    blk = model.block(0)
    base = _one_block(model, x, mods)[0] - x
    assert _rel(_one_block(model, x, mods, {"to_v": blk["to_v"] * 2})[0] - x, 2 * base) < 1e-12
    assert _rel(_one_block(model, x, mods, {"to_out": blk["to_out"] * 2})[0] - x, 2 * base) < 1e-12
    # q and k are RMS-normalised per head: with eps = 0 their scale drops out
    base0 = _one_block(model, x, mods, eps=0.0)[0] - x
    assert _rel(_one_block(model, x, mods, {"to_q": blk["to_q"] * 4}, eps=0.0)[0] - x, base0) < 1e-12
    assert _rel(_one_block(model, x, mods, {"to_k": blk["to_k"] * 0.25}, eps=0.0)[0] - x, base0) < 1e-12
    # but the norm weights do not
    assert _rel(_one_block(model, x, mods, {"norm_q": blk["norm_q"] * 3}, eps=0.0)[0] - x, base0) > 1e-3


def test_rope_depends_on_relative_position_only(tiny):
    _, model, d = tiny
    g = model.geom
    n = 12
    x = d["x_prefix"][:n].astype(F64)
    vis = np.full(n, n, np.int64)
    blk = model.block(0)
    base = np.stack([np.arange(n), np.arange(n) % 3 - 1, np.arange(n) % 4 - 2], 1)
    outs = []
    for shift in (0, 5):
        rope = O.rope_tables(base + shift, g.axes, g.theta)
        outs.append(O.block(blk, x, d["mods"].astype(F64), rope, None, vis, g, F64)[0])
    assert _rel(outs[1] - x, outs[0] - x) < 1e-5
    # a shift of one row's position alone does change things
    moved = base.copy()
    moved[0] += 5
    rope = O.rope_tables(moved, g.axes, g.theta)
    other = O.block(blk, x, d["mods"].astype(F64), rope, None, vis, g, F64)[0]
    assert _rel(other - x, outs[0] - x) > 1e-3


def test_prefix_mask_is_block_causal(tiny):
    _, model, d = tiny
    g = model.geom
    lay = O.Layout([("text", 3), ("image", 2, 2), ("text", 2), ("image", 2, 2)])
    lp = lay.prefix_len
    x = d["x_prefix"][:lp].astype(F64)
    pos = lay.positions()
    rope = O.rope_tables(pos[:lp], g.axes, g.theta)
    vis = O.prefix_visibility(lay)
    blk = model.block(0)
    out0 = O.block(blk, x, model.mods0, rope, None, vis, g, F64)[0]
    # perturb text row 1: rows 0 keeps its value, every later row changes
    bump = np.random.default_rng(10).normal(size=g.dim)  # not a constant: LN removes those
    x1 = x.copy()
    x1[1] += bump
    out1 = O.block(blk, x1, model.mods0, rope, None, vis, g, F64)[0]
    assert np.array_equal(out1[0], out0[0])
    assert np.all(np.abs(out1[2:] - out0[2:]).max(1) > 0)
    # perturb the last row of the image block (row 6): earlier image rows see it
    x2 = x.copy()
    x2[6] += bump
    out2 = O.block(blk, x2, model.mods0, rope, None, vis, g, F64)[0]
    assert np.array_equal(out2[:3], out0[:3])
    assert np.all(np.abs(out2[3:] - out0[3:]).max(1) > 0)


def test_prefix_unchanged_when_target_changes(tiny):
    w, model, d = tiny
    lay = O.Layout([("text", 5), ("image", 3, 4), ("image", 4, 4)])
    lp, n = lay.prefix_len, lay.target_len
    xp = d["x_prefix"][:1].repeat(lp, 0) * np.linspace(0.5, 1.5, lp, dtype=np.float32)[:, None]
    tok_a = d["tok"][:n]
    tok_b = d["tok"][n:2 * n]
    va, xa, kva = O.joint_forward(model, xp, tok_a, lay, d["mods"], d["final_scale"])
    vb, xb, kvb = O.joint_forward(model, xp, tok_b, lay, d["mods"], d["final_scale"])
    assert np.array_equal(xa, xb)
    for (ka, va_), (kb, vb_) in zip(kva, kvb):
        assert np.array_equal(ka[:lp], kb[:lp]) and np.array_equal(va_[:lp], vb_[:lp])
    assert not np.array_equal(va, vb)


@pytest.mark.parametrize("segs", [
    [("text", 18), ("image", 16, 16)],
    [("text", 5), ("image", 3, 4), ("image", 8, 8)],
    [("text", 2), ("image", 2, 4), ("text", 1), ("image", 5, 7)],
])
def test_cache_equals_joint_recompute(tiny, segs):
    _, model, d = tiny
    lay = O.Layout(segs)
    lp, n = lay.prefix_len, lay.target_len
    xp = d["x_prefix"][np.arange(lp) % 18] * np.float32(1.25)
    tok = d["tok"][:n]
    pre = O.prefill(model, xp, lay)
    v_cache = O.step(model, pre, tok, d["mods"], d["final_scale"])
    v_joint, _, kv = O.joint_forward(model, xp, tok, lay, d["mods"], d["final_scale"])
    assert _rel(v_cache, v_joint) < 1e-6
    for l in range(model.layers):
        assert _rel(pre.k[l], kv[l][0][:lp]) < 1e-6
        assert _rel(pre.v[l], kv[l][1][:lp]) < 1e-6


def test_f32_oracle_within_bound_of_f64(tiny):
    w, model, d = tiny
    lay = O.Layout(w.layout())
    v32 = O.step(model, O.prefill(model, d["x_prefix"], lay), d["tok"], d["mods"], d["final_scale"])
    p64 = O.prefill(model, d["x_prefix"], lay, dt=F64)
    v64 = O.step(model, p64, d["tok"], d["mods"], d["final_scale"], dt=F64)
    assert _rel(v32, v64) < 1e-5


def test_f16_storage_mode_moves_v_by_rounding_order(tiny):
    # storage="f16" rounds the device design's f16 sites; on the tiny model
    # that moves v by f16 rounding's order, never by an O(1) change
    w, model, d = tiny
    lay = O.Layout(w.layout())
    v32 = O.step(model, O.prefill(model, d["x_prefix"], lay), d["tok"], d["mods"], d["final_scale"])
    p16 = O.prefill(model, d["x_prefix"], lay, storage="f16")
    v16 = O.step(model, p16, d["tok"], d["mods"], d["final_scale"], storage="f16")
    assert 1e-5 < _rel(v16, v32) < 5e-3


def test_f16_store_is_round_to_nearest_even_binary16():
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -24, 2.0 ** -26, 65504.0, 1 / 3], np.float32)
    got = O.store(x, "f16")
    want = np.array([1.0, 1 + 2.0 ** -9, 2.0 ** -24, 0.0, 65504.0, 0.333251953125], np.float32)
    assert np.array_equal(got, want)
    assert O.store(x, None) is x


def test_f16_storage_attention_normalises_by_the_rounded_weights():
    # with V = 1 the output is the sum of the normalised weights: exactly 1
    # when the row sum is taken over the same rounded values that multiply V
    rng = np.random.default_rng(5)
    n, m, hd = 7, 23, 128
    q = rng.standard_normal((n, hd)).astype(np.float32)
    k = rng.standard_normal((m, hd)).astype(np.float32)
    vis = np.array([1, 3, 5, 9, 12, 20, 23])
    out = O.attention(q, k, np.ones((m, hd), np.float32), vis, 1, hd, storage="f16")
    assert np.all(np.abs(out - 1) <= 2 ** -23)
    # one visible key: the output is that key's value row, exactly
    v = rng.standard_normal((m, hd)).astype(np.float32)
    one = O.attention(q, k, v, np.ones(n, int), 1, hd, storage="f16")
    assert np.array_equal(one, np.broadcast_to(v[0], (n, hd)))


def test_softmax_rows_not_flat_on_synthetic_inputs(tiny):
    # the synthetic norm weights (1 + N(0, 0.02)) keep attention peaked
    # enough that the mask matters
    w, model, d = tiny
    g = model.geom
    lay = O.Layout(w.layout())
    lp = lay.prefix_len
    xn = O.norm_mod(d["x_prefix"], model.mods0[:g.dim], g.eps)
    blk = model.block(0)
    rope = O.rope_tables(lay.positions()[:lp], g.axes, g.theta)
    q = O.qk_norm_rope(O.lin(xn, blk["to_q"]), blk["norm_q"], rope[0], rope[1], g.heads, g.head_dim, g.eps)
    k = O.qk_norm_rope(O.lin(xn, blk["to_k"]), blk["norm_k"], rope[0], rope[1], g.heads, g.head_dim, g.eps)
    sc = (q[:, :128] @ k[:, :128].T) / math.sqrt(128)
    assert sc.std() > 0.5


def test_modulation_chunks_route_to_their_branch(tiny):
    # [s1|g1|s2|g2]: with g1 = 0 the attention branch (and s1, to_v) has no
    # effect; with g2 = 0 the FFN branch (and s2, up) has none.  A swap of
    # the chunks' roles fails one of the four checks.
    _, model, d = tiny
    h = model.geom.dim
    x = d["x_prefix"][:8].astype(F64)
    blk = model.block(0)
    rnd = np.random.default_rng(11).normal(0, 0.3, size=h)
    m = d["mods"].astype(F64).copy()
    m[h:2 * h] = 0.0
    base = _one_block(model, x, m)[0]
    m_s1 = m.copy()
    m_s1[:h] += rnd
    assert np.array_equal(_one_block(model, x, m_s1)[0], base)
    assert np.array_equal(_one_block(model, x, m, {"to_v": blk["to_v"] * 2})[0], base)
    m_s2 = m.copy()
    m_s2[2 * h:3 * h] += rnd
    assert _rel(_one_block(model, x, m_s2)[0] - x, base - x) > 1e-3
    m = d["mods"].astype(F64).copy()
    m[3 * h:] = 0.0
    base = _one_block(model, x, m)[0]
    m_s2 = m.copy()
    m_s2[2 * h:3 * h] += rnd
    assert np.array_equal(_one_block(model, x, m_s2)[0], base)
    assert np.array_equal(_one_block(model, x, m, {"up": blk["up"] * 2})[0], base)
    m_s1 = m.copy()
    m_s1[:h] += rnd
    assert _rel(_one_block(model, x, m_s1)[0] - x, base - x) > 1e-3


# ───────────────────────────── time path and sampler ─────────────────────────────

def test_timestep_embedding_hand_values():
    # t = 0: every cosine 1, every sine 0; ts = 1000 t = 1 makes the first
    # frequency (exactly 1) give cos 1, sin 1; the last frequency is
    # 10000^(-127/128); cosines come first
    e0 = O.timestep_embedding(0.0)
    assert np.array_equal(e0[:128], np.ones(128, np.float32)) and np.array_equal(e0[128:], np.zeros(128, np.float32))
    e = O.timestep_embedding(0.001)
    assert e.shape == (256,) and e.dtype == np.float32
    assert abs(e[0] - math.cos(1.0)) < 1e-6 and abs(e[128] - math.sin(1.0)) < 1e-6
    f127 = 10000.0 ** (-127 / 128)
    assert abs(e[127] - math.cos(1.0 * f127)) < 1e-6 and abs(e[255] - math.sin(1.0 * f127)) < 1e-6
    e7 = O.timestep_embedding(0.7)
    for i in (0, 5, 64, 127):
        a = 700.0 * 10000.0 ** (-i / 128)
        assert abs(e7[i] - math.cos(a)) < 2e-4 * max(1.0, a / 100) and abs(e7[128 + i] - math.sin(a)) < 2e-4 * max(1.0, a / 100)


def test_lin_row_accumulates_in_f64():
    # 1e8 + 1 - 1e8 is lost in float32 accumulation, kept in float64
    w = np.array([[1e8, 1.0, -1e8], [2.0, 3.0, 4.0]], np.float32)
    x = np.array([1.0, 1.0, 1.0], np.float32)
    assert np.array_equal(O.lin_row(w, x), np.array([1.0, 9.0], np.float32))


def test_time_mods_structure(tiny):
    _, model, _ = tiny
    tw = dict(model.time())
    mods, fs = O.time_mods(tw, 0.37)
    assert mods.shape == (4 * model.geom.dim,) and fs.shape == (model.geom.dim,)
    # linear in the last projections, which see the same silu(temb)
    t2 = dict(tw, modulation=tw["modulation"] * 2, norm_out=tw["norm_out"] * 4)
    m2, f2 = O.time_mods(t2, 0.37)
    assert np.array_equal(m2, mods * 2) and np.array_equal(f2, fs * 4)
    # a zero first layer: silu(0) = 0 feeds the second, temb = 0, so s = 0
    z = dict(tw, t_lin1=np.zeros_like(tw["t_lin1"]))
    mz, fz = O.time_mods(z, 0.37)
    assert not np.any(mz) and not np.any(fz)
    # the time matters
    m3, _ = O.time_mods(tw, 0.9)
    assert _rel(m3, mods) > 1e-3


def test_time_mods_hand_values():
    # A two-wide time path whose values are worked out by hand at t = 0, where
    # e = [cos 0 ...| sin 0 ...] = [1]*128 + [0]*128 ([QI] Qi21Dit::temb,
    # Qi21Dit::mods).  t_lin1 reads e[0] with weights -3 and 2, so its output
    # is (-3, 2) and h = silu of it = (-0.14227762, 1.76159416); t_lin2 =
    # diag(1, -4) gives temb = (-0.14227762, -7.04637662); the second silu
    # gives s = (-0.06608660, -0.00612894); modulation and norm_out are small
    # integer matrices applied to s.  Dropping either silu, or moving the
    # second one before t_lin2, changes s by more than 100x somewhere.
    t_lin1 = np.zeros((2, 256), np.float32)
    t_lin1[0, 0], t_lin1[1, 0] = -3.0, 2.0
    tw = {
        "t_lin1": t_lin1,
        "t_lin2": np.array([[1.0, 0.0], [0.0, -4.0]], np.float32),
        "modulation": np.array([[1, 0], [0, 1], [2, 0], [0, -1], [1, 1], [0, 0], [-1, 0], [0, 3]], np.float32),
        "norm_out": np.array([[0, 1], [1, 0]], np.float32),
    }
    s0, s1 = -0.06608659926223291, -0.006128941176595901
    mods, fs = O.time_mods(tw, 0.0)
    want_m = [s0, s1, 2 * s0, -s1, s0 + s1, 0.0, -s0, 3 * s1]
    assert np.allclose(mods, want_m, rtol=2e-6, atol=1e-9)
    assert np.allclose(fs, [s1, s0], rtol=2e-6, atol=1e-9)


def test_sampler_steps(tiny):
    w, model, d = tiny
    lay = O.Layout(w.layout())
    pre = O.prefill(model, d["x_prefix"], lay)
    tok = d["tok"]
    # no time elapses: no change
    assert np.array_equal(O.sample(model, pre, tok, [0.6, 0.6]), tok)
    # one step is x + (t1 - t0) v with v the step at the modulation of t0
    mods, fs = O.time_mods(model.time(), 0.6)
    v = O.step(model, pre, tok, mods, fs)
    one = O.sample(model, pre, tok, [0.6, 0.35])
    assert np.array_equal(one, (tok + (np.float32(0.35) - np.float32(0.6)) * v).astype(np.float32))
    # two steps start the second from the first's result
    two = O.sample(model, pre, tok, [0.6, 0.35, 0.1])
    m2, f2 = O.time_mods(model.time(), 0.35)
    v2 = O.step(model, pre, one, m2, f2)
    assert np.array_equal(two, (one + (np.float32(0.1) - np.float32(0.35)) * v2).astype(np.float32))


# ───────────────────────────── txt_in front ─────────────────────────────

def test_gelu_tanh_values():
    g = O.gelu_tanh(np.array([0.0, 1.0, -1.0, 3.0, -6.0], np.float32))
    # 0.5 x (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3))) by hand
    want = [0.0, 0.8411919906, -0.1588080094, 2.9963625, -0.0]
    assert np.allclose(g, want, rtol=0, atol=2e-7)


def test_embed_text_norm_and_structure():
    rng = np.random.default_rng(3)
    n, c, d = 5, 64, 48
    feats = rng.standard_normal((n, c)).astype(np.float32)
    w0 = np.zeros(c, np.float32)
    eye = np.eye(d, c, dtype=np.float32)
    ident = np.eye(d, dtype=np.float32)
    # zero-centred weight 0 scales by 1; identity projections expose
    # gelu(rms-normalised features), whose mean square is 1 before the gelu
    out = O.embed_text(feats, w0, eye, ident, 1e-6)
    xn = feats / np.sqrt((feats.astype(np.float64) ** 2).mean(axis=1, keepdims=True) + 1e-6)
    assert np.allclose(out, O.gelu_tanh(xn[:, :d]), rtol=0, atol=1e-6)
    # a constant row normalises to +-1; the weight w scales it by (w + 1)
    const = np.full((1, c), -7.0, np.float32)
    w = np.full(c, 0.5, np.float32)
    o2 = O.embed_text(const, w, eye, ident, 0.0)
    assert np.allclose(o2, O.gelu_tanh(np.full((1, d), -1.5, np.float32)), rtol=0, atol=1e-7)
    # scale invariance of the norm (eps = 0): features x 8 give the same rows
    assert np.array_equal(O.embed_text(feats * 8, w0, eye, ident, 0.0), O.embed_text(feats, w0, eye, ident, 0.0))


def test_embed_text_gelu_sits_between_the_projections():
    # [QI] Qi21Dit::embed_text: txt_in1, then the tanh GELU, then txt_in2.
    # Row 0 (constant -7) normalises to -1 and the weight w = 0.5 scales it
    # to (-1.5, -1.5); row 1 (3, -3) becomes (1.5, -1.5).  txt_in1 =
    # diag(2, 1) gives (-3, -1.5) and (3, -1.5); the GELU gives (gelu(-3),
    # gelu(-1.5)) and (gelu(3), gelu(-1.5)); txt_in2 doubles and swaps the
    # two columns: (2 gelu(-1.5), 2 gelu(-3)) = (-0.20085685, -0.00727478)
    # and (2 gelu(-1.5), 2 gelu(3)) = (-0.20085685, 5.99272522).  The GELU
    # before txt_in1 gives 2 gelu(-1.5) * 2 in column 1 of row 0; after
    # txt_in2 it gives gelu(-3) in column 0; a transposed txt_in2 or txt_in1
    # swaps the columns.
    feats = np.array([[-7.0, -7.0], [3.0, -3.0]], np.float32)
    w = np.full(2, 0.5, np.float32)
    d21 = np.diag([2.0, 1.0]).astype(np.float32)
    swap2 = np.array([[0.0, 2.0], [2.0, 0.0]], np.float32)
    out = O.embed_text(feats, w, d21, swap2, 0.0)
    want = np.array([[-0.20085684603953413, -0.007274784163545989], [-0.20085684603953413, 5.992725215836454]])
    assert np.allclose(out, want, rtol=1e-6, atol=1e-7)
