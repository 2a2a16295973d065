"""Parity at the full-size workloads' shapes, in the launch configuration the
benchmark times (needs a GPU).

Each kernel runs through the C ABI on seeded inputs generated in device
memory; the oracle recomputes a sample of the outputs one by one from the
same seeded values regenerated on the host (the generator is indexable, so
only the rows a sample touches are produced).  End to end, the step's
velocity at 512^2, 1024^2, with the condition-image prefix and for the CFG
pair is compared with the oracle's stored output (written by
``tests/golden/make_oracle_golden.py`` from the oracle alone).

End-to-end tolerances.  The benchmark's configuration keeps the FFN input
and SwiGLU hidden in the lo4 form (QI21_FFN_LO4: f16 plus a scaled fp4
residual); it, the lo8 form (fp8 residual) and the f16-pair form
(QI21_FFN_PAIR) are held to the 1e-3 relative L2 bar on v, and every target row compared to 3e-3 relative L2
over its 64 channels (a row-local fault a few times the bar fails it even
where the global figure hides it).  With every site in single f16 (the
pages' design) the error after 32 blocks of these N(0, 0.02) weights is
the storage's own: the oracle run with the same sites rounded to f16 (its
``storage="f16"`` mode) is itself ~1.8e-3 from the f32 oracle at 512^2,
growing as the square root of the depth from ~3e-4 per block.  That path
is therefore bounded by 1.5x that storage error, measured on the same
workload, not by 1e-3.
"""
import os

import numpy as np
import pytest

import bench
import inputs
from inputs import CONFIGS
from oracle import qi21_oracle as O
from parity import ROW_FACTOR, assert_close, rowrel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F16_TOL = 2e-3
F32_TOL = 1e-5
V_TOL = 1e-3
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def Q():
    from diffusion_transformer_denoiser_qi21_amd import qi21
    return qi21


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def dev_f16(seed, tid, shape, sigma):
    return inputs.device_tensor(seed, tid, shape, sigma).half()


def host_rows_f16(seed, tid, ncols, rows, sigma):
    """rows of a seeded [*, ncols] matrix, rounded to f16 like the device copy"""
    return np.stack([inputs.host_array(seed, tid, (ncols,), sigma, start=int(r) * ncols) for r in rows]) \
        .astype(np.float16).astype(np.float32)


H, I, N1024 = 4096, 12288, 4096


@pytest.mark.parametrize("site", ["qkv", "o", "gate_up", "down"])
def test_gemm_sites_at_1024_sampled(site):
    q = Q()
    M = N1024
    N, K, epi = {"qkv": (3 * H, H, q.QI21_EPI_QKV), "o": (H, H, q.QI21_EPI_F32),
                 "gate_up": (2 * I, H, q.QI21_EPI_SWIGLU), "down": (H, I, q.QI21_EPI_F32)}[site]
    seed = 4000 + N
    A = dev_f16(seed, 1, (M, K), 1.0)
    rng = np.random.default_rng(N + K)
    rows = np.sort(rng.choice(M, 64, replace=False))
    Ah = host_rows_f16(seed, 1, K, rows, 1.0)
    scale = 0.5
    if site == "gate_up":
        G = dev_f16(seed, 2, (I, K), 0.02)
        U = dev_f16(seed, 3, (I, K), 0.02)
        w13 = torch.empty(2 * I, K, device="cuda", dtype=torch.float16)
        q.qi21_op_plane(q.QI21_F16, G, I, K, w13, 32, 64, 0)
        q.qi21_op_plane(q.QI21_F16, U, I, K, w13, 32, 64, 32)
        out = torch.empty(M, I, device="cuda", dtype=torch.float16)
        q.qi21_op_gemm(epi, M, 2 * I, K, A, K, w13, out, I, oscale=scale, inscale=4.0)
        torch.cuda.synchronize()
        cols = np.sort(rng.choice(I, 96, replace=False))
        g = O.lin(Ah, host_rows_f16(seed, 2, K, cols, 0.02)) * np.float32(4.0)
        u = O.lin(Ah, host_rows_f16(seed, 3, K, cols, 0.02)) * np.float32(4.0)
        want = O.silu(g) * u * np.float32(scale)
        got = out.float().cpu().numpy()[np.ix_(rows, cols)]
        assert_close(got, want, F16_TOL)
        return
    W = dev_f16(seed, 2, (N, K), 0.02)
    cols = np.sort(rng.choice(N, 96, replace=False))
    want = O.lin(Ah, host_rows_f16(seed, 2, K, cols, 0.02)) * np.float32(scale)
    if site == "qkv":
        out = torch.empty(M, 2 * H, device="cuda", dtype=torch.float16)
        vt = torch.empty(H, M, device="cuda", dtype=torch.float16)
        q.qi21_op_gemm(epi, M, N, K, A, K, W, out, 2 * H, vt, M, oscale=scale)
        torch.cuda.synchronize()
        o_ = out.float().cpu().numpy()
        v_ = vt.float().cpu().numpy()
        got = np.stack([o_[rows, c] if c < 2 * H else v_[c - 2 * H, vt_pos(rows)] for c in cols], axis=1)
        assert_close(got, want, F16_TOL)
    else:
        out = torch.empty(M, N, device="cuda")
        q.qi21_op_gemm(epi, M, N, K, A, K, W, out, N, oscale=scale)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy()[np.ix_(rows, cols)], want, F32_TOL)


def vt_pos(j):
    """column of key j in a V^T row: bits 2 and 3 of j swapped"""
    j = np.asarray(j)
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1)


def _vt_dev(v_dev, ld):
    """device V [n][H] f16 -> V^T [H][ld] f16 in the attention kernel's key order, zero padding"""
    n = v_dev.shape[0]
    out = torch.zeros(v_dev.shape[1], ld, device="cuda", dtype=torch.float16)
    out[:, torch.from_numpy(vt_pos(np.arange(n))).cuda()] = v_dev.t()
    return out


@pytest.mark.parametrize("case", ["step1024", "cond_prefill", "step2048"])
def test_flash_full_shape_sampled(case):
    q = Q()
    heads, hd = 32, 128
    vis = None
    if case == "step1024":
        nq, n1, n2 = 4096, 18, 4096
    elif case == "step2048":
        nq, n1, n2 = 16384, 18, 16384
    else:
        lay = O.Layout([("text", 22), ("image", 64, 64), ("image", 64, 64)])
        vis = O.prefix_visibility(lay)
        nq, n1, n2 = lay.prefix_len, lay.prefix_len, 0
    m = n1 + n2
    seed = 7000 + nq
    # q in the kernel's base-2 units: f16 of (f16 q) * f32(log2(e) / sqrt(128))
    ql2 = np.log2(np.e) / np.sqrt(128.0)
    qd = (dev_f16(seed, 1, (nq, H), 1.0).float() * float(np.float32(ql2))).half()
    kd = dev_f16(seed, 2, (m, H), 1.0)
    vd = dev_f16(seed, 3, (m, H), 1.0)
    ld1 = (n1 + 63) // 64 * 64
    ld2 = (max(n2, 1) + 63) // 64 * 64
    k1, vt1 = kd[:n1].contiguous(), _vt_dev(vd[:n1], ld1)
    k2 = kd[n1:].contiguous() if n2 else None
    vt2 = _vt_dev(vd[n1:], ld2) if n2 else None
    dvis = torch.from_numpy(vis.astype(np.int32)).cuda() if vis is not None else None
    out = torch.empty(nq, H, device="cuda", dtype=torch.float16)
    q.qi21_op_flash(nq, heads, qd, H, k1, H, vt1, ld1, n1, k2, H, vt2, ld2, n2, dvis, out, H, 1.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(nq)
    rows = np.sort(np.concatenate([rng.choice(nq, 24, replace=False), [0, 5, 21, 22, nq - 1]]))
    qh = (host_rows_f16(seed, 1, H, rows, 1.0).astype(np.float32) * np.float32(ql2)).astype(np.float16)
    qh = qh.astype(np.float64) / ql2
    kh = inputs.host_array(seed, 2, (m, H), 1.0).astype(np.float16).astype(np.float32)
    vh = inputs.host_array(seed, 3, (m, H), 1.0).astype(np.float16).astype(np.float32)
    visible = vis[rows] if vis is not None else np.full(len(rows), m, np.int64)
    want = O.attention(qh, kh, vh, visible, heads, hd)
    assert_close(out.float().cpu().numpy()[rows], want, F16_TOL)


# The 8-wave form (one block of 256 queries per CU, at least two rounds:
# 4096 queries x 32 heads) with key counts that end both sources inside a
# tile, a single tile per source, and a prefix-only pass: its tail masks
# and its short loops, on sampled rows against the oracle.
@pytest.mark.parametrize("n1,n2", [(37, 4133), (5, 60), (64, 64), (18, 0), (130, 257)])
def test_flash_eight_wave_ragged_keys(n1, n2):
    q = Q()
    heads, hd = 32, 128
    nq = 4096 + 64 if (n1, n2) == (64, 64) else 4096  # and a partial last query block
    m = n1 + n2
    seed = 7100 + n1 + n2
    ql2 = np.log2(np.e) / np.sqrt(128.0)
    qd = (dev_f16(seed, 1, (nq, H), 1.0).float() * float(np.float32(ql2))).half()
    kd = dev_f16(seed, 2, (m, H), 1.0)
    vd = dev_f16(seed, 3, (m, H), 1.0)
    ld1 = (n1 + 63) // 64 * 64
    ld2 = (max(n2, 1) + 63) // 64 * 64
    k1, vt1 = kd[:n1].contiguous(), _vt_dev(vd[:n1], ld1)
    k2 = kd[n1:].contiguous() if n2 else None
    vt2 = _vt_dev(vd[n1:], ld2) if n2 else None
    out = torch.full((nq, H), 7.0, device="cuda", dtype=torch.float16)
    q.qi21_op_flash(nq, heads, qd, H, k1, H, vt1, ld1, n1, k2, H, vt2, ld2, n2, None, out, H, 1.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = np.sort(np.unique(np.concatenate([rng.choice(nq, 20, replace=False), [0, 31, 32, 255, 256, nq - 1]])))
    qh = (host_rows_f16(seed, 1, H, rows, 1.0).astype(np.float32) * np.float32(ql2)).astype(np.float16)
    qh = qh.astype(np.float64) / ql2
    kh = inputs.host_array(seed, 2, (m, H), 1.0).astype(np.float16).astype(np.float32)
    vh = inputs.host_array(seed, 3, (m, H), 1.0).astype(np.float16).astype(np.float32)
    want = O.attention(qh, kh, vh, np.full(len(rows), m, np.int64), heads, hd)
    got = out.float().cpu().numpy()[rows]
    g, r = rel(got, want), rowrel(got, want)
    print(f"flash 8-wave n1 {n1} n2 {n2}: rel L2 {g:.3e}, worst row {r:.3e}")
    assert g < F16_TOL and r < ROW_FACTOR * F16_TOL


def test_rowop_full_shape_sampled():
    q = Q()
    rows, h = N1024, H
    x = inputs.device_tensor(31, 1, (rows, h), 1.0)
    y = inputs.device_tensor(31, 2, (rows, h), 0.5)
    mods = inputs.device_tensor(31, 3, (4 * h,), 0.1)
    xn = torch.empty(rows, h, device="cuda", dtype=torch.float16)
    q.qi21_op_rowop(rows, h, 3, x, y, xn, h, mods, 3 * h, 0, 1e-6, 0.25)
    torch.cuda.synchronize()
    sample = np.sort(np.random.default_rng(3).choice(rows, 32, replace=False))
    xh = np.stack([inputs.host_array(31, 1, (h,), 1.0, start=int(r) * h) for r in sample])
    yh = np.stack([inputs.host_array(31, 2, (h,), 0.5, start=int(r) * h) for r in sample])
    mh = inputs.host_array(31, 3, (4 * h,), 0.1)
    xe = O.gated_add(xh, yh, mh[3 * h:])
    assert_close(x.cpu().numpy()[sample], xe, 1e-6)
    want = O.norm_mod(xe, mh[:h], 1e-6) * np.float32(0.25)
    assert_close(xn.float().cpu().numpy()[sample], want, F16_TOL)


# ───────────────────────────── end to end ─────────────────────────────

ROW_TOL = 3e-3


def _full(opt_mode=None):
    q = Q()
    opt = q.qi21_default_options()
    if opt_mode is not None:
        opt.ffn_mode = opt_mode
    return bench.build_model(CONFIGS["1024"].model, opt)


@pytest.fixture(scope="module")
def full_model():
    m = _full()
    yield m
    Q().qi21_model_destroy(m)


@pytest.fixture(scope="module")
def full_model_pair():
    m = _full(Q().QI21_FFN_PAIR)
    yield m
    Q().qi21_model_destroy(m)


@pytest.fixture(scope="module")
def full_model_lo8():
    m = _full(Q().QI21_FFN_LO8)
    yield m
    Q().qi21_model_destroy(m)


@pytest.fixture(scope="module")
def full_model_lo4():
    m = _full(Q().QI21_FFN_LO4)
    yield m
    Q().qi21_model_destroy(m)


def _golden(name, p=0, tag=""):
    import glob
    f = glob.glob(os.path.join(GOLD, f"oracle_v_{name}_p{p}{tag}_rows*.npy"))
    if not f:
        pytest.skip(f"no stored oracle output {name}{tag} (tests/golden/make_oracle_golden.py)")
    stride = int(f[0].rsplit("rows", 1)[1].split(".")[0])
    return np.load(f[0]), stride


def _step_v(m, w, key, stride):
    d = bench.workload_tensors(w)
    bench.prefill(m, key, d)
    out = torch.full((d["n"], 64), 7.0, device="cuda")
    Q().qi21_step(m, key, d["tok"], d["mods"], d["fs"], out)
    Q().qi21_release_key(m, key)
    return out.cpu().numpy()[::stride]


def _check_v(got, want, label):
    err = rel(got, want)
    g, w = np.asarray(got, np.float64), np.asarray(want, np.float64)
    rows = np.linalg.norm(g - w, axis=1) / np.linalg.norm(w, axis=1)
    print(f"{label}: v rel L2 vs oracle {err:.3e}, worst row {rows.max():.3e} (row {int(rows.argmax())})")
    assert err < V_TOL
    assert rows.max() < ROW_TOL


@pytest.mark.parametrize("mode", ["lo4", "lo8"])
@pytest.mark.parametrize("name", ["512", "1024", "cond", "ragged", "2048"])
def test_step_full_size_residual_forms_against_oracle(request, mode, name):
    # lo4 is the configuration bench.py times.  ragged: 4087 target rows
    # behind 37 prefix rows, so the last row tile of every GEMM, the last
    # V^T columns and the last key tile of attention are partial on the
    # large-pass path
    m = request.getfixturevalue(f"full_model_{mode}")
    want, stride = _golden(name)
    _check_v(_step_v(m, CONFIGS[name], 52, stride), want, f"{name} ({mode})")


@pytest.mark.parametrize("name", ["512", "1024", "cond", "ragged", "2048"])
def test_step_full_size_pair_against_oracle(full_model_pair, name):
    want, stride = _golden(name)
    _check_v(_step_v(full_model_pair, CONFIGS[name], 50, stride), want, f"{name} (pair)")


@pytest.mark.parametrize("name", ["512", "1024"])
def test_step_full_size_single_f16_within_storage_error(full_model, name):
    want, stride = _golden(name)
    want16, stride16 = _golden(name, tag="_f16")
    storage = rel(want16, want[::stride16 // stride])  # what f16 storage alone costs, per the oracle
    err = rel(_step_v(full_model, CONFIGS[name], 51, stride), want)
    print(f"{name} (single f16): v rel L2 vs oracle {err:.3e}; oracle f16-storage error {storage:.3e}")
    assert storage > V_TOL  # the reason this path has its own bound
    assert err < 1.5 * storage


@pytest.mark.parametrize("mode", ["lo4", "lo8", "pair"])
def test_cfg_pair_full_size_against_oracle(request, mode):
    m = request.getfixturevalue(f"full_model_{mode}")
    w = CONFIGS["cfg512"]
    wants = [_golden("cfg512", p) for p in range(2)]
    ds = [bench.workload_tensors(w, p) for p in range(2)]
    for p in range(2):
        bench.prefill(m, 60 + p, ds[p])
    outs = [torch.zeros(d["n"], 64, device="cuda") for d in ds]
    Q().qi21_step_batch(m, [60, 61], [d["tok"] for d in ds], ds[0]["mods"], ds[0]["fs"], outs)
    for p in range(2):
        want, stride = wants[p]
        _check_v(outs[p].cpu().numpy()[::stride], want, f"cfg prefix {p} ({mode})")
    for p in range(2):
        Q().qi21_release_key(m, 60 + p)


def test_step_1024_gate_zero_closed_form_and_determinism(full_model):
    # with both gates zero every block is the identity, so v is
    # (LN(tok img_in^T) * fs) proj_out^T, which the oracle computes row by
    # row; the same step twice is bitwise identical
    w = CONFIGS["1024"]
    spec = w.model
    d = bench.workload_tensors(w)
    bench.prefill(full_model, 70, d)
    mods = d["mods"].clone()
    mods[spec.dim:2 * spec.dim] = 0
    mods[3 * spec.dim:] = 0
    a = torch.zeros(d["n"], 64, device="cuda")
    b = torch.zeros(d["n"], 64, device="cuda")
    Q().qi21_step(full_model, 70, d["tok"], mods, d["fs"], a)
    Q().qi21_step(full_model, 70, d["tok"], mods, d["fs"], b)
    assert torch.equal(a, b)
    from inputs.configs import TID_FINAL_SCALE, TID_IMG_IN, TID_PROJ_OUT, TID_TOK, W_SIGMA, MOD_SIGMA
    img_in = inputs.host_array(spec.seed, TID_IMG_IN, (spec.dim, 64), W_SIGMA, bf16=True)
    proj_out = inputs.host_array(spec.seed, TID_PROJ_OUT, (64, spec.dim), W_SIGMA, bf16=True)
    fsc = inputs.host_array(w.seed, TID_FINAL_SCALE, (spec.dim,), MOD_SIGMA)
    rows = np.arange(0, d["n"], 37)
    tok = np.stack([inputs.host_array(w.seed, TID_TOK, (64,), 1.0, start=int(r) * 64) for r in rows])
    want = O.final_layer(O.embed_image(tok, img_in), fsc, proj_out, spec.eps)
    assert_close(a.cpu().numpy()[rows], want, V_TOL)
    Q().qi21_release_key(full_model, 70)


def test_time_mods_full_size():
    # the full model's time path (bf16 weights widened to f32, f64 sums)
    from oracle import SynthModel
    spec = CONFIGS["1024"].model
    q = Q()
    m = bench.build_model(spec, time_path=True)
    try:
        mods = torch.zeros(4 * spec.dim, device="cuda")
        fs = torch.zeros(spec.dim, device="cuda")
        q.qi21_time_mods(m, 0.81, mods, fs)
        torch.cuda.synchronize()
        want_m, want_f = O.time_mods(SynthModel(spec, cache_layers=0).time(), 0.81)
        assert_close(mods.cpu().numpy(), want_m, 1e-5)
        assert_close(fs.cpu().numpy(), 1.0 + want_f, 1e-6)
    finally:
        q.qi21_model_destroy(m)


def test_txt_in_full_size():
    from oracle import SynthModel
    from inputs.configs import TID_TXT_FEATS
    spec = CONFIGS["1024"].model
    q = Q()
    m = bench.build_model(spec, txt_in=True)
    try:
        n = 22
        f = inputs.host_array(5, TID_TXT_FEATS, (n, spec.dim), 1.0)
        out = torch.zeros(n, spec.dim, device="cuda")
        q.qi21_txt_in(m, n, torch.from_numpy(f).cuda(), out)
        torch.cuda.synchronize()
        t = SynthModel(spec, cache_layers=0).txt()
        want = O.embed_text(f, t["txt_norm"], t["txt_in1"], t["txt_in2"], spec.eps)
        assert_close(out.cpu().numpy(), want, 2e-3)
    finally:
        q.qi21_model_destroy(m)
