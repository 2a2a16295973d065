"""Parity of the lo8 kernels (the QI21_FFN_LO8 storage of the FFN sites;
needs a GPU).

A lo8 value is hi = f16(v) plus the residual v - hi in OCP e4m3 (fp8)
times a power-of-two scale; rows are grouped by 128 columns (128 halves,
then their 128 fp8 bytes).  The checks below decode what the kernels wrote
with a plain e4m3 definition (sign, 4 exponent bits with bias 7, 3
mantissa bits; exponent 0 subnormal; S.1111.111 NaN; no infinities) and
compare with the oracle's f32 functions on the same inputs:

* the fp8 conversion itself: round to nearest, ties to even, in the OCP
  encoding (a mismatch of format, e.g. the bias-8 variant, or of rounding
  fails it);
* the weight plane: f16 values bit-exact, fp8 copy bit-exact against the
  encoder, per-row scale by its rule;
* the row op writing the FFN input: the decoded value within 2^-14 of
  each row's largest magnitude from the oracle's f32 value, per row;
* the GEMM on random lo8 operands (every byte pattern but NaN, random
  scales), each epilogue, against an f64 sum of the decoded operands;
* the three FFN kernels chained at the 1024^2 step's shape against the
  oracle's f32 FFN on sampled rows.
"""
import numpy as np
import pytest

import inputs
from oracle import qi21_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def Q():
    from diffusion_transformer_denoiser_qi21_amd import qi21
    return qi21


def sync():
    torch.cuda.synchronize()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


# ───────────────────────────── e4m3 and the lo8 row form ─────────────────────────────

def e4m3_decode(b):
    """OCP e4m3 byte(s) -> float64 (NaN for S.1111.111)"""
    b = np.asarray(b, np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    return np.where((e == 15) & (m == 7), np.nan, s * v)


_CODES = np.arange(256)
_VALS = e4m3_decode(_CODES)
_FIN = np.isfinite(_VALS)


def e4m3_encode(x):
    """float -> nearest finite OCP e4m3 code, ties to the even mantissa (x
    within the finite range); a negative value that rounds to zero gives -0
    (the sign is kept, as in IEEE rounding)"""
    x = np.asarray(x, np.float64).ravel()
    codes, vals = _CODES[_FIN], _VALS[_FIN]
    d = np.abs(x[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes prefer an even mantissa, then +0 over -0
    score = cand * (2 + ((codes[None, :] & 1) == 0) * 2 + (codes[None, :] == 0))
    out = codes[np.argmax(score, axis=1)]
    out = np.where(np.signbit(x) & (out == 0), 0x80, out)
    return out.reshape(np.shape(x))


def lo8_split(buf, ncols):
    """rows of a lo8 buffer (uint8 [rows][>= 3 ncols]) -> (hi f64, fp8 codes)"""
    rows = buf.shape[0]
    g = buf[:, :3 * ncols].reshape(rows, ncols // 128, 384)
    hi = g[:, :, :256].copy().view(np.float16).reshape(rows, ncols).astype(np.float64)
    codes = g[:, :, 256:].reshape(rows, ncols)
    return hi, codes


def lo8_join(hi16, codes):
    """(f16 [rows][n], uint8 codes [rows][n]) -> a lo8 buffer uint8 [rows][3n]"""
    rows, n = hi16.shape
    g = np.empty((rows, n // 128, 384), np.uint8)
    g[:, :, :256] = np.ascontiguousarray(hi16.astype(np.float16)).view(np.uint8).reshape(rows, n // 128, 256)
    g[:, :, 256:] = codes.reshape(rows, n // 128, 128)
    return g.reshape(rows, 3 * n)


def lo8_value(buf, ncols, sc, block):
    """the value a lo8 buffer represents: hi + e4m3 * 2^(scale - 127), one
    scale per `block` columns (64: activations, ncols: a weight row)"""
    hi, codes = lo8_split(buf, ncols)
    f = 2.0 ** (np.repeat(np.asarray(sc, np.float64).reshape(buf.shape[0], -1), block, axis=1)[:, :ncols] - 127.0)
    return hi + e4m3_decode(codes) * f


def _expected_scale(mx):
    """the scale rule: e with mx 2^-e in [128, 256) (mx > 0, normal)"""
    return np.floor(np.log2(mx)).astype(np.int64) - 7


# ───────────────────────────── fp8 conversion and weight planes ─────────────────────────────

def test_e4m3_conversion_is_ocp_round_to_nearest_even():
    """A weight row whose largest |w| is 240 keeps scale 2^0 (240 in [128,
    256)), so its fp8 copy is the plain conversion of its values: every
    finite e4m3 value, the midpoints between neighbours (ties) and points
    a quarter of a step from them, and subnormals."""
    q = Q()
    fin = np.sort(np.unique(_VALS[_FIN & (_VALS >= 0)]))
    fin = fin[fin <= 240]
    mids = (fin[:-1] + fin[1:]) / 2
    quarter = fin[:-1] + (fin[1:] - fin[:-1]) / 4
    vals = np.concatenate([fin, mids, quarter, -fin[1:], -mids])
    vals = vals[np.abs(vals.astype(np.float16).astype(np.float64) - vals) == 0]  # exactly representable in f16
    n = (len(vals) + 127) // 128 * 128
    row = np.zeros(n, np.float64)
    row[:len(vals)] = vals
    row[-1] = 240.0
    w = row.astype(np.float16)[None, :]
    plane = torch.zeros(1, 3 * n // 2, device="cuda", dtype=torch.float16)
    sc = torch.zeros(1, device="cuda", dtype=torch.uint8)
    q.qi21_op_plane_lo8(q.QI21_F16, dev(w), 1, n, plane, 3 * n // 2, 1, 0, 0)
    q.qi21_op_plane8(1, n, plane, 3 * n // 2, sc)
    sync()
    hi, codes = lo8_split(plane.cpu().numpy().view(np.uint8), n)
    assert int(sc.cpu()[0]) == 127
    assert np.array_equal(hi[0], w[0].astype(np.float64))
    want = e4m3_encode(w[0].astype(np.float64))
    assert np.array_equal(codes[0], want.astype(np.uint8))


@pytest.mark.parametrize("rows,cols,group", [(300, 384, 300), (96, 256, 32)])
def test_plane_lo8_layout_and_scales(rows, cols, group):
    """f16 values bit-exact at their grouped positions, the fp8 copy
    bit-exact against the encoder at the row's scale, the scale by its rule;
    with group 32 the rows land interleaved as the gate/up plane's"""
    q = Q()
    w = inputs.host_array(41, 1, (rows, cols), 0.02)
    w[5] *= 1e3  # one row far from the others' scale
    ld = 3 * cols // 2
    inter = group < rows  # the gate/up interleave (group 32), else the plain row order
    prow = 2 * rows if inter else rows
    plane = torch.zeros(prow, ld, device="cuda", dtype=torch.float16)
    sc = torch.zeros(prow, device="cuda", dtype=torch.uint8)
    gstride = 64 if inter else 0
    q.qi21_op_plane_lo8(q.QI21_F32, dev(w), rows, cols, plane, ld, group, gstride, 0)
    if inter:
        q.qi21_op_plane_lo8(q.QI21_F32, dev(-w), rows, cols, plane, ld, group, gstride, 32)
    q.qi21_op_plane8(prow, cols, plane, ld, sc)
    sync()
    buf = plane.cpu().numpy().view(np.uint8)
    hi, codes = lo8_split(buf, cols)
    s = sc.cpu().numpy().astype(np.int64)
    dst = (np.arange(rows) // group) * gstride + np.arange(rows) % group if inter else np.arange(rows)
    w16 = w.astype(np.float16).astype(np.float64)
    assert np.array_equal(hi[dst], w16)
    if inter:
        assert np.array_equal(hi[dst + 32], -w16)
    for r in range(prow):
        e = _expected_scale(np.abs(hi[r]).max())
        assert s[r] == e + 127
        assert np.array_equal(codes[r], e4m3_encode(hi[r] * 2.0 ** -e).astype(np.uint8))


# ───────────────────────────── the FFN-input row op ─────────────────────────────

def _check_lo8_rows(buf, xsc, h, want):
    """decoded rows against want: per row, error within 2^-14 of the row's
    largest |want|; hi is the f16 of the represented value; scale rule"""
    v = lo8_value(buf, h, xsc, 64)
    hi, codes = lo8_split(buf, h)
    res = e4m3_decode(codes) * 2.0 ** (np.repeat(xsc.astype(np.float64), 64, axis=1) - 127.0)
    assert np.isfinite(v).all()
    err = np.abs(v - want).max(axis=1)
    assert (err <= 2.0 ** -14 * np.abs(want).max(axis=1)).all(), err.max()
    # the residual is below half an f16 step of hi (plus the fp8 rounding)
    ulp = np.spacing(np.abs(hi).astype(np.float16)).astype(np.float64)
    assert (np.abs(res) <= 0.5 * ulp * (1 + 2.0 ** -3) + 1e-30).all()
    # each 64-column block's largest |residual| / scale lies in [128, 256]
    # (256 only where the fp8 rounding carried the largest one up)
    blk = np.abs(e4m3_decode(codes)).reshape(buf.shape[0], h // 64, 64).max(axis=2)
    nz = blk > 0
    assert ((blk[nz] >= 128) & (blk[nz] <= 256)).all()


@pytest.mark.parametrize("rows,h,mode,nparts", [(1, 256, 2, 1), (37, 256, 3, 1), (300, 4096, 3, 3),
                                                (2049, 4096, 2, 1), (5, 8192, 3, 4), (64, 1280, 3, 1)])
def test_rowop_lo8(rows, h, mode, nparts):
    """the modulated LayerNorm (after the gated residual of nparts planes
    for mode 3) written in the lo8 form, both row-pass forms (one wave per
    row below 2048 columns, one block per row above)"""
    q = Q()
    x = inputs.host_array(51, 1, (rows, h), 1.0)
    y = inputs.host_array(51, 2, (nparts, rows, h), 0.5)
    mods = inputs.host_array(51, 3, (4 * h,), 0.1)
    g_off, s_off, eps, oscale = 3 * h, 2 * h, 1e-6, 0.25
    dx = dev(x)
    ldxn = 3 * h // 2 + 64  # a padded row stride
    xn = torch.zeros(rows, ldxn, device="cuda", dtype=torch.float16)
    xsc = torch.zeros(rows, h // 64, device="cuda", dtype=torch.uint8)
    q.qi21_op_rowop_lo8(rows, h, mode, dx, dev(y), nparts, rows * h, xn, ldxn, xsc, dev(mods), g_off, s_off, eps,
                        oscale)
    sync()
    xe = x
    if mode & 1:
        xe = O.gated_add(x, y.sum(axis=0, dtype=np.float32), mods[g_off:g_off + h])
        assert np.abs(dx.cpu().numpy() - xe).max() <= 1e-5 * np.abs(xe).max()
    want = O.norm_mod(xe, mods[s_off:s_off + h], eps, dt=np.float64) * oscale
    buf = xn.cpu().numpy().view(np.uint8)
    assert not buf[:, 3 * h:].any()  # the padding is not written
    _check_lo8_rows(buf, xsc.cpu().numpy(), h, want)


# ───────────────────────────── the lo8 GEMM ─────────────────────────────

def _random_lo8(rng, rows, cols, hi_sigma, block, sc_lo, sc_hi):
    """random lo8 rows: f16 values, any non-NaN fp8 byte, random scales"""
    hi = (rng.standard_normal((rows, cols)) * hi_sigma).astype(np.float16)
    codes = rng.integers(0, 256, (rows, cols)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11
    sc = rng.integers(sc_lo, sc_hi + 1, (rows, max(cols // block, 1))).astype(np.uint8)
    return hi, codes, sc


def _decoded(hi, codes, sc, block):
    return hi.astype(np.float64), e4m3_decode(codes) * 2.0 ** (
        np.repeat(sc.astype(np.float64), block, axis=1)[:, :hi.shape[1]] - 127.0)


@pytest.mark.parametrize("M", [1, 77, 300, 1040])
@pytest.mark.parametrize("epi", ["f32", "resid", "split", "swiglu8"])
def test_gemm_lo8_epilogues(epi, M):
    q = Q()
    rng = np.random.default_rng(1000 + M)
    N, K = (512, 256) if epi == "swiglu8" else (256, 384)
    ahi, acod, asc = _random_lo8(rng, M, K, 1.0, 64, 108, 116)
    whi, wcod, wsc = _random_lo8(rng, N, K, 0.05, K, 110, 116)
    A = dev(lo8_join(ahi, acod))
    W = dev(lo8_join(whi, wcod))
    da, ds = dev(asc), dev(wsc[:, 0].copy())
    a_h, a_l = _decoded(ahi, acod, asc, 64)
    w_h, w_l = _decoded(whi, wcod, wsc, K)
    acc = a_h @ w_h.T + a_l @ w_l.T
    oscale = 0.5
    if epi in ("f32", "split"):
        ks = 3 if epi == "split" else 1
        out = torch.full((ks, M, N), float("nan"), device="cuda")
        q.qi21_op_gemm_lo8(q.QI21_EPI_F32, M, N, K, A, 3 * K // 2, da, K // 64, W, 3 * K // 2, ds, out, N,
                           ksplit=ks, oscale=oscale)
        sync()
        o = out.cpu().numpy().astype(np.float64)
        for p in range(ks):  # each plane its own third of the columns
            c = slice(p * K // ks, (p + 1) * K // ks)
            want_p = (a_h[:, c] @ w_h[:, c].T + a_l[:, c] @ w_l[:, c].T) * oscale
            assert np.abs(o[p] - want_p).max() <= 1e-5 * np.abs(want_p).max()
        assert np.abs(o.sum(axis=0) - acc * oscale).max() <= 1e-5 * np.abs(acc * oscale).max()
    elif epi == "resid":
        x0 = rng.standard_normal((M, N)).astype(np.float32)
        gate = rng.standard_normal(N).astype(np.float32) * 0.1
        x = dev(x0)
        q.qi21_op_gemm_lo8(q.QI21_EPI_RESID, M, N, K, A, 3 * K // 2, da, K // 64, W, 3 * K // 2, ds, x, N,
                           gate=dev(gate), oscale=oscale)
        sync()
        want = x0 + gate * acc * oscale
        assert np.abs(x.cpu().numpy() - want).max() <= 1e-5 * np.abs(want).max()
    else:
        # W is the interleaved gate/up plane: rows 64j .. 64j + 31 gate,
        # 64j + 32 .. 64j + 63 up, of hidden columns 32j .. 32j + 31
        Nh = N // 2
        ldo = 3 * Nh // 2 + 32
        out = torch.zeros(M, ldo, device="cuda", dtype=torch.float16)
        osc = torch.zeros(M, Nh // 64, device="cuda", dtype=torch.uint8)
        inscale = 4.0
        q.qi21_op_gemm_lo8(q.QI21_EPI_SWIGLU8, M, N, K, A, 3 * K // 2, da, K // 64, W, 3 * K // 2, ds, out, ldo,
                           osc=osc, ldos=Nh // 64, oscale=oscale, inscale=inscale)
        sync()
        j = np.arange(Nh)
        g = acc[:, (j // 32) * 64 + j % 32] * inscale
        u = acc[:, (j // 32) * 64 + 32 + j % 32] * inscale
        want = g / (1.0 + np.exp(-g)) * u * oscale
        buf = out.cpu().numpy().view(np.uint8)
        assert not buf[:, 3 * Nh:].any()
        v = lo8_value(buf, Nh, osc.cpu().numpy(), 64)
        err = np.abs(v - want).max(axis=1)
        assert (err <= 2e-5 * np.abs(want).max(axis=1) + 1e-30).all(), err.max()


# ───────────────────────────── the FFN at the 1024^2 step's shape ─────────────────────────────

def test_lo8_ffn_at_1024_sampled():
    """x -> the FFN input (lo8 row op) -> gate/up + SwiGLU (lo8 GEMM, lo8
    hidden) -> down with the gated residual (lo8 GEMM) at 4096 rows, dim
    4096, hidden 12288, synthetic N(0, 0.02) weights; sampled rows against
    the oracle's f32 FFN on the same values (f16 weights)."""
    q = Q()
    M, H, I = 4096, 4096, 12288
    s = 61
    x = inputs.device_tensor(s, 1, (M, H), 1.0)
    mods = inputs.device_tensor(s, 2, (4 * H,), 0.1)
    G = inputs.device_tensor(s, 3, (I, H), 0.02).half()
    U = inputs.device_tensor(s, 4, (I, H), 0.02).half()
    D = inputs.device_tensor(s, 5, (H, I), 0.02).half()
    w13 = torch.empty(2 * I, 3 * H // 2, device="cuda", dtype=torch.float16)
    w2 = torch.empty(H, 3 * I // 2, device="cuda", dtype=torch.float16)
    s13 = torch.empty(2 * I, device="cuda", dtype=torch.uint8)
    s2 = torch.empty(H, device="cuda", dtype=torch.uint8)
    q.qi21_op_plane_lo8(q.QI21_F16, G, I, H, w13, 3 * H // 2, 32, 64, 0)
    q.qi21_op_plane_lo8(q.QI21_F16, U, I, H, w13, 3 * H // 2, 32, 64, 32)
    q.qi21_op_plane8(2 * I, H, w13, 3 * H // 2, s13)
    q.qi21_op_plane_lo8(q.QI21_F16, D, H, I, w2, 3 * I // 2, H, 0, 0)
    q.qi21_op_plane8(H, I, w2, 3 * I // 2, s2)
    del G, U, D
    xn = torch.empty(M, 3 * H // 2, device="cuda", dtype=torch.float16)
    xsc = torch.empty(M, H // 64, device="cuda", dtype=torch.uint8)
    hid = torch.empty(M, 3 * I // 2, device="cuda", dtype=torch.float16)
    hsc = torch.empty(M, I // 64, device="cuda", dtype=torch.uint8)
    eps, f_ffn, f_hid = 1e-6, 0.25, 2.0 ** -8
    q.qi21_op_rowop_lo8(M, H, 2, x, None, 1, 0, xn, 3 * H // 2, xsc, mods, 0, 2 * H, eps, f_ffn)
    q.qi21_op_gemm_lo8(q.QI21_EPI_SWIGLU8, M, 2 * I, H, xn, 3 * H // 2, xsc, H // 64, w13, 3 * H // 2, s13, hid,
                       3 * I // 2, osc=hsc, ldos=I // 64, oscale=f_hid, inscale=1.0 / f_ffn)
    x1 = x.clone()
    q.qi21_op_gemm_lo8(q.QI21_EPI_RESID, M, H, I, hid, 3 * I // 2, hsc, I // 64, w2, 3 * I // 2, s2, x1, H,
                       gate=mods[3 * H:], oscale=1.0 / f_hid)
    sync()
    rows = np.sort(np.concatenate([np.random.default_rng(5).choice(M, 14, replace=False), [0, M - 1]]))
    cols = np.sort(np.random.default_rng(6).choice(I, 64, replace=False))
    xh = np.stack([inputs.host_array(s, 1, (H,), 1.0, start=int(r) * H) for r in rows])
    mh = inputs.host_array(s, 2, (4 * H,), 0.1)
    f16w = lambda tid, shape: inputs.host_array(s, tid, shape, 0.02).astype(np.float16).astype(np.float32)  # noqa: E731
    xn_o = O.norm_mod(xh, mh[2 * H:3 * H], eps)                      # the FFN input, f32
    hid_o = O.silu(O.lin(xn_o, f16w(3, (I, H)))) * O.lin(xn_o, f16w(4, (I, H)))  # f32
    x_o = O.gated_add(xh, O.lin(hid_o, f16w(5, (H, I))), mh[3 * H:])  # the gate as the kernel took it
    # the hidden, decoded, against the oracle's on the sampled columns
    hb = hid.cpu().numpy().view(np.uint8)[rows]
    hv = lo8_value(hb, I, hsc.cpu().numpy()[rows], 64) / f_hid
    assert np.abs(hv[:, cols] - hid_o[:, cols]).max() <= 1e-4 * np.abs(hid_o).max()
    rel_h = np.linalg.norm(hv - hid_o) / np.linalg.norm(hid_o)
    # the residual stream after the FFN, per row, against the oracle
    got = x1.cpu().numpy()[rows].astype(np.float64)
    d = got - xh
    do = x_o.astype(np.float64) - xh
    rel_rows = np.linalg.norm(d - do, axis=1) / np.linalg.norm(do, axis=1)
    print(f"lo8 FFN at 1024^2: hidden rel L2 {rel_h:.2e}, branch rel L2 per row max {rel_rows.max():.2e}")
    assert rel_h < 2e-5
    assert rel_rows.max() < 5e-5
