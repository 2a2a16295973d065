"""Parity of the residual-form kernels (the QI21_FFN_LO8 and QI21_FFN_LO4
storage of the FFN sites; needs a GPU).

A residual-form value is hi = f16(v) plus the residual v - hi in a narrow
float (OCP e4m3 for lo8, e2m1 for lo4) times a power-of-two scale; rows
are grouped by 128 (lo8) or 256 (lo4) columns: the group's halves, then
its narrow values.  The checks below decode what the kernels wrote with
plain definitions of the two formats:
  e4m3: sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
        subnormal; S.1111.111 NaN; no infinities;
  e2m1: sign, 2 exponent bits with bias 1, 1 mantissa bit; exponent 0
        subnormal (0, 0.5); largest 6; two per byte, the even column in the
        low nibble;
and compare with the oracle's f32 functions on the same inputs:

* the conversions themselves: round to nearest, ties to even, in these
  encodings (a mismatch of format, bias, nibble order or rounding fails);
* the weight plane: f16 values bit-exact, the narrow copy bit-exact
  against the encoder, the scales by their rule;
* the row op writing the FFN input: the decoded value within 2^-14 (lo8)
  or 2^-12 (lo4) of each row's largest magnitude from the oracle's f32
  value, per row;
* the GEMM on random residual-form operands (every byte pattern but NaN,
  random scales), each epilogue, against an f64 sum of the decoded operands;
* the three FFN kernels chained at the 1024^2 step's shape against the
  oracle's f32 FFN on sampled rows.
"""
import numpy as np
import pytest

import inputs
from oracle import qi21_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FMTS = ["lo8", "lo4"]


def Q():
    from diffusion_transformer_denoiser_qi21_amd import qi21
    return qi21


def fmt_id(fmt):
    q = Q()
    return q.QI21_FFN_LO8 if fmt == "lo8" else q.QI21_FFN_LO4


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


def e2m1_decode(n):
    """e2m1 nibble(s) -> float64"""
    n = np.asarray(n, np.int64)
    s = np.where(n & 8, -1.0, 1.0)
    e = (n >> 1) & 3
    m = n & 1
    return s * np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * 2.0 ** (e - 1.0))


_N4 = np.arange(16)
_V4 = e2m1_decode(_N4)


def e2m1_encode(x):
    """float (|x| <= 6) -> nearest e2m1 nibble, ties to the even mantissa;
    a negative value that rounds to zero gives -0"""
    x = np.asarray(x, np.float64).ravel()
    d = np.abs(x[:, None] - _V4[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    score = cand * (2 + ((_N4[None, :] & 1) == 0) * 2 + (_N4[None, :] == 0))
    out = _N4[np.argmax(score, axis=1)]
    out = np.where(np.signbit(x) & (out == 0), 8, out)
    return out.reshape(np.shape(x))


def lo4_split(buf, ncols):
    """rows of a lo4 buffer (uint8 [rows][>= 2.5 ncols]) -> (hi f64, nibbles)"""
    rows = buf.shape[0]
    g = buf[:, :5 * ncols // 2].reshape(rows, ncols // 256, 640)
    hi = g[:, :, :512].copy().view(np.float16).reshape(rows, ncols).astype(np.float64)
    b = g[:, :, 512:].astype(np.int64)
    nib = np.stack([b & 15, b >> 4], axis=-1).reshape(rows, ncols)
    return hi, nib


def lo4_join(hi16, nib):
    rows, n = hi16.shape
    g = np.empty((rows, n // 256, 640), np.uint8)
    g[:, :, :512] = np.ascontiguousarray(hi16.astype(np.float16)).view(np.uint8).reshape(rows, n // 256, 512)
    nb = nib.reshape(rows, n // 256, 128, 2).astype(np.uint8)
    g[:, :, 512:] = nb[..., 0] | (nb[..., 1] << 4)
    return g.reshape(rows, 5 * n // 2)


def sc_index(fmt, rows, ncols):
    """flat byte position of the scale of each (row, block) in a blocked
    scale array (blocks of 64 columns for lo8 activations, of 32 for lo4,
    in their natural order): 256-row blocks, group by group, q bytes per
    row and group"""
    q, gw = (2, 128) if fmt == "lo8" else (8, 256)
    bw = 64 if fmt == "lo8" else 32
    nb = ncols // bw
    r = np.arange(rows)[:, None]
    b = np.arange(nb)[None, :]
    g, k = (b * bw) // gw, b % (gw // bw)
    pos = k if fmt == "lo8" else 4 * (k % 2) + k // 2
    per_row = ncols // bw
    return (r // 256) * 256 * per_row + g * 256 * q + (r % 256) * q + pos


def sc_rows(fmt, arr, rows, ncols):
    """a blocked scale array (any shape, flat bytes) -> [rows][blocks]"""
    return np.asarray(arr).reshape(-1)[sc_index(fmt, rows, ncols)]


def sc_alloc(fmt, rows, ncols):
    """device bytes of a blocked scale array for rows x ncols (whole blocks)"""
    bw = 64 if fmt == "lo8" else 32
    return torch.zeros((rows + 255) // 256 * 256 * (ncols // bw), device="cuda", dtype=torch.uint8)


def lo4_value(buf, ncols, per_block):
    hi, nib = lo4_split(buf, ncols)
    f = 2.0 ** (np.repeat(np.asarray(per_block, np.float64), 32, axis=1) - 127.0)
    return hi + e2m1_decode(nib) * f


def lo_value(fmt, buf, ncols, sc):
    """the value activation rows in the form represent (sc: the blocked
    scale array of those rows, which start at row 0 of a block)"""
    pb = sc_rows(fmt, sc, buf.shape[0], ncols)
    return lo8_value(buf, ncols, pb, 64) if fmt == "lo8" else lo4_value(buf, ncols, pb)


def _expected_scale4(mx):
    """the lo4 rule: the smallest e with mx 2^-e <= 6"""
    return np.ceil(np.log2(mx / 6.0)).astype(np.int64)


def _expected_scale(mx):
    """the scale rule: e with mx 2^-e in [128, 256) (mx > 0, normal)"""
    return np.floor(np.log2(mx)).astype(np.int64) - 7


# ───────────────────────────── conversions and weight planes ─────────────────────────────

def _plane(fmt, w16, group=None, gstride=0, goff=0, plane=None, rows_out=None):
    """weight rows f16 -> a residual-form plane on the device (f16 part and
    narrow part); returns (plane, scales)"""
    q = Q()
    rows, cols = w16.shape
    ld = 3 * cols // 2 if fmt == "lo8" else 5 * cols // 4
    nr = rows_out or rows
    if plane is None:
        plane = torch.zeros(nr, ld, device="cuda", dtype=torch.float16)
    q.qi21_op_plane_lo(fmt_id(fmt), q.QI21_F16, dev(w16), rows, cols, plane, ld, group or rows, gstride, goff)
    return plane, ld


def _fill(fmt, plane, nr, cols, ld):
    """the narrow part of a plane; returns the scales: lo8 [nr] (one per
    row), lo4 [nr][cols / 32] per block (from the blocked array)"""
    q = Q()
    sc = torch.zeros(nr, device="cuda", dtype=torch.uint8) if fmt == "lo8" else sc_alloc("lo4", nr, cols)
    q.qi21_op_plane_lo_fill(fmt_id(fmt), nr, cols, plane, ld, sc)
    sync()
    return sc.cpu().numpy() if fmt == "lo8" else sc_rows("lo4", sc.cpu().numpy(), nr, cols)


def test_e4m3_conversion_is_ocp_round_to_nearest_even():
    """A weight row whose largest |w| is 240 keeps scale 2^0 (240 in [128,
    256)), so its fp8 copy is the plain conversion of its values: every
    finite e4m3 value, the midpoints between neighbours (ties) and points
    a quarter of a step from them, and subnormals."""
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
    plane, ld = _plane("lo8", w)
    sc = _fill("lo8", plane, 1, n, ld)
    hi, codes = lo8_split(plane.cpu().numpy().view(np.uint8), n)
    assert int(sc[0]) == 127
    assert np.array_equal(hi[0], w[0].astype(np.float64))
    assert np.array_equal(codes[0], e4m3_encode(w[0].astype(np.float64)).astype(np.uint8))


def test_e2m1_conversion_is_round_to_nearest_even_low_nibble_first():
    """Each 32-column block of a weight row holds 6 (so its scale is 2^0:
    the largest value lands exactly on e2m1's 6) and a run of values: every
    e2m1 value, the midpoints between neighbours (ties), points a quarter
    of a step from them, and their negatives.  The fp4 copy must be the
    plain conversion, the even column in the low nibble."""
    fin = np.unique(_V4[_V4 >= 0])
    mids = (fin[:-1] + fin[1:]) / 2
    quarter = fin[:-1] + (fin[1:] - fin[:-1]) / 4
    vals = np.concatenate([fin, mids, quarter, -fin[1:], -mids, -quarter])
    per = 31  # values per block; the block's last column is 6
    nb = (len(vals) + per - 1) // per
    cols = ((nb * 32 + 255) // 256) * 256
    row = np.zeros(cols, np.float64)
    for b in range(cols // 32):
        chunk = vals[b * per:(b + 1) * per] if b < nb else np.zeros(0)
        row[b * 32:b * 32 + len(chunk)] = chunk
        row[b * 32 + 31] = 6.0
    w = row.astype(np.float16)[None, :]
    plane, ld = _plane("lo4", w)
    sc = _fill("lo4", plane, 1, cols, ld)
    hi, nib = lo4_split(plane.cpu().numpy().view(np.uint8), cols)
    assert np.array_equal(hi[0], w[0].astype(np.float64))
    assert (sc[0] == 127).all()
    assert np.array_equal(nib[0], e2m1_encode(w[0].astype(np.float64)))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols,group", [(300, 512, 300), (96, 256, 32)])
def test_plane_lo_layout_and_scales(fmt, rows, cols, group):
    """f16 values bit-exact at their grouped positions, the narrow copy
    bit-exact against the encoder at the scale its rule gives, per row
    (lo8) or per 32 columns (lo4); with group 32 the rows land interleaved
    as the gate/up plane's"""
    w = inputs.host_array(41, 1, (rows, cols), 0.02)
    w[5] *= 1e3  # one row far from the others' scale
    w[7, :64] *= 1e-3  # lo4: two blocks far below the rest of their row
    inter = group < rows
    prow = 2 * rows if inter else rows
    w16 = w.astype(np.float16)
    plane, ld = _plane(fmt, w16, group, 64 if inter else 0, 0, rows_out=prow)
    if inter:
        _plane(fmt, -w16, group, 64, 32, plane=plane)
    sc = _fill(fmt, plane, prow, cols, ld).astype(np.int64)
    buf = plane.cpu().numpy().view(np.uint8)
    hi, nar = (lo8_split if fmt == "lo8" else lo4_split)(buf, cols)
    dst = (np.arange(rows) // group) * 64 + np.arange(rows) % group if inter else np.arange(rows)
    assert np.array_equal(hi[dst], w16.astype(np.float64))
    if inter:
        assert np.array_equal(hi[dst + 32], -w16.astype(np.float64))
    for r in range(prow):
        if fmt == "lo8":
            e = _expected_scale(np.abs(hi[r]).max())
            assert sc[r] == e + 127
            assert np.array_equal(nar[r], e4m3_encode(hi[r] * 2.0 ** -e).astype(np.uint8))
        else:
            e = _expected_scale4(np.abs(hi[r]).reshape(-1, 32).max(axis=1))
            assert np.array_equal(sc[r], e + 127)
            assert np.array_equal(nar[r], e2m1_encode(hi[r] * 2.0 ** -np.repeat(e, 32)))


# ───────────────────────────── the FFN-input row op ─────────────────────────────

def _check_lo_rows(fmt, buf, xsc, h, want):
    """decoded rows against want: per row, error within 2^-14 (lo8) / 2^-12
    (lo4) of the row's largest |want|; the residual below half an f16 step
    of hi (plus the narrow rounding); each scale block's largest narrow
    value by its rule"""
    v = lo_value(fmt, buf, h, xsc)
    pb = sc_rows(fmt, xsc, buf.shape[0], h).astype(np.float64)
    assert np.isfinite(v).all()
    tol = 2.0 ** -14 if fmt == "lo8" else 2.0 ** -12
    err = np.abs(v - want).max(axis=1)
    assert (err <= tol * np.abs(want).max(axis=1)).all(), err.max()
    if fmt == "lo8":
        hi, codes = lo8_split(buf, h)
        nar = e4m3_decode(codes)
        res = nar * 2.0 ** (np.repeat(pb, 64, axis=1) - 127.0)
        blk, lo_b, hi_b, grow = 64, 128, 256, 1 + 2.0 ** -3
    else:
        hi, nib = lo4_split(buf, h)
        nar = e2m1_decode(nib)
        res = nar * 2.0 ** (np.repeat(pb, 32, axis=1) - 127.0)
        blk, lo_b, hi_b, grow = 32, 3, 6, 1.5
    ulp = np.spacing(np.abs(hi).astype(np.float16)).astype(np.float64)
    assert (np.abs(res) <= 0.5 * ulp * grow + 1e-30).all()
    bm = np.abs(nar).reshape(buf.shape[0], h // blk, blk).max(axis=2)
    nz = bm > 0
    assert ((bm[nz] >= lo_b) & (bm[nz] <= hi_b)).all()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,h,mode,nparts", [(1, 256, 2, 1), (37, 256, 3, 1), (300, 4096, 3, 3),
                                                (2049, 4096, 2, 1), (5, 8192, 3, 4), (64, 1280, 3, 1)])
def test_rowop_lo(fmt, rows, h, mode, nparts):
    """the modulated LayerNorm (after the gated residual of nparts planes
    for mode 3) written in the residual form, both row-pass forms (one wave
    per row below 2048 columns, one block per row above)"""
    q = Q()
    if fmt == "lo4" and h % 256:
        pytest.skip("lo4 rows are whole groups of 256 columns")
    x = inputs.host_array(51, 1, (rows, h), 1.0)
    y = inputs.host_array(51, 2, (nparts, rows, h), 0.5)
    mods = inputs.host_array(51, 3, (4 * h,), 0.1)
    g_off, s_off, eps, oscale = 3 * h, 2 * h, 1e-6, 0.25
    dx = dev(x)
    row_h = 3 * h // 2 if fmt == "lo8" else 5 * h // 4
    ldxn = row_h + 64  # a padded row stride
    xn = torch.zeros(rows, ldxn, device="cuda", dtype=torch.float16)
    xsc = sc_alloc(fmt, rows, h)
    q.qi21_op_rowop_lo(fmt_id(fmt), rows, h, mode, dx, dev(y), nparts, rows * h, xn, ldxn, xsc, dev(mods), g_off,
                       s_off, eps, oscale)
    sync()
    xe = x
    if mode & 1:
        xe = O.gated_add(x, y.sum(axis=0, dtype=np.float32), mods[g_off:g_off + h])
        assert np.abs(dx.cpu().numpy() - xe).max() <= 1e-5 * np.abs(xe).max()
    want = O.norm_mod(xe, mods[s_off:s_off + h], eps, dt=np.float64) * oscale
    buf = xn.cpu().numpy().view(np.uint8)
    assert not buf[:, 2 * row_h:].any()  # the padding is not written
    _check_lo_rows(fmt, buf, xsc.cpu().numpy(), h, want)


# ───────────────────────────── the residual-form GEMM ─────────────────────────────

def _random_rows(fmt, rng, rows, cols, hi_sigma, act, sc_lo, sc_hi):
    """random residual-form rows: f16 values, any non-NaN narrow value,
    random scales; returns (buffer bytes, the scale array as the kernels
    take it, hi f64, narrow-times-scale f64).  Scale arrays: blocked (lo8
    activations, lo4), or one byte per row (lo8 weights)."""
    hi = (rng.standard_normal((rows, cols)) * hi_sigma).astype(np.float16)
    if fmt == "lo8" and not act:
        codes = rng.integers(0, 256, (rows, cols)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x11
        sc = rng.integers(sc_lo, sc_hi + 1, rows).astype(np.uint8)
        f = np.repeat(sc[:, None].astype(np.float64), cols, axis=1) - 127.0
        return lo8_join(hi, codes), sc, hi.astype(np.float64), e4m3_decode(codes) * 2.0 ** f
    bw = 64 if fmt == "lo8" else 32
    blocks = rng.integers(sc_lo, sc_hi + 1, (rows, cols // bw))
    arr = np.zeros((rows + 255) // 256 * 256 * (cols // bw), np.uint8)
    arr[sc_index(fmt, rows, cols)] = blocks
    f = np.repeat(blocks.astype(np.float64), bw, axis=1) - 127.0
    if fmt == "lo8":
        codes = rng.integers(0, 256, (rows, cols)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x11
        return lo8_join(hi, codes), arr, hi.astype(np.float64), e4m3_decode(codes) * 2.0 ** f
    nib = rng.integers(0, 16, (rows, cols))
    return lo4_join(hi, nib), arr, hi.astype(np.float64), e2m1_decode(nib) * 2.0 ** f


@pytest.mark.parametrize("even", [False, True])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 77, 300, 1040])
@pytest.mark.parametrize("epi", ["f32", "resid", "split", "swiglu"])
def test_gemm_lo_epilogues(fmt, epi, M, even):
    """even: an even number of column groups per work unit, which lo4 runs
    on the 16 x 16 x 32 kernel; odd counts take the 32 x 32 x 16 one."""
    q = Q()
    rng = np.random.default_rng(1000 + M + (7 if fmt == "lo4" else 0) + (3 if even else 0))
    g = 128 if fmt == "lo8" else 256
    ng, ks = ((2 if even else 3), 1) if epi == "swiglu" else ((4, 2) if even else (3, 3)) if epi == "split" else \
        ((4 if even else 3), 1)
    N, K = (512 if fmt == "lo8" else 1024, ng * g) if epi == "swiglu" else (256, ng * g)
    kr = 3 * K // 2 if fmt == "lo8" else 5 * K // 4  # halves per row
    abuf, asc, a_h, a_l = _random_rows(fmt, rng, M, K, 1.0, True, 108, 116)
    wbuf, wsc, w_h, w_l = _random_rows(fmt, rng, N, K, 0.05, False, 110, 116)
    A, W = dev(abuf), dev(wbuf)
    da, dw = dev(asc), dev(wsc)
    acc = a_h @ w_h.T + a_l @ w_l.T
    oscale = 0.5
    f = fmt_id(fmt)
    if epi in ("f32", "split"):
        out = torch.full((ks, M, N), float("nan"), device="cuda")
        q.qi21_op_gemm_lo(f, q.QI21_EPI_F32, M, N, K, A, kr, da, W, kr, dw, out, N, ksplit=ks, oscale=oscale)
        sync()
        o = out.cpu().numpy().astype(np.float64)
        for p in range(ks):  # each plane its own share of the columns
            c = slice(p * K // ks, (p + 1) * K // ks)
            want_p = (a_h[:, c] @ w_h[:, c].T + a_l[:, c] @ w_l[:, c].T) * oscale
            assert np.abs(o[p] - want_p).max() <= 1e-5 * np.abs(want_p).max()
        assert np.abs(o.sum(axis=0) - acc * oscale).max() <= 1e-5 * np.abs(acc * oscale).max()
    elif epi == "resid":
        x0 = rng.standard_normal((M, N)).astype(np.float32)
        gate = rng.standard_normal(N).astype(np.float32) * 0.1
        x = dev(x0)
        q.qi21_op_gemm_lo(f, q.QI21_EPI_RESID, M, N, K, A, kr, da, W, kr, dw, x, N, gate=dev(gate), oscale=oscale)
        sync()
        want = x0 + gate * acc * oscale
        assert np.abs(x.cpu().numpy() - want).max() <= 1e-5 * np.abs(want).max()
    else:
        # W is the interleaved gate/up plane: rows 64j .. 64j + 31 gate,
        # 64j + 32 .. 64j + 63 up, of hidden columns 32j .. 32j + 31
        Nh = N // 2
        hrow = 3 * Nh // 2 if fmt == "lo8" else 5 * Nh // 4
        ldo = hrow + 32
        out = torch.zeros(M, ldo, device="cuda", dtype=torch.float16)
        osc = sc_alloc(fmt, M, Nh)
        inscale = 4.0
        epi_sw = q.QI21_EPI_SWIGLU8 if fmt == "lo8" else q.QI21_EPI_SWIGLU4
        q.qi21_op_gemm_lo(f, epi_sw, M, N, K, A, kr, da, W, kr, dw, out, ldo, osc=osc, oscale=oscale,
                          inscale=inscale)
        sync()
        j = np.arange(Nh)
        gg = acc[:, (j // 32) * 64 + j % 32] * inscale
        uu = acc[:, (j // 32) * 64 + 32 + j % 32] * inscale
        want = gg / (1.0 + np.exp(-gg)) * uu * oscale
        buf = out.cpu().numpy().view(np.uint8)
        assert not buf[:, 2 * hrow:].any()
        _check_lo_rows(fmt, buf, osc.cpu().numpy(), Nh, want)


# ───────────────────────────── the FFN at the 1024^2 step's shape ─────────────────────────────

@pytest.mark.parametrize("fmt", FMTS)
def test_lo_ffn_at_1024_sampled(fmt):
    """x -> the FFN input (row op) -> gate/up + SwiGLU (hidden in the form)
    -> down with the gated residual, at 4096 rows, dim 4096, hidden 12288,
    synthetic N(0, 0.02) weights; sampled rows against the oracle's f32 FFN
    on the same values (f16 weights)."""
    q = Q()
    f = fmt_id(fmt)
    M, H, I = 4096, 4096, 12288
    s = 61
    x = inputs.device_tensor(s, 1, (M, H), 1.0)
    mods = inputs.device_tensor(s, 2, (4 * H,), 0.1)
    G = inputs.device_tensor(s, 3, (I, H), 0.02).half()
    U = inputs.device_tensor(s, 4, (I, H), 0.02).half()
    D = inputs.device_tensor(s, 5, (H, I), 0.02).half()
    rx = 3 * H // 2 if fmt == "lo8" else 5 * H // 4   # halves per row of dim H
    ri = 3 * I // 2 if fmt == "lo8" else 5 * I // 4   # and of dim I
    w13 = torch.empty(2 * I, rx, device="cuda", dtype=torch.float16)
    w2 = torch.empty(H, ri, device="cuda", dtype=torch.float16)
    s13 = torch.empty(2 * I, device="cuda", dtype=torch.uint8) if fmt == "lo8" else sc_alloc("lo4", 2 * I, H)
    s2 = torch.empty(H, device="cuda", dtype=torch.uint8) if fmt == "lo8" else sc_alloc("lo4", H, I)
    q.qi21_op_plane_lo(f, q.QI21_F16, G, I, H, w13, rx, 32, 64, 0)
    q.qi21_op_plane_lo(f, q.QI21_F16, U, I, H, w13, rx, 32, 64, 32)
    q.qi21_op_plane_lo_fill(f, 2 * I, H, w13, rx, s13)
    q.qi21_op_plane_lo(f, q.QI21_F16, D, H, I, w2, ri, H, 0, 0)
    q.qi21_op_plane_lo_fill(f, H, I, w2, ri, s2)
    del G, U, D
    xn = torch.empty(M, rx, device="cuda", dtype=torch.float16)
    xsc = sc_alloc(fmt, M, H)
    hid = torch.empty(M, ri, device="cuda", dtype=torch.float16)
    hsc = sc_alloc(fmt, M, I)
    eps, f_ffn, f_hid = 1e-6, 0.25, 2.0 ** -8
    q.qi21_op_rowop_lo(f, M, H, 2, x, None, 1, 0, xn, rx, xsc, mods, 0, 2 * H, eps, f_ffn)
    epi_sw = q.QI21_EPI_SWIGLU8 if fmt == "lo8" else q.QI21_EPI_SWIGLU4
    q.qi21_op_gemm_lo(f, epi_sw, M, 2 * I, H, xn, rx, xsc, w13, rx, s13, hid, ri, osc=hsc, oscale=f_hid,
                      inscale=1.0 / f_ffn)
    x1 = x.clone()
    q.qi21_op_gemm_lo(f, q.QI21_EPI_RESID, M, H, I, hid, ri, hsc, w2, ri, s2, x1, H, gate=mods[3 * H:],
                      oscale=1.0 / f_hid)
    sync()
    rows = np.sort(np.concatenate([np.random.default_rng(5).choice(M, 14, replace=False), [0, M - 1]]))
    cols = np.sort(np.random.default_rng(6).choice(I, 64, replace=False))
    xh = np.stack([inputs.host_array(s, 1, (H,), 1.0, start=int(r) * H) for r in rows])
    mh = inputs.host_array(s, 2, (4 * H,), 0.1)
    f16w = lambda tid, shape: inputs.host_array(s, tid, shape, 0.02).astype(np.float16).astype(np.float32)  # noqa: E731
    xn_o = O.norm_mod(xh, mh[2 * H:3 * H], eps)                      # the FFN input, f32
    hid_o = O.silu(O.lin(xn_o, f16w(3, (I, H)))) * O.lin(xn_o, f16w(4, (I, H)))  # f32
    x_o = O.gated_add(xh, O.lin(hid_o, f16w(5, (H, I))), mh[3 * H:])  # the gate as the kernel took it
    hb = hid.cpu().numpy().view(np.uint8)
    hv = lo_value(fmt, hb, I, hsc.cpu().numpy())[rows] / f_hid
    tol_h, tol_b = (2e-5, 5e-5) if fmt == "lo8" else (1e-4, 2e-4)
    assert np.abs(hv[:, cols] - hid_o[:, cols]).max() <= 5 * tol_h * np.abs(hid_o).max()
    rel_h = np.linalg.norm(hv - hid_o) / np.linalg.norm(hid_o)
    got = x1.cpu().numpy()[rows].astype(np.float64)
    d, do = got - xh, x_o.astype(np.float64) - xh
    rel_rows = np.linalg.norm(d - do, axis=1) / np.linalg.norm(do, axis=1)
    print(f"{fmt} FFN at 1024^2: hidden rel L2 {rel_h:.2e}, branch rel L2 per row max {rel_rows.max():.2e}")
    assert rel_h < tol_h
    assert rel_rows.max() < tol_b
