"""Per-kernel parity of the HIP library against the CPU oracle (needs a GPU).

Every kernel is called through the C ABI (``qi21_op_*``) on seeded inputs
and compared element by element with the oracle's function on the same
values: f32 outputs to 1e-5 relative L2, f16 outputs (one rounding to
binary16) to 2e-3.  Besides the whole tensor's relative L2, every row's
own relative L2 must stay within ROW_FACTOR times the same bound, so that
an error confined to a tail tile, a mask edge or one row cannot hide in
the global figure.  Sizes span several tiles with a ragged tail.
"""
import math

import numpy as np
import pytest

import inputs
from oracle import qi21_oracle as O
from parity import ROW_FACTOR, assert_close, rel, rowrel  # noqa: F401

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F16_TOL = 2e-3
F32_TOL = 1e-5


def Q():
    from diffusion_transformer_denoiser_qi21_amd import qi21
    return qi21


def f16_host(seed, tid, shape, sigma):
    """seeded values rounded to f16, as float32 numpy (exactly what the GPU sees)"""
    return inputs.host_array(seed, tid, shape, sigma).astype(np.float16).astype(np.float32)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def sync():
    torch.cuda.synchronize()


def vt_pos(j):
    """column of key j in a V^T row: bits 2 and 3 of j swapped (the layout
    the QKV epilogue writes and the attention kernel reads)"""
    j = np.asarray(j)
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1)


# ───────────────────────────── GEMM ─────────────────────────────

@pytest.mark.parametrize("tile", [-1, 0, 1, 2])
@pytest.mark.parametrize("M", [1, 77, 300, 1040])
@pytest.mark.parametrize("epi", ["f16", "f32", "swiglu", "qkv"])
def test_gemm_epilogues(epi, M, tile):
    q = Q()
    N, K = 768, 512
    A = f16_host(1, 1, (M, K), 1.0)
    W = f16_host(1, 2, (N, K), 0.05)
    oscale, inscale = 0.25, 4.0
    dA, dW = dev(A, torch.float16), dev(W, torch.float16)
    if epi in ("f16", "f32"):
        out = torch.zeros(M, N, device="cuda", dtype=torch.float16 if epi == "f16" else torch.float32)
        q.qi21_op_gemm(q.QI21_EPI_F16 if epi == "f16" else q.QI21_EPI_F32, M, N, K, dA, K, dW, out, N,
                       oscale=oscale, tile=tile)
        sync()
        want = O.lin(A, W) * np.float32(oscale)
        assert_close(out.float().cpu().numpy(), want, (F16_TOL if epi == "f16" else F32_TOL))
    elif epi == "swiglu":
        G, U = W[: N // 2], W[N // 2:]
        w13 = torch.empty(N, K, device="cuda", dtype=torch.float16)
        q.qi21_op_plane(q.QI21_F32, dev(G), N // 2, K, w13, 32, 64, 0)
        q.qi21_op_plane(q.QI21_F32, dev(U), N // 2, K, w13, 32, 64, 32)
        out = torch.zeros(M, N // 2, device="cuda", dtype=torch.float16)
        q.qi21_op_gemm(q.QI21_EPI_SWIGLU, M, N, K, dA, K, w13, out, N // 2, oscale=oscale, inscale=inscale, tile=tile)
        sync()
        g = O.lin(A, G) * np.float32(inscale)
        u = O.lin(A, U) * np.float32(inscale)
        want = O.silu(g) * u * np.float32(oscale)
        assert_close(out.float().cpu().numpy(), want, F16_TOL)
    else:
        h = N // 3
        ld2 = ((M + 63) // 64) * 64
        out = torch.zeros(M, 2 * h, device="cuda", dtype=torch.float16)
        vt = torch.zeros(h, ld2, device="cuda", dtype=torch.float16)
        q.qi21_op_gemm(q.QI21_EPI_QKV, M, N, K, dA, K, dW, out, 2 * h, vt, ld2, oscale=oscale, tile=tile)
        sync()
        want = O.lin(A, W) * np.float32(oscale)
        assert_close(out.float().cpu().numpy(), want[:, :2 * h], F16_TOL)
        vtn = vt.float().cpu().numpy()
        cols = vt_pos(np.arange(M))
        assert_close(vtn[:, cols], want[:, 2 * h:].T, F16_TOL)
        rest = np.setdiff1d(np.arange(ld2), cols)
        assert np.all(vtn[:, rest] == 0)  # nothing written for rows past M


@pytest.mark.parametrize("M,ld2", [(300, 308), (77, 84), (256, 260), (1040, 1044)])
def test_qkv_vt_leading_dimension_tail(M, ld2):
    """The qkv split's V^T with a leading dimension that is not a whole
    number of 16-key groups, on the 256 x 256 tile (tile 0): keys below M
    hold v, keys from M up to the last whole group of 16 below ld2 hold
    zeros, and the columns past that group are not written."""
    q = Q()
    N, K = 768, 512
    h = N // 3
    A = f16_host(3, 1, (M, K), 1.0)
    W = f16_host(3, 2, (N, K), 0.05)
    out = torch.zeros(M, 2 * h, device="cuda", dtype=torch.float16)
    vt = torch.full((h, ld2), 7.0, device="cuda", dtype=torch.float16)
    q.qi21_op_gemm(q.QI21_EPI_QKV, M, N, K, dev(A, torch.float16), K, dev(W, torch.float16), out, 2 * h, vt, ld2,
                   oscale=0.5, tile=0)
    sync()
    want = O.lin(A, W) * np.float32(0.5)
    assert_close(out.float().cpu().numpy(), want[:, :2 * h], F16_TOL)
    vtn = vt.float().cpu().numpy()
    assert_close(vtn[:, vt_pos(np.arange(M))], want[:, 2 * h:].T, F16_TOL)
    rz = ld2 & ~15
    pad = np.setdiff1d(np.arange(rz), vt_pos(np.arange(M)))
    assert np.all(vtn[:, pad] == 0)
    assert np.all(vtn[:, rz:] == 7.0)


def _pair(a32):
    """an f32 array as the f16 pair (hi, lo) = (f16(a), f16(a - hi))"""
    hi = a32.astype(np.float16)
    lo = (a32 - hi.astype(np.float32)).astype(np.float16)
    return hi, lo


def _check_pair(hi, lo):
    """lo is at most half an f16 step of hi: hi is the f16 rounding of hi + lo"""
    hi = np.asarray(hi, np.float16)
    half_step = np.spacing(np.abs(hi)).astype(np.float32) / 2
    assert np.all(np.abs(np.asarray(lo, np.float32)) <= half_step)


PAIR_TOL = 1e-5  # f32 accumulation; the pair carries ~22 significant bits


@pytest.mark.parametrize("tile", [-1, 0, 1, 2])
@pytest.mark.parametrize("M", [1, 77, 300, 1600])
@pytest.mark.parametrize("epi", ["f32", "swiglu", "swiglu2"])
def test_gemm_pair_operand(epi, M, tile):
    """(A_hi + A_lo) W^T with each W row read for both halves (the QI21_FFN_PAIR
    GEMMs): within f32 accumulation of the float operand's exact product,
    where a single f16 operand is ~1e-4 away."""
    q = Q()
    N, K = 768, 512
    A = inputs.host_array(2, 1, (M, K), 1.0)
    W = f16_host(2, 2, (N, K), 0.05)
    hi, lo = _pair(A)
    dA = dev(np.concatenate([hi, lo], axis=1))
    dW = dev(W, torch.float16)
    oscale, inscale = 0.25, 4.0
    A64, W64 = A.astype(np.float64), W.astype(np.float64)
    if epi == "f32":
        out = torch.zeros(M, N, device="cuda", dtype=torch.float32)
        q.qi21_op_gemm_pair(q.QI21_EPI_F32, M, N, K, dA, 2 * K, dW, out, N, oscale=oscale, tile=tile)
        sync()
        want = A64 @ W64.T * oscale
        assert_close(out.cpu().numpy(), want, PAIR_TOL)
        single = O.lin(hi.astype(np.float32), W) * np.float32(oscale)
        assert rel(single, want) > 10 * PAIR_TOL  # the lo half matters at this tolerance
        return
    G, U = W[: N // 2], W[N // 2:]
    w13 = torch.empty(N, K, device="cuda", dtype=torch.float16)
    q.qi21_op_plane(q.QI21_F32, dev(G), N // 2, K, w13, 32, 64, 0)
    q.qi21_op_plane(q.QI21_F32, dev(U), N // 2, K, w13, 32, 64, 32)
    g = A64 @ G.astype(np.float64).T * inscale
    u = A64 @ U.astype(np.float64).T * inscale
    want = g / (1 + np.exp(-g)) * u * oscale
    if epi == "swiglu":
        out = torch.zeros(M, N // 2, device="cuda", dtype=torch.float16)
        q.qi21_op_gemm_pair(q.QI21_EPI_SWIGLU, M, N, K, dA, 2 * K, w13, out, N // 2, oscale=oscale, inscale=inscale,
                            tile=tile)
        sync()
        assert_close(out.float().cpu().numpy(), want, F16_TOL)
    else:
        out = torch.zeros(M, N, device="cuda", dtype=torch.float16)
        q.qi21_op_gemm_pair(q.QI21_EPI_SWIGLU2, M, N, K, dA, 2 * K, w13, out, N, oscale=oscale, inscale=inscale,
                            tile=tile)
        sync()
        o = out.cpu().numpy()
        ohi, olo = o[:, : N // 2], o[:, N // 2:]
        _check_pair(ohi, olo)
        assert_close(ohi.astype(np.float64) + olo.astype(np.float64), want, PAIR_TOL)


@pytest.mark.parametrize("M", [77, 1600])
def test_gemm_swiglu_pair_output(M):
    """SWIGLU2 on a single f16 operand: the hidden as an f16 pair equals the
    f32 epilogue value, hi being its f16 rounding."""
    q = Q()
    N, K = 512, 256
    A = f16_host(4, 1, (M, K), 1.0)
    W = f16_host(4, 2, (N, K), 0.05)
    G, U = W[: N // 2], W[N // 2:]
    w13 = torch.empty(N, K, device="cuda", dtype=torch.float16)
    q.qi21_op_plane(q.QI21_F32, dev(G), N // 2, K, w13, 32, 64, 0)
    q.qi21_op_plane(q.QI21_F32, dev(U), N // 2, K, w13, 32, 64, 32)
    out = torch.zeros(M, N, device="cuda", dtype=torch.float16)
    q.qi21_op_gemm(q.QI21_EPI_SWIGLU2, M, N, K, dev(A, torch.float16), K, w13, out, N)
    sync()
    g = A.astype(np.float64) @ G.astype(np.float64).T
    u = A.astype(np.float64) @ U.astype(np.float64).T
    want = g / (1 + np.exp(-g)) * u
    o = out.cpu().numpy()
    _check_pair(o[:, : N // 2], o[:, N // 2:])
    assert_close(o[:, : N // 2].astype(np.float64) + o[:, N // 2:], want, PAIR_TOL)


def test_gemm_plane_conversion_exact():
    q = Q()
    rows, cols = 96, 128
    src = inputs.host_array(3, 4, (rows, cols), 0.02, bf16=True)
    bf = dev(src).to(torch.bfloat16)
    dst = torch.zeros(2 * rows, cols, device="cuda", dtype=torch.float16)
    q.qi21_op_plane(q.QI21_BF16, bf, rows, cols, dst, 32, 64, 32)
    sync()
    d = dst.cpu()
    for r in range(rows):
        assert torch.equal(d[(r // 32) * 64 + 32 + r % 32], bf[r].cpu().half())
    assert torch.all(d.view(-1, 64, cols)[:, :32] == 0)


# ───────────────────────────── flash attention ─────────────────────────────

QL2 = np.log2(np.e) / np.sqrt(128.0)  # the attention kernels take q * QL2


def _vt(v, ld):
    """V [n][H] -> V^T [H][ld] in the attention kernel's key order, zero padding"""
    out = np.zeros((v.shape[1], ld), np.float32)
    out[:, vt_pos(np.arange(v.shape[0]))] = v.T
    return out


@pytest.mark.parametrize("case", ["step", "step_tiny", "step_tiles", "prefill_cond", "prefill_text", "one_key"])
def test_flash_parity(case):
    q = Q()
    heads, hd = 2, 128
    H = heads * hd
    vis = None
    if case == "step":
        nq, n1, n2 = 300, 18, 300
    elif case == "step_tiny":
        nq, n1, n2 = 1, 1, 1
    elif case == "step_tiles":
        nq, n1, n2 = 257, 130, 257
    elif case == "one_key":
        nq, n1, n2 = 70, 1, 0
    else:
        segs = [("text", 22), ("image", 12, 12), ("image", 4, 4)] if case == "prefill_cond" else \
            [("text", 150), ("image", 2, 2)]
        lay = O.Layout(segs)
        vis = O.prefix_visibility(lay)
        nq, n1, n2 = lay.prefix_len, lay.prefix_len, 0
    m = n1 + n2
    # q in the kernel's base-2 units (f16 of q log2(e) / sqrt(128)); the
    # oracle gets the q that stands for
    qa = f16_host(5, 1, (nq, H), 1.0)
    ql = (qa * np.float32(QL2)).astype(np.float16)
    qa = ql.astype(np.float64) / QL2
    k = f16_host(5, 2, (m, H), 1.0)
    v = f16_host(5, 3, (m, H), 1.0)
    oscale = 2.0
    ld1 = ((max(n1, 1) + 63) // 64) * 64
    ld2 = ((max(n2, 1) + 63) // 64) * 64 + 64
    k2panel = np.zeros((max(n2, 1), 2 * H), np.float32)  # k at column H of a wider panel
    k2panel[:n2, H:] = k[n1:]
    dq = dev(ql)
    dk1 = dev(k[:n1] if n1 else np.zeros((1, H), np.float32), torch.float16)
    dvt1 = dev(_vt(v[:n1], ld1), torch.float16)
    dk2 = dev(k2panel, torch.float16)
    dvt2 = dev(_vt(v[n1:], ld2), torch.float16)
    dvis = dev(vis.astype(np.int32)) if vis is not None else None
    out = torch.zeros(nq, H, device="cuda", dtype=torch.float16)
    q.qi21_op_flash(nq, heads, dq, H, dk1, H, dvt1, ld1, n1,
                    dk2.data_ptr() + H * 2 if n2 else None, 2 * H, dvt2 if n2 else None, ld2, n2,
                    dvis, out, H, oscale)
    sync()
    visible = vis if vis is not None else np.full(nq, m, np.int64)
    want = O.attention(qa, k, v, visible, heads, hd) * np.float32(oscale)
    assert_close(out.float().cpu().numpy(), want, F16_TOL)


# 32 heads; on 256 CUs 96 queries run as key-split blocks, 2048 as 4-wave
# blocks and 4096 as 8-wave blocks
@pytest.mark.parametrize("nq", [96, 2048, 4096])
@pytest.mark.parametrize("order", ["growing", "shrinking", "masked_start"])
def test_flash_lazy_rescale_paths(order, nq):
    """Key scales that make a query's maximum grow by far more than the lazy
    rescale threshold from tile to tile (a rescale at every tile), shrink
    (later tiles underflow against the first), or a block-causal start where
    the first visible keys are few: the running-maximum bookkeeping of the
    base-2 scores against the oracle's softmax, in each launch form."""
    q = Q()
    heads, hd = 32, 128
    H = heads * hd
    n1 = 333
    qa = f16_host(6, 1, (nq, H), 1.0)
    ql = (qa * np.float32(QL2)).astype(np.float16)
    qe = ql.astype(np.float64) / QL2
    k = inputs.host_array(6, 2, (n1, H), 1.0)
    j = np.arange(n1, dtype=np.float64)[:, None]
    if order == "growing":
        k = k * (0.05 + j / 12.0)        # maxima grow by ~2^10 per tile
    elif order == "shrinking":
        k = k * (30.0 / (1.0 + j / 8.0))  # the first tile dominates
    k = k.astype(np.float16).astype(np.float32)
    v = f16_host(6, 3, (n1, H), 1.0)
    vis = None
    if order == "masked_start":
        vis = np.minimum(1 + np.arange(nq) * 4, n1).astype(np.int64)  # 1, 5, 9, ... keys
    ld1 = ((n1 + 63) // 64) * 64
    out = torch.zeros(nq, H, device="cuda", dtype=torch.float16)
    dvis = dev(vis.astype(np.int32)) if vis is not None else None
    q.qi21_op_flash(nq, heads, dev(ql), H, dev(k, torch.float16), H, dev(_vt(v, ld1), torch.float16), ld1, n1,
                    None, 0, None, 0, 0, dvis, out, H, 1.0)
    sync()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    visible = vis if vis is not None else np.full(nq, n1, np.int64)
    want = O.attention(qe, k, v, visible, heads, hd)
    assert_close(got, want, F16_TOL)


# ───────────────────────────── row kernels ─────────────────────────────

@pytest.mark.parametrize("h", [256, 4096])
@pytest.mark.parametrize("rows", [1, 300])
@pytest.mark.parametrize("mode", [6, 7])
def test_rowop_pair_output(mode, rows, h):
    """mode bit 2: the modulated LayerNorm written as an f16 pair [rows][2h]
    whose sum is the f32 value (the QI21_FFN_PAIR FFN input)"""
    q = Q()
    x = inputs.host_array(8, 1, (rows, h), 1.0)
    y = inputs.host_array(8, 2, (rows, h), 0.5)
    mods = inputs.host_array(8, 3, (4 * h,), 0.1)
    g_off, s_off, eps, oscale = 3 * h, 2 * h, 1e-6, 0.25
    dx, dy, dm = dev(x), dev(y), dev(mods)
    xn = torch.zeros(rows, 2 * h, device="cuda", dtype=torch.float16)
    q.qi21_op_rowop(rows, h, mode, dx, dy, xn, xn.shape[1], dm, g_off, s_off, eps, oscale)
    sync()
    xe = O.gated_add(x, y, mods[g_off:g_off + h]) if mode & 1 else x
    assert_close(dx.cpu().numpy(), xe, 1e-6)
    want = O.norm_mod(xe, mods[s_off:s_off + h], eps, dt=np.float64) * oscale
    o = xn.cpu().numpy()
    _check_pair(o[:, :h], o[:, h:])
    assert_close(o[:, :h].astype(np.float64) + o[:, h:], want, 2e-6)



@pytest.mark.parametrize("h", [256, 4096])
@pytest.mark.parametrize("rows", [1, 37, 300])
@pytest.mark.parametrize("mode", [1, 2, 3])
def test_rowop_modes(mode, rows, h):
    q = Q()
    x = inputs.host_array(7, 1, (rows, h), 1.0)
    y = inputs.host_array(7, 2, (rows, h), 0.5)
    mods = inputs.host_array(7, 3, (4 * h,), 0.1)
    g_off, s_off, eps, oscale = 3 * h, 2 * h, 1e-6, 0.25
    dx, dy, dm = dev(x), dev(y), dev(mods)
    xn = torch.zeros(rows, h, device="cuda", dtype=torch.float16)
    q.qi21_op_rowop(rows, h, mode, dx, dy, xn, xn.shape[1], dm, g_off, s_off, eps, oscale)
    sync()
    xe = O.gated_add(x, y, mods[g_off:g_off + h]) if mode & 1 else x
    assert_close(dx.cpu().numpy(), xe, 1e-6)
    if mode & 2:
        want = O.norm_mod(xe, mods[s_off:s_off + h], eps) * np.float32(oscale)
        assert_close(xn.float().cpu().numpy(), want, F16_TOL)
    else:
        assert torch.all(xn == 0)


@pytest.mark.parametrize("n", [1, 5, 4118])
def test_rope_pack_layout(n):
    """The packed RoPE table holds, per row and pair couple m, cos 2m, cos
    2m+1, sin 2m, sin 2m+1: bit-exact copies of the separate tables."""
    q = Q()
    c = inputs.host_array(17, 1, (n, 64), 1.0)
    s = inputs.host_array(17, 2, (n, 64), 1.0)
    out = torch.full((n, 128), float("nan"), device="cuda")
    q.qi21_op_rope_pack(n, dev(c), dev(s), out)
    sync()
    o = out.cpu().numpy().reshape(n, 32, 4)
    assert np.array_equal(o[:, :, 0], c[:, 0::2]) and np.array_equal(o[:, :, 1], c[:, 1::2])
    assert np.array_equal(o[:, :, 2], s[:, 0::2]) and np.array_equal(o[:, :, 3], s[:, 1::2])


@pytest.mark.parametrize("rows,h,mode", [(2048, 4096, 3), (2049, 4096, 3), (2049, 4096, 2), (5, 8192, 3),
                                         (5, 2052, 7), (3000, 2048, 1), (64, 2044, 3)])
def test_rowop_row_forms(rows, h, mode):
    """Both row-pass forms and the choice between them: one block per row for
    wide rows, one wave per row for narrower rows and for long passes with a
    residual (more than 2048 rows); widths that are not a multiple of the
    block's 1024-float stride leave threads with partial chunk sets."""
    q = Q()
    x = inputs.host_array(16, 1, (rows, h), 1.0)
    y = inputs.host_array(16, 2, (rows, h), 0.5)
    mods = inputs.host_array(16, 3, (4 * h,), 0.1)
    g_off, s_off, eps, oscale = 3 * h, 2 * h, 1e-6, 0.25
    dx, dy, dm = dev(x), dev(y), dev(mods)
    xn = torch.zeros(rows, 2 * h if mode & 4 else h, device="cuda", dtype=torch.float16)
    q.qi21_op_rowop(rows, h, mode, dx, dy, xn, xn.shape[1], dm, g_off, s_off, eps, oscale)
    sync()
    xe = O.gated_add(x, y, mods[g_off:g_off + h]) if mode & 1 else x
    assert_close(dx.cpu().numpy(), xe, 1e-6)
    if mode & 2:
        want = O.norm_mod(xe, mods[s_off:s_off + h], eps, dt=np.float64) * oscale
        o = xn.float().cpu().numpy()
        if mode & 4:
            _check_pair(xn[:, :h].cpu().numpy(), xn[:, h:].cpu().numpy())
            assert_close(o[:, :h].astype(np.float64) + o[:, h:], want, 2e-6)
        else:
            assert_close(o, want, F16_TOL)
    else:
        assert torch.all(xn == 0)


@pytest.mark.parametrize("kdst", [False, True])
@pytest.mark.parametrize("rows", [5, 300])
def test_qkrope(rows, kdst):
    q = Q()
    heads, hd = 2, 128
    H = heads * hd
    ldp = 2 * H + 64
    lay = O.Layout([("text", 7), ("image", 17, 18)])
    pos = lay.positions()[:rows]
    c, s = O.rope_tables(pos)
    panel = f16_host(9, 1, (rows, ldp), 1.0 / 16)  # stored values carry 2^-4
    wq = inputs.host_array(9, 2, (hd,), 0.02, mean=1.0)
    wk = inputs.host_array(9, 3, (hd,), 0.02, mean=1.0)
    eps = 1e-6 * 2.0 ** -8
    dp = dev(panel, torch.float16)
    kd = torch.zeros(rows, H, device="cuda", dtype=torch.float16) if kdst else None
    q.qi21_op_qkrope(rows, heads, dp, ldp, dev(wq), dev(wk), dev(c), dev(s), eps, kd, H)
    sync()
    got = dp.float().cpu().numpy()
    wq_ = O.qk_norm_rope(panel[:, :H], wq, c, s, heads, hd, eps)
    wk_ = O.qk_norm_rope(panel[:, H:2 * H], wk, c, s, heads, hd, eps)
    assert_close(got[:, :H], wq_, F16_TOL)
    if kdst:
        assert_close(kd.float().cpu().numpy(), wk_, F16_TOL)
        assert np.array_equal(got[:, H:], panel[:, H:])  # k untouched in the panel
    else:
        assert_close(got[:, H:2 * H], wk_, F16_TOL)
        assert np.array_equal(got[:, 2 * H:], panel[:, 2 * H:])


@pytest.mark.parametrize("pair", [False, True])
@pytest.mark.parametrize("tile", [-1, 0, 1, 2])
@pytest.mark.parametrize("M", [1, 77, 1600])
def test_gemm_gated_residual(M, tile, pair):
    """x += gate * (A W^T) * oscale in the GEMM epilogue ([QI] gated_add)"""
    q = Q()
    N, K = 768, 512
    x = inputs.host_array(12, 1, (M, N), 1.0)
    gate = np.tanh(inputs.host_array(12, 2, (N,), 0.1)).astype(np.float32)
    W = f16_host(12, 3, (N, K), 0.05)
    if pair:
        A32 = inputs.host_array(12, 4, (M, K), 1.0)
        hi, lo = _pair(A32)
        A = np.concatenate([hi, lo], axis=1)
        prod = A32.astype(np.float64) @ W.astype(np.float64).T
    else:
        A = f16_host(12, 4, (M, K), 1.0)
        prod = A.astype(np.float64) @ W.astype(np.float64).T
    dx = dev(x)
    q.qi21_op_gemm_resid(M, N, A.shape[1], K, dev(A, torch.float16), A.shape[1], dev(W, torch.float16), dx, N,
                         dev(gate), 0.5, tile)
    sync()
    want = x.astype(np.float64) + gate.astype(np.float64) * prod * 0.5
    assert_close(dx.cpu().numpy(), want, (PAIR_TOL if pair else F32_TOL * 10))


@pytest.mark.parametrize("tile", [0, 1, 2])
@pytest.mark.parametrize("K", [64, 128, 192, 320, 4160])
def test_gemm_k_depths(K, tile):
    """Depths of one, two, an odd number and many 64-wide k-tiles: the
    two-stage pipeline's first, last and refetched k-tiles (f32 store), and
    the pair form whose W columns wrap after kw = K (2K columns of A)."""
    q = Q()
    M, N = 300, 512
    A = f16_host(13, 1, (M, K), 1.0)
    W = f16_host(13, 2, (N, K), 0.05)
    out = torch.zeros(M, N, device="cuda", dtype=torch.float32)
    q.qi21_op_gemm(q.QI21_EPI_F32, M, N, K, dev(A, torch.float16), K, dev(W, torch.float16), out, N, tile=tile)
    sync()
    assert_close(out.cpu().numpy(), O.lin(A, W), F32_TOL * 10)
    A32 = inputs.host_array(13, 3, (M, K), 1.0)
    hi, lo = _pair(A32)
    Ap = np.concatenate([hi, lo], axis=1)
    x = np.zeros((M, N), np.float32)
    gate = np.ones(N, np.float32)
    dx = dev(x)
    q.qi21_op_gemm_resid(M, N, 2 * K, K, dev(Ap, torch.float16), 2 * K, dev(W, torch.float16), dx, N, dev(gate), 1.0,
                         tile)
    sync()
    want = A32.astype(np.float64) @ W.astype(np.float64).T
    assert_close(dx.cpu().numpy(), want, PAIR_TOL)


@pytest.mark.parametrize("tile", [0, 2])
@pytest.mark.parametrize("ksplit,K", [(2, 256), (3, 576), (4, 4352), (4, 1024)])
@pytest.mark.parametrize("M", [1, 300, 1024])
def test_gemm_split_partials(M, ksplit, K, tile):
    """Each partial plane is the product over its quarter (third, half) of K;
    the planes add up to the whole product.  The pair form (A of K columns,
    W rows of kw = K / 2, each read twice) splits the same way."""
    q = Q()
    N = 512
    A = f16_host(14, 1, (M, K), 1.0)
    W = f16_host(14, 2, (N, K), 0.05)
    part = torch.zeros(ksplit, M, N, device="cuda")
    q.qi21_op_gemm_split(M, N, K, K, dev(A, torch.float16), K, dev(W, torch.float16), part, ksplit, 0.5, tile)
    sync()
    ks = K // ksplit
    got = part.cpu().numpy()
    for p in range(ksplit):
        want = O.lin(A[:, p * ks:(p + 1) * ks], W[:, p * ks:(p + 1) * ks]) * np.float32(0.5)
        assert_close(got[p], want, F32_TOL * 10)
    assert_close(got.sum(axis=0), O.lin(A, W) * np.float32(0.5), F32_TOL * 10)
    if K % (128 * ksplit) == 0:
        kw = K // 2
        Wp = W[:, :kw]
        part.zero_()
        q.qi21_op_gemm_split(M, N, K, kw, dev(A, torch.float16), K, dev(Wp, torch.float16), part, ksplit, 1.0, tile)
        sync()
        want = A[:, :kw].astype(np.float64) @ Wp.astype(np.float64).T + A[:, kw:].astype(np.float64) @ Wp.astype(np.float64).T
        assert_close(part.cpu().numpy().sum(axis=0), want, F32_TOL * 10)


@pytest.mark.parametrize("nparts", [1, 2, 3, 4])
@pytest.mark.parametrize("mode", [1, 3, 7])
def test_rowop_adds_partial_planes(mode, nparts):
    """x += gate * (sum of the planes, in order), then the modulated LayerNorm
    (and its f16 pair for mode 7), against the same computation in numpy."""
    q = Q()
    rows, h = 37, 4096
    x = inputs.host_array(15, 1, (rows, h), 1.0)
    y = inputs.host_array(15, 2, (nparts, rows + 3, h), 1.0)  # planes rows + 3 rows apart
    mods = inputs.host_array(15, 3, (4 * h,), 0.1)
    g_off, s_off, eps, oscale = 3 * h, 0, 1e-6, 0.25
    dx, xn = dev(x), torch.zeros(rows, 2 * h if mode & 4 else h, device="cuda", dtype=torch.float16)
    q.qi21_op_rowop_parts(rows, h, mode, dx, dev(y), nparts, (rows + 3) * h, xn, xn.shape[1], dev(mods), g_off, s_off, eps, oscale)
    sync()
    ysum = y[0, :rows].copy()
    for p in range(1, nparts):
        ysum = ysum + y[p, :rows]
    xw = x + mods[g_off:g_off + h] * ysum
    assert_close(dx.cpu().numpy(), xw, F32_TOL)
    if mode & 2:
        v = O.layer_norm(xw, eps) * (1.0 + mods[s_off:s_off + h]) * np.float32(oscale)
        got = xn.float().cpu().numpy()
        if mode & 4:
            got = got[:, :h] + got[:, h:]
            assert_close(got, v, F32_TOL)
        else:
            assert_close(got, v, F16_TOL)


@pytest.mark.parametrize("tile", [0, 2])
@pytest.mark.parametrize("M", [1, 77, 300, 1600])
def test_qk_gemm_fused_norm_rope(M, tile):
    """q|k projection with the per-head RMSNorm + RoPE in the epilogue vs
    the oracle's lin then qk_norm_rope on the same f16 inputs"""
    q = Q()
    heads, hd = 2, 128
    H = heads * hd
    lay = O.Layout([("text", 7), ("image", 40, 41)])
    pos = lay.positions()[:M]
    c, s = O.rope_tables(pos)
    A = f16_host(10, 1, (M, H), 0.25)  # the attention input carries 2^-2
    W = f16_host(10, 2, (2 * H, H), 0.05)
    wq = inputs.host_array(10, 3, (hd,), 0.02, mean=1.0)
    wk = inputs.host_array(10, 4, (hd,), 0.02, mean=1.0)
    eps = 1e-6 * 2.0 ** -4
    ldq, ldk = H + 64, H
    qo = torch.zeros(M, ldq, device="cuda", dtype=torch.float16)
    ko = torch.zeros(M, ldk, device="cuda", dtype=torch.float16)
    rope = torch.empty(M, 128, device="cuda")
    q.qi21_op_rope_pack(M, dev(c), dev(s), rope)
    q.qi21_op_qk_gemm(M, H, dev(A, torch.float16), H, dev(W, torch.float16), qo, ldq, ko, ldk, dev(wq), dev(wk),
                      rope, eps, tile)
    sync()
    want_q = O.qk_norm_rope(O.lin(A, W[:H]), wq, c, s, heads, hd, eps)
    want_k = O.qk_norm_rope(O.lin(A, W[H:]), wk, c, s, heads, hd, eps)
    got_q = qo.float().cpu().numpy()
    assert_close(got_q[:, :H], want_q, F16_TOL)
    assert_close(ko.float().cpu().numpy(), want_k, F16_TOL)
    assert np.all(got_q[:, H:] == 0)  # nothing past the q heads


@pytest.mark.parametrize("tile", [0, 2])
@pytest.mark.parametrize("nkeys", [1, 18, 300, 4118])
def test_vt_gemm_key_order_and_bound(nkeys, tile):
    """V^T = Wv X^T with key j at vt_pos(j), only keys < nkeys written"""
    q = Q()
    H, K = 384, 256
    rows = ((nkeys + 255) // 256) * 256
    X = np.zeros((rows, K), np.float32)
    X[:nkeys] = f16_host(11, 1, (nkeys, K), 1.0)
    Wv = f16_host(11, 2, (H, K), 0.05)
    ldo = ((nkeys + 63) // 64) * 64 + 8
    out = torch.zeros(H, ldo, device="cuda", dtype=torch.float16)
    q.qi21_op_vt_gemm(H, nkeys, K, dev(Wv, torch.float16), K, dev(X, torch.float16), out, ldo, 0.5, tile)
    sync()
    got = out.float().cpu().numpy()
    want = (O.lin(X[:nkeys], Wv) * np.float32(0.5)).T
    cols = vt_pos(np.arange(nkeys))
    assert_close(got[:, cols], want, F16_TOL)
    rest = np.setdiff1d(np.arange(ldo), cols)
    assert np.all(got[:, rest] == 0)


@pytest.mark.parametrize("h", [256, 4096])
@pytest.mark.parametrize("rows", [1, 100, 300])
def test_embed(rows, h):
    q = Q()
    tok = inputs.host_array(11, 1, (rows, 64), 1.0)
    w = inputs.host_array(11, 2, (h, 64), 0.02)
    x = torch.zeros(rows, h, device="cuda")
    q.qi21_op_embed(rows, h, dev(tok), dev(w), x)
    sync()
    assert_close(x.cpu().numpy(), O.embed_image(tok, w), F32_TOL)


@pytest.mark.parametrize("h", [256, 4096])
@pytest.mark.parametrize("rows", [1, 17, 300])
@pytest.mark.parametrize("offset", [0.5, 200.0])
def test_final_and_nonfinite_flag(rows, h, offset):
    """The final layer against the oracle; a large common offset of the rows
    checks that the LayerNorm statistics do not cancel."""
    q = Q()
    x = inputs.host_array(12, 1, (rows, h), 1.0) * np.float32(3.0) + np.float32(offset)
    fs = 1.0 + inputs.host_array(12, 2, (h,), 0.1)
    po = inputs.host_array(12, 3, (64, h), 0.02)
    out = torch.zeros(rows, 64, device="cuda")
    flag = torch.zeros(1, device="cuda", dtype=torch.int32)
    q.qi21_op_final(rows, h, dev(x), dev(fs), dev(po), 1e-6, out, flag)
    sync()
    want = O.lin(O.layer_norm(x, 1e-6) * fs, po)  # LN(x) * (1 + final_scale), fs = 1 + final_scale
    assert_close(out.cpu().numpy(), want, F32_TOL)
    assert int(flag.item()) == 0
    x[rows // 2, 3] = np.inf
    q.qi21_op_final(rows, h, dev(x), dev(fs), dev(po), 1e-6, out, flag)
    sync()
    assert int(flag.item()) == 1


def test_mods_gate_tanh_pages_example():
    q = Q()
    h = 3
    m = (np.arange(12, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    out = torch.zeros(12, device="cuda")
    q.qi21_op_mods(h, dev(m), out)
    sync()
    d = out.cpu().numpy()
    assert np.array_equal(d[:3], m[:3]) and np.array_equal(d[6:9], m[6:9])
    assert abs(d[4] - math.tanh(0.4)) < 1e-6 and abs(d[11] - math.tanh(1.1)) < 1e-6
