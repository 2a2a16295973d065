"""The C ABI on the host: the library loads, exports every declared symbol,
its layout helpers reproduce the pages' worked values, and its host-side
validation refuses bad arguments before any device work (no GPU needed)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from diffusion_transformer_denoiser_qi21_amd import qi21 as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_examples.json")))


def _declared(header):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(qi21_\w+)\s*\(", src))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(Q.LIB_PATH)
    declared = _declared("qi21.h") | _declared("qi21_ops.h")
    assert len(declared) >= 20
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(Q.exported_symbols())


def test_layout_sizes_and_errors():
    assert Q.qi21_layout_sizes([("text", 18), ("image", 64, 64)]) == (18, 4096)
    assert Q.qi21_layout_sizes([("text", 22), ("image", 64, 64), ("image", 64, 64)]) == (4118, 4096)
    for bad in ([("text", 3)], [("image", 2, 2)], [("text", 3), ("image", 0, 2)], [("text", 0), ("image", 2, 2)]):
        with pytest.raises(Q.Qi21Error) as e:
            Q.qi21_layout_sizes(bad)
        assert e.value.code == Q.QI21_EINVAL


def test_layout_positions_pages_worked_examples():
    g = GOLD["positions_t2i"]
    t = Q.qi21_layout_tables([tuple(s) for s in g["layout"]])
    for r, want in g["rows"].items():
        assert list(t["pos"][int(r)]) == want
    assert t["lp"] == g["prefix_len"]
    g = GOLD["positions_text_after_image"]
    t = Q.qi21_layout_tables([tuple(s) for s in g["layout"]])
    for r, want in g["rows"].items():
        assert list(t["pos"][int(r)]) == want


def test_layout_rope_tables_unit_and_identity():
    g = GOLD["rope_unit_rotations"]
    t = Q.qi21_layout_tables([tuple(s) for s in g["layout"]], tuple(g["axes"]), g["theta"])
    c = np.concatenate([t["cos_p"], t["cos_t"]]).astype(np.float64)
    s = np.concatenate([t["sin_p"], t["sin_t"]]).astype(np.float64)
    assert c.shape[1] == g["columns_per_row"]
    assert np.all(np.abs(c * c + s * s - 1) < g["unit_tol"])
    assert np.all(np.abs(c[0] - 1) < g["identity_at_position_zero_tol"])


def test_layout_vis_block_causal():
    t = Q.qi21_layout_tables([("text", 3), ("image", 2, 2), ("text", 2), ("image", 1, 1)])
    assert list(t["vis"]) == [1, 2, 3, 7, 7, 7, 7, 8, 9]
    t = Q.qi21_layout_tables([("text", 22), ("image", 64, 64), ("image", 64, 64)])
    assert list(t["vis"][:22]) == list(range(1, 23)) and np.all(t["vis"][22:] == 4118)


def test_default_options_are_the_pages_guards():
    o = Q.qi21_default_options()
    assert (o.shift_attn, o.shift_qkv, o.shift_ao, o.shift_ffn, o.shift_hid) == (2, 4, 4, 2, 8)
    assert o.max_programs == 2 and o.gemm_tile == -1 and o.ffn_mode == 0


def _geom(**kw):
    d = dict(hidden=256, heads=2, head_dim=128, inter=768, in_ch=64, eps=1e-6)
    d.update(kw)
    return Q.qi21_geom(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64, hidden=128), Q.QI21_EUNSUPPORTED),
    (dict(heads=3), Q.QI21_EUNSUPPORTED),
    (dict(inter=100), Q.QI21_EUNSUPPORTED),
    (dict(in_ch=32), Q.QI21_EUNSUPPORTED),
    (dict(hidden=16384, heads=128), Q.QI21_EUNSUPPORTED),
])
def test_model_create_refuses_geometry_before_device_work(kw, code):
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_model_create(_geom(**kw), None, 2, 1, 1, stream=0)
    assert e.value.code == code


def test_model_create_refuses_null_and_block_count():
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_model_create(_geom(), None, 0, 1, 1, stream=0)
    assert e.value.code == Q.QI21_EINVAL
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_model_create(_geom(), None, 2, None, 1, stream=0)
    assert e.value.code == Q.QI21_EINVAL


def test_model_create_refuses_bad_ffn_mode_before_device_work():
    # the option is checked, and lo8's geometry bounds, before any allocation
    opt = Q.qi21_default_options()
    opt.ffn_mode = 4
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_model_create(_geom(), opt, 2, 1, 1, stream=0)
    assert e.value.code == Q.QI21_EINVAL
    opt.ffn_mode = Q.QI21_FFN_LO8
    g = _geom()
    g.hidden, g.heads = 384, 3  # hidden % 256 != 0
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_model_create(g, opt, 2, 1, 1, stream=0)
    assert e.value.code == Q.QI21_EUNSUPPORTED
    g = _geom()
    g.inter = 704  # inter % 128 != 0
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_model_create(g, opt, 2, 1, 1, stream=0)
    assert e.value.code == Q.QI21_EUNSUPPORTED
    opt.ffn_mode = Q.QI21_FFN_LO4
    g = _geom()
    g.inter = 640  # inter % 256 != 0 (fine for lo8)
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_model_create(g, opt, 2, 1, 1, stream=0)
    assert e.value.code == Q.QI21_EUNSUPPORTED


class _FakePool:
    """An alloc/free hook that hands out made-up addresses (never touched:
    qi21_model_create takes all its buffers before any device work) and
    refuses the request numbered ``fail_at``."""

    def __init__(self, fail_at):
        self.fail_at, self.n, self.live, self.freed = fail_at, 0, {}, []
        self.alloc = Q.ALLOC_FN(self._alloc)
        self.free = Q.FREE_FN(self._free)

    def _alloc(self, nbytes, ctx):
        self.n += 1
        if self.n - 1 == self.fail_at:
            return None
        p = 0x7f0000000000 + self.n * (1 << 32)
        self.live[p] = nbytes
        return p

    def _free(self, ptr, ctx):
        self.freed.append(ptr)
        del self.live[ptr]


@pytest.mark.parametrize("mode", [Q.QI21_FFN_F16, Q.QI21_FFN_LO4])
def test_failing_allocator_gives_enomem_and_every_block_back(mode):
    # per block: qkv, O, gate/up, down planes and the two RMSNorm weights
    # (+ the two scale arrays of a residual form); then img_in, proj_out and
    # the device flag
    per_block = 6 + (2 if mode == Q.QI21_FFN_LO4 else 0)
    total = 2 * per_block + 3
    for fail_at in (0, 1, per_block + 2, total - 1):
        pool = _FakePool(fail_at)
        opt = Q.qi21_default_options()
        opt.ffn_mode = mode
        pool_opt = opt
        pool_opt.alloc, pool_opt.free = pool.alloc, pool.free
        with pytest.raises(Q.Qi21Error) as e:
            Q.qi21_model_create(_geom(), pool_opt, 2, 1, 1, stream=0)
        assert e.value.code == Q.QI21_ENOMEM, (fail_at, str(e.value))
        assert "did not fit" in str(e.value)
        assert pool.n == fail_at + 1  # nothing asked after the refusal
        assert pool.live == {} and len(pool.freed) == fail_at == len(set(pool.freed))


def test_allocator_hooks_come_in_pairs():
    pool = _FakePool(None)
    opt = Q.qi21_default_options()
    opt.alloc = pool.alloc
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_model_create(_geom(), opt, 2, 1, 1, stream=0)
    assert e.value.code == Q.QI21_EINVAL and pool.n == 0


def test_op_entry_points_validate_shapes_on_host():
    L8, L4 = Q.QI21_FFN_LO8, Q.QI21_FFN_LO4
    cases = [
        lambda: Q.qi21_op_gemm(0, 16, 100, 64, 1, 64, 1, 1, 100, stream=0),        # N % 128
        lambda: Q.qi21_op_gemm(0, 16, 128, 60, 1, 64, 1, 1, 128, stream=0),        # K % 64
        lambda: Q.qi21_op_gemm(0, 16, 128, 64, 1, 60, 1, 1, 128, stream=0),        # lda < K
        lambda: Q.qi21_op_gemm(3, 16, 384, 64, 1, 64, 1, 1, 256, None, 0, stream=0),  # qkv without out2
        lambda: Q.qi21_op_gemm(0, 16, 128, 64, 1, 64, 1, 1, 128, tile=0, stream=0),   # 256 tile, N % 256
        lambda: Q.qi21_op_flash(0, 1, 1, 128, 1, 128, 1, 64, 10, None, 0, None, 0, 0, None, 1, 128, stream=0),
        lambda: Q.qi21_op_flash(4, 1, 1, 128, 1, 128, 1, 32, 40, None, 0, None, 0, 0, None, 1, 128, stream=0),
        lambda: Q.qi21_op_rowop(4, 4098, 2, 1, 1, 1, 4100, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop(4, 256, 4, 1, 1, 1, 512, 1, 0, 0, 1e-6, 1.0, stream=0),    # pair bit without the norm
        lambda: Q.qi21_op_rowop(4, 256, 5, 1, 1, 1, 512, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop(4, 256, 8, 1, 1, 1, 256, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_gemm(5, 16, 128, 64, 1, 64, 1, 1, 128, stream=0),           # no such epilogue
        # f16 output rows are written in 16-byte vectors: ldo % 8
        lambda: Q.qi21_op_gemm(0, 16, 128, 64, 1, 64, 1, 1, 132, stream=0),
        lambda: Q.qi21_op_gemm(2, 16, 256, 64, 1, 64, 1, 1, 132, stream=0),
        lambda: Q.qi21_op_qk_gemm(16, 256, 1, 256, 1, 1, 260, 1, 256, 1, 1, 1, 1e-6, stream=0),
        lambda: Q.qi21_op_vt_gemm(256, 100, 256, 1, 256, 1, 1, 116, stream=0),
        lambda: Q.qi21_op_gemm(4, 16, 128, 64, 1, 64, 1, 1, 64, stream=0),            # swiglu2 needs ldo >= N
        lambda: Q.qi21_op_gemm_pair(1, 16, 128, 64, 1, 100, 1, 1, 128, stream=0),     # lda < 2K
        lambda: Q.qi21_op_gemm_pair(3, 16, 384, 64, 1, 128, 1, 1, 384, stream=0),     # no qkv pair epilogue
        lambda: Q.qi21_op_qk_gemm(16, 200, 1, 256, 1, 1, 256, 1, 256, 1, 1, 1, 1e-6, stream=0),  # H % 128
        lambda: Q.qi21_op_qk_gemm(16, 256, 1, 256, 1, 1, 256, 1, 256, 1, 1, 1, 1e-6, tile=1, stream=0),
        lambda: Q.qi21_op_qk_gemm(16, 256, 1, 256, 1, 1, 256, 1, 256, 1, 1, None, 1e-6, stream=0),  # no table
        lambda: Q.qi21_op_rope_pack(0, 1, 1, 1, stream=0),
        lambda: Q.qi21_op_rope_pack(4, 1, None, 1, stream=0),
        lambda: Q.qi21_op_vt_gemm(256, 100, 256, 1, 256, 1, 1, 100, stream=0),        # ldo < round_up(n, 16)
        lambda: Q.qi21_op_vt_gemm(256, 100, 100, 1, 256, 1, 1, 112, stream=0),        # K % 64
        lambda: Q.qi21_op_qkrope(4, 2, 1, 256, 1, 1, 1, 1, 1e-6, stream=0),
        lambda: Q.qi21_op_embed(4, 100, 1, 1, 1, stream=0),
        lambda: Q.qi21_op_final(4, 100, 1, 1, 1, 1e-6, 1, 1, stream=0),
        lambda: Q.qi21_op_gemm_split(16, 256, 192, 192, 1, 192, 1, 1, 2, stream=0),     # K % (64 ksplit)
        lambda: Q.qi21_op_gemm_split(16, 256, 256, 256, 1, 256, 1, 1, 9, stream=0),     # ksplit > 8
        lambda: Q.qi21_op_gemm_split(16, 128, 256, 256, 1, 256, 1, 1, 2, stream=0),     # N % 256
        lambda: Q.qi21_op_gemm_split(16, 256, 256, 256, 1, 256, 1, 1, 2, tile=1, stream=0),
        lambda: Q.qi21_op_rowop_parts(4, 256, 3, 1, 1, 0, 1024, 1, 256, 1, 0, 0, 1e-6, 1.0, stream=0),  # nparts 0
        lambda: Q.qi21_op_rowop_parts(4, 256, 3, 1, 1, 2, 1000, 1, 256, 1, 0, 0, 1e-6, 1.0, stream=0),  # planes overlap
        # the xn row stride: at least h, 2h with the pair bit, a multiple of 4
        lambda: Q.qi21_op_rowop(4, 256, 2, 1, 1, 1, 252, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop(4, 256, 6, 1, 1, 1, 256, 1, 0, 0, 1e-6, 1.0, stream=0),    # pair rows into [rows][h]
        lambda: Q.qi21_op_rowop(4, 256, 2, 1, 1, 1, 258, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop_parts(4, 256, 7, 1, 1, 2, 1024, 1, 500, 1, 0, 0, 1e-6, 1.0, stream=0),
        # the residual-form row op: h % 128 (lo8) / 256 (lo4), ldxn >= 1.5 h / 1.25 h, scales,
        # modes 2 / 3 only, a known format
        lambda: Q.qi21_op_rowop_lo(L8, 4, 192, 2, 1, 1, 1, 0, 1, 288, 1, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop_lo(L8, 4, 256, 2, 1, 1, 1, 0, 1, 380, 1, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop_lo(L8, 4, 256, 2, 1, 1, 1, 0, 1, 384, None, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop_lo(L8, 4, 256, 6, 1, 1, 1, 0, 1, 512, 1, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop_lo(L4, 4, 384, 2, 1, 1, 1, 0, 1, 480, 1, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop_lo(L4, 4, 512, 2, 1, 1, 1, 0, 1, 636, 1, 1, 0, 0, 1e-6, 1.0, stream=0),
        lambda: Q.qi21_op_rowop_lo(5, 4, 512, 2, 1, 1, 1, 0, 1, 1024, 1, 1, 0, 0, 1e-6, 1.0, stream=0),
        # the residual-form GEMM: K % 128 / 256, N % 256, lda / ldw, split, epilogue arguments
        lambda: Q.qi21_op_gemm_lo(L8, 1, 16, 256, 192, 1, 288, 1, 1, 288, 1, 1, 256, stream=0),   # K % 128
        lambda: Q.qi21_op_gemm_lo(L8, 1, 16, 128, 256, 1, 384, 1, 1, 384, 1, 1, 128, stream=0),   # N % 256
        lambda: Q.qi21_op_gemm_lo(L8, 1, 16, 256, 256, 1, 256, 1, 1, 384, 1, 1, 256, stream=0),   # lda < 1.5 K
        lambda: Q.qi21_op_gemm_lo(L8, 1, 16, 256, 256, 1, 384, 1, 1, 380, 1, 1, 256, stream=0),   # ldw
        lambda: Q.qi21_op_gemm_lo(L8, 1, 16, 256, 256, 1, 384, 1, 1, 384, 1, 1, 256, ksplit=3, stream=0),
        lambda: Q.qi21_op_gemm_lo(L8, 7, 16, 256, 256, 1, 384, 1, 1, 384, 1, 1, 256, stream=0),   # no gate
        lambda: Q.qi21_op_gemm_lo(L8, 9, 16, 512, 256, 1, 384, 1, 1, 384, 1, 1, 384, stream=0),   # no osc
        lambda: Q.qi21_op_gemm_lo(L8, 10, 16, 512, 256, 1, 384, 1, 1, 384, 1, 1, 384, osc=1, stream=0),  # lo4 SwiGLU
        lambda: Q.qi21_op_gemm_lo(L8, 0, 16, 256, 256, 1, 384, 1, 1, 384, 1, 1, 256, stream=0),   # F16
        lambda: Q.qi21_op_gemm_lo(L8, 7, 16, 256, 256, 1, 384, 1, 1, 384, 1, 1, 256, gate=1, ksplit=2, stream=0),
        lambda: Q.qi21_op_gemm_lo(L4, 1, 16, 256, 384, 1, 480, 1, 1, 480, 1, 1, 256, stream=0),   # K % 256
        lambda: Q.qi21_op_gemm_lo(L4, 1, 16, 256, 512, 1, 632, 1, 1, 640, 1, 1, 256, stream=0),   # lda
        lambda: Q.qi21_op_gemm_lo(L4, 1, 16, 256, 512, 1, 640, 1, 1, 640, 1, 1, 256, ksplit=3, stream=0),
        lambda: Q.qi21_op_gemm_lo(L4, 9, 16, 1024, 512, 1, 640, 1, 1, 640, 1, 1, 640, osc=1, stream=0),  # lo8 SwiGLU
        lambda: Q.qi21_op_gemm_lo(L4, 10, 16, 512, 512, 1, 640, 1, 1, 640, 1, 1, 312, osc=1, stream=0),  # ldo
        lambda: Q.qi21_op_gemm_lo(L4, 10, 16, 256, 512, 1, 640, 1, 1, 640, 1, 1, 320, osc=1, stream=0),  # N / 2 % 256
        lambda: Q.qi21_op_plane_lo(L8, 0, 1, 16, 192, 1, 288, 16, 0, 0, stream=0),
        lambda: Q.qi21_op_plane_lo(L8, 0, 1, 16, 256, 1, 256, 16, 0, 0, stream=0),
        lambda: Q.qi21_op_plane_lo(L4, 0, 1, 16, 384, 1, 480, 16, 0, 0, stream=0),
        lambda: Q.qi21_op_plane_lo(L4, 0, 1, 16, 512, 1, 636, 16, 0, 0, stream=0),
        lambda: Q.qi21_op_plane_lo_fill(L8, 16, 256, 1, 380, 1, stream=0),
        lambda: Q.qi21_op_plane_lo_fill(L8, 16, 256, 1, 384, None, stream=0),
        lambda: Q.qi21_op_plane_lo_fill(L4, 16, 512, 1, 636, 1, stream=0),
        lambda: Q.qi21_op_plane_lo_fill(2 * L4, 16, 512, 1, 640, 1, stream=0),
    ]
    for c in cases:
        with pytest.raises(Q.Qi21Error) as e:
            c()
        assert e.value.code == Q.QI21_EINVAL


def test_null_model_calls_are_refused():
    with pytest.raises(Q.Qi21Error) as e:
        Q.qi21_step(None, 1, 1, 1, 1, 1, stream=0)
    assert e.value.code == Q.QI21_EINVAL
    with pytest.raises(Q.Qi21Error):
        Q.qi21_release_key(None, 1)
    Q.qi21_model_destroy(None)
