"""Python binding of the qi21 C ABI (``include/qi21.h``, ``include/qi21_ops.h``).

Argument marshalling only: every function has the C entry point's name and
arguments, takes torch tensors (or raw device addresses) where the C call
takes device pointers, and raises :class:`Qi21Error` (with the status code
and ``qi21_last_error()``) when the call does not return ``QI21_OK``.  All
compute runs in the HIP library; importing this module fails loudly when
``libqi21.so`` has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqi21.so")

QI21_OK, QI21_EINVAL, QI21_EUNSUPPORTED, QI21_ENOMEM, QI21_ENOKEY, QI21_ENONFINITE, QI21_EDEVICE = range(7)
QI21_F32, QI21_BF16, QI21_F16 = 0, 1, 2
QI21_EPI_F16, QI21_EPI_F32, QI21_EPI_SWIGLU, QI21_EPI_QKV, QI21_EPI_SWIGLU2 = 0, 1, 2, 3, 4
QI21_EPI_RESID, QI21_EPI_SWIGLU8, QI21_EPI_SWIGLU4 = 7, 9, 10
QI21_FFN_F16, QI21_FFN_PAIR, QI21_FFN_LO8, QI21_FFN_LO4 = 0, 1, 2, 3
PROFILE_CLASSES = ("qkv", "qkrope", "flash", "o", "gate_up", "down", "rowop", "io")

C = ctypes
vp, i32, i64, u32, u64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64, C.c_float


class Qi21Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"qi21 status {code}: {msg}")
        self.code = code


class qi21_geom(C.Structure):
    _fields_ = [("hidden", i32), ("heads", i32), ("head_dim", i32), ("inter", i32), ("in_ch", i32), ("eps", f32)]


ALLOC_FN = C.CFUNCTYPE(vp, C.c_size_t, vp)
FREE_FN = C.CFUNCTYPE(None, vp, vp)


class qi21_options(C.Structure):
    _fields_ = [("shift_attn", i32), ("shift_qkv", i32), ("shift_ao", i32), ("shift_ffn", i32), ("shift_hid", i32),
                ("max_programs", i32), ("profile", i32), ("gemm_tile", i32), ("ffn_mode", i32),
                ("alloc", ALLOC_FN), ("free", FREE_FN), ("alloc_ctx", vp)]


class qi21_seg(C.Structure):
    _fields_ = [("kind", i32), ("h", i32), ("w", i32)]


_SIGS = {
    "qi21_default_options": (None, [C.POINTER(qi21_options)]),
    "qi21_model_create": (C.c_int, [C.POINTER(qi21_geom), C.POINTER(qi21_options), C.c_int, vp, vp, vp, C.POINTER(vp)]),
    "qi21_model_set_block": (C.c_int, [vp, C.c_int, C.c_int, C.POINTER(vp), vp, vp, vp]),
    "qi21_prefill": (C.c_int, [vp, u64, C.c_int, C.c_int, vp, vp, vp, vp, vp, vp, vp, vp]),
    "qi21_step": (C.c_int, [vp, u64, vp, vp, vp, vp, vp]),
    "qi21_step_batch": (C.c_int, [vp, C.c_int, C.POINTER(u64), C.POINTER(vp), vp, vp, C.POINTER(vp), vp]),
    "qi21_release_key": (C.c_int, [vp, u64]),
    "qi21_model_set_time": (C.c_int, [vp, C.c_int, vp, vp, vp, vp, vp]),
    "qi21_model_set_txt_in": (C.c_int, [vp, C.c_int, C.c_int, vp, vp, vp, vp]),
    "qi21_txt_in": (C.c_int, [vp, C.c_int, vp, vp, vp]),
    "qi21_txt_in_noalloc": (C.c_int, [vp, C.c_int, vp, vp, vp]),
    "qi21_txt_in_noalloc_bytes": (C.c_size_t, []),
    "qi21_time_mods": (C.c_int, [vp, f32, vp, vp, vp]),
    "qi21_step_t": (C.c_int, [vp, u64, vp, f32, vp, vp]),
    "qi21_sample": (C.c_int, [vp, u64, vp, C.c_int, C.POINTER(f32), vp]),
    "qi21_model_destroy": (None, [vp]),
    "qi21_last_error": (C.c_char_p, []),
    "qi21_model_bytes": (C.c_size_t, [vp]),
    "qi21_profile_read": (C.c_int, [vp, C.POINTER(C.c_double), C.POINTER(i64)]),
    "qi21_set_profile": (C.c_int, [vp, C.c_int]),
    "qi21_set_profile_every": (C.c_int, [vp, C.c_int]),
    "qi21_layout_sizes": (C.c_int, [C.POINTER(qi21_seg), C.c_int, C.POINTER(i32), C.POINTER(i32)]),
    "qi21_layout_tables": (C.c_int, [C.POINTER(qi21_seg), C.c_int, C.POINTER(i32), f32, vp, vp, vp, vp, vp, vp]),
    "qi21_op_gemm": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, vp, C.c_int, vp, vp, C.c_int, vp, C.c_int, f32, f32,
                               C.c_int, vp]),
    "qi21_op_gemm_pair": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, vp, C.c_int, vp, vp, C.c_int, f32, f32, C.c_int,
                                    vp]),
    "qi21_op_gemm_split": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, vp, C.c_int, vp, vp, C.c_int, f32, C.c_int,
                                     vp]),
    "qi21_op_rowop_parts": (C.c_int, [C.c_int, C.c_int, C.c_int, vp, vp, C.c_int, C.c_size_t, vp, C.c_int, vp,
                                      C.c_int, C.c_int, f32, f32, vp]),
    "qi21_op_rowop_lo": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, vp, vp, C.c_int, C.c_size_t, vp, C.c_int, vp,
                                   vp, C.c_int, C.c_int, f32, f32, vp]),
    "qi21_op_gemm_lo": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, vp, C.c_int, vp, vp, C.c_int, vp, vp,
                                  C.c_int, vp, vp, C.c_int, f32, f32, vp]),
    "qi21_op_plane_lo": (C.c_int, [C.c_int, C.c_int, vp, C.c_int, C.c_int, vp, C.c_int, C.c_int, C.c_int, C.c_int,
                                   vp]),
    "qi21_op_plane_lo_fill": (C.c_int, [C.c_int, C.c_int, C.c_int, vp, C.c_int, vp, vp]),
    "qi21_op_gemm_resid": (C.c_int, [C.c_int, C.c_int, C.c_int, C.c_int, vp, C.c_int, vp, vp, C.c_int, vp, f32,
                                     C.c_int, vp]),
    "qi21_op_qk_gemm": (C.c_int, [C.c_int, C.c_int, vp, C.c_int, vp, vp, C.c_int, vp, C.c_int, vp, vp, vp, f32,
                                  C.c_int, vp]),
    "qi21_op_rope_pack": (C.c_int, [C.c_int, vp, vp, vp, vp]),
    "qi21_op_vt_gemm": (C.c_int, [C.c_int, C.c_int, C.c_int, vp, C.c_int, vp, vp, C.c_int, f32, C.c_int, vp]),
    "qi21_op_flash": (C.c_int, [C.c_int, C.c_int, vp, C.c_int, vp, C.c_int, vp, C.c_int, C.c_int, vp, C.c_int, vp,
                                C.c_int, C.c_int, vp, vp, C.c_int, f32, vp]),
    "qi21_op_rowop": (C.c_int, [C.c_int, C.c_int, C.c_int, vp, vp, vp, C.c_int, vp, C.c_int, C.c_int, f32, f32, vp]),
    "qi21_op_qkrope": (C.c_int, [C.c_int, C.c_int, vp, C.c_int, vp, vp, vp, vp, f32, vp, C.c_int, vp]),
    "qi21_op_embed": (C.c_int, [C.c_int, C.c_int, vp, vp, vp, vp]),
    "qi21_op_final": (C.c_int, [C.c_int, C.c_int, vp, vp, vp, f32, vp, vp, vp]),
    "qi21_op_mods": (C.c_int, [C.c_int, vp, vp, vp]),
    "qi21_op_plane": (C.c_int, [C.c_int, vp, C.c_int, C.c_int, vp, C.c_int, C.c_int, C.c_int, vp]),
}

_lib = None


def lib():
    """The loaded ``libqi21.so`` (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m diffusion_transformer_denoiser_qi21_amd.build` (there is no fallback path)")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def exported_symbols():
    return tuple(_SIGS)


def _p(t) -> Optional[int]:
    """Device (or host) address of a tensor / array, a raw int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> int:
    if rc != QI21_OK:
        raise Qi21Error(rc, qi21_last_error())
    return rc


def qi21_last_error() -> str:
    return lib().qi21_last_error().decode()


def qi21_default_options() -> qi21_options:
    o = qi21_options()
    lib().qi21_default_options(C.byref(o))
    return o


class DeviceAllocator:
    """The ``qi21_options`` alloc/free hook backed by torch's caching allocator.

    The library then takes its planes, activations and prefix caches from
    the same pool as the caller's tensors instead of calling hipMalloc.
    ``budget`` (bytes, None = unlimited) makes an allocation return NULL once
    the live total would pass it, which the library reports as ENOMEM.
    ``live`` maps each address handed out to its size; ``failed`` counts the
    refused requests.  Callbacks never raise into C: any error is a NULL.
    """

    def __init__(self, device=None, budget: Optional[int] = None):
        import torch
        idx = None if device is None else torch.device(device).index
        self.device = torch.cuda.current_device() if idx is None else idx
        self.budget = budget
        self.live = {}
        self.failed = 0
        self.alloc = ALLOC_FN(self._alloc)
        self.free = FREE_FN(self._free)

    @property
    def live_bytes(self) -> int:
        return sum(self.live.values())

    def _alloc(self, nbytes, ctx):
        try:
            if self.budget is not None and self.live_bytes + nbytes > self.budget:
                self.failed += 1
                return None
            import torch
            p = int(torch.cuda.caching_allocator_alloc(int(nbytes), self.device))
            self.live[p] = int(nbytes)
            return p
        except Exception:
            self.failed += 1
            return None

    def _free(self, ptr, ctx):
        try:
            if ptr in self.live:
                del self.live[ptr]
                import torch
                torch.cuda.caching_allocator_delete(ptr)
        except Exception:
            pass

    def install(self, opt: qi21_options) -> qi21_options:
        opt.alloc, opt.free, opt.alloc_ctx = self.alloc, self.free, None
        return opt


# options (and with them any allocator callbacks) of each live model
_MODEL_OPTS = {}


def qi21_model_create(geom: qi21_geom, opt: Optional[qi21_options], nblocks: int, img_in, proj_out, stream=None):
    h = vp()
    _check(lib().qi21_model_create(C.byref(geom), C.byref(opt) if opt is not None else None, int(nblocks),
                                   _p(img_in), _p(proj_out), _stream(stream), C.byref(h)))
    _MODEL_OPTS[h.value] = opt
    return h


def _wdtype(t) -> int:
    import torch
    return {torch.float32: QI21_F32, torch.bfloat16: QI21_BF16, torch.float16: QI21_F16}[t.dtype]


def qi21_model_set_block(m, layer: int, w_dtype: Optional[int], w: Sequence, norm_q, norm_k, stream=None):
    if w_dtype is None:
        w_dtype = _wdtype(w[0])
    arr = (vp * 7)(*[_p(t) for t in w])
    _check(lib().qi21_model_set_block(m, int(layer), int(w_dtype), arr, _p(norm_q), _p(norm_k), _stream(stream)))


def qi21_prefill(m, key: int, lp: int, n: int, x, rope_p_cos, rope_p_sin, rope_t_cos, rope_t_sin, vis, mods0,
                 stream=None):
    _check(lib().qi21_prefill(m, int(key), int(lp), int(n), _p(x), _p(rope_p_cos), _p(rope_p_sin), _p(rope_t_cos),
                              _p(rope_t_sin), _p(vis), _p(mods0), _stream(stream)))


def qi21_step(m, key: int, xtok, mods, fs, out, stream=None):
    _check(lib().qi21_step(m, int(key), _p(xtok), _p(mods), _p(fs), _p(out), _stream(stream)))


def qi21_step_batch(m, keys: Sequence[int], xtok: Sequence, mods, fs, out: Sequence, stream=None):
    n = len(keys)
    _check(lib().qi21_step_batch(m, n, (u64 * n)(*[int(k) for k in keys]), (vp * n)(*[_p(t) for t in xtok]),
                                 _p(mods), _p(fs), (vp * n)(*[_p(t) for t in out]), _stream(stream)))


def qi21_model_set_time(m, w_dtype: Optional[int], t_lin1, t_lin2, modulation, norm_out, stream=None):
    ws = (t_lin1, t_lin2, modulation, norm_out)
    dt = _wdtype(t_lin1) if w_dtype is None else w_dtype
    _check(lib().qi21_model_set_time(m, dt, *[_p(w) for w in ws], _stream(stream)))


def qi21_model_set_txt_in(m, context_in: int, w_dtype: Optional[int], txt_norm, txt_in1, txt_in2, stream=None):
    dt = _wdtype(txt_in1) if w_dtype is None else w_dtype
    _check(lib().qi21_model_set_txt_in(m, context_in, dt, _p(txt_norm), _p(txt_in1), _p(txt_in2), _stream(stream)))


def qi21_txt_in(m, n: int, feats, out, stream=None):
    _check(lib().qi21_txt_in(m, n, _p(feats), _p(out), _stream(stream)))


def qi21_txt_in_noalloc(m, n: int, feats, out, stream=None):
    _check(lib().qi21_txt_in_noalloc(m, int(n), _p(feats), _p(out), _stream(stream)))


def qi21_txt_in_noalloc_bytes() -> int:
    return int(lib().qi21_txt_in_noalloc_bytes())


def qi21_time_mods(m, t: float, mods, fs, stream=None):
    _check(lib().qi21_time_mods(m, float(t), _p(mods), _p(fs), _stream(stream)))


def qi21_step_t(m, key: int, xtok, t: float, out, stream=None):
    _check(lib().qi21_step_t(m, key, _p(xtok), float(t), _p(out), _stream(stream)))


def qi21_sample(m, key: int, x, times: Sequence[float], stream=None):
    n = len(times) - 1
    arr = (f32 * max(1, len(times)))(*[float(v) for v in times])
    _check(lib().qi21_sample(m, key, _p(x), n, arr, _stream(stream)))


def qi21_release_key(m, key: int):
    _check(lib().qi21_release_key(m, int(key)))


def qi21_model_destroy(m):
    lib().qi21_model_destroy(m)
    _MODEL_OPTS.pop(m.value if isinstance(m, vp) else m, None)


def qi21_model_bytes(m) -> int:
    return int(lib().qi21_model_bytes(m))


def qi21_set_profile(m, class_mask: int):
    _check(lib().qi21_set_profile(m, int(class_mask)))


def qi21_set_profile_every(m, every: int):
    _check(lib().qi21_set_profile_every(m, int(every)))


def qi21_profile_read(m):
    ms = (C.c_double * 8)()
    n = (i64 * 8)()
    _check(lib().qi21_profile_read(m, ms, n))
    return list(ms), list(n)


def _segs(segs):
    arr = (qi21_seg * len(segs))()
    for i, s in enumerate(segs):
        if s[0] == "text":
            arr[i] = qi21_seg(0, int(s[1]), 0)
        else:
            arr[i] = qi21_seg(1, int(s[1]), int(s[2]))
    return arr


def qi21_layout_sizes(segs):
    lp, n = i32(), i32()
    _check(lib().qi21_layout_sizes(_segs(segs), len(segs), C.byref(lp), C.byref(n)))
    return lp.value, n.value


def qi21_layout_tables(segs, axes=(16, 56, 56), theta: float = 10000.0):
    """Host arrays: pos [total,3] int64, vis [lp] uint32, cos_p/sin_p [lp,hd/2], cos_t/sin_t [n,hd/2]."""
    lp, n = qi21_layout_sizes(segs)
    half = sum(axes) // 2
    pos = np.zeros((lp + n, 3), np.int64)
    vis = np.zeros(lp, np.uint32)
    cp, sp = np.zeros((lp, half), np.float32), np.zeros((lp, half), np.float32)
    ct, st = np.zeros((n, half), np.float32), np.zeros((n, half), np.float32)
    ax = (i32 * 3)(*axes)
    _check(lib().qi21_layout_tables(_segs(segs), len(segs), ax, float(theta), _p(pos), _p(vis), _p(cp), _p(sp),
                                    _p(ct), _p(st)))
    return {"pos": pos, "vis": vis, "cos_p": cp, "sin_p": sp, "cos_t": ct, "sin_t": st, "lp": lp, "n": n}


# ── single-kernel entry points ──

def qi21_op_gemm(epi, M, N, K, A, lda, W, out, ldo, out2=None, ld2=0, oscale=1.0, inscale=1.0, tile=-1, stream=None):
    _check(lib().qi21_op_gemm(epi, M, N, K, _p(A), lda, _p(W), _p(out), ldo, _p(out2), ld2, oscale, inscale, tile,
                              _stream(stream)))


def qi21_op_gemm_pair(epi, M, N, K, A, lda, W, out, ldo, oscale=1.0, inscale=1.0, tile=-1, stream=None):
    _check(lib().qi21_op_gemm_pair(epi, M, N, K, _p(A), lda, _p(W), _p(out), ldo, oscale, inscale, tile,
                                   _stream(stream)))


def qi21_op_gemm_resid(M, N, K, kw, A, lda, W, x, ldx, gate, oscale=1.0, tile=-1, stream=None):
    _check(lib().qi21_op_gemm_resid(M, N, K, kw, _p(A), lda, _p(W), _p(x), ldx, _p(gate), oscale, tile,
                                    _stream(stream)))


def qi21_op_qk_gemm(M, H, A, lda, W, q_out, ldq, k_out, ldk, norm_q, norm_k, rope, eps, tile=-1, stream=None):
    _check(lib().qi21_op_qk_gemm(M, H, _p(A), lda, _p(W), _p(q_out), ldq, _p(k_out), ldk, _p(norm_q), _p(norm_k),
                                 _p(rope), eps, tile, _stream(stream)))


def qi21_op_rope_pack(n, cos, sin, out, stream=None):
    _check(lib().qi21_op_rope_pack(n, _p(cos), _p(sin), _p(out), _stream(stream)))


def qi21_op_vt_gemm(H, nkeys, K, Wv, lda, X, out, ldo, oscale=1.0, tile=-1, stream=None):
    _check(lib().qi21_op_vt_gemm(H, nkeys, K, _p(Wv), lda, _p(X), _p(out), ldo, oscale, tile, _stream(stream)))


def qi21_op_flash(nq, heads, q, ldq, k1, ldk1, vt1, ldvt1, n1, k2, ldk2, vt2, ldvt2, n2, vis, out, ldo, oscale=1.0,
                  stream=None):
    _check(lib().qi21_op_flash(nq, heads, _p(q), ldq, _p(k1), ldk1, _p(vt1), ldvt1, n1, _p(k2), ldk2, _p(vt2), ldvt2,
                               n2, _p(vis), _p(out), ldo, oscale, _stream(stream)))


def qi21_op_gemm_split(M, N, K, kw, A, lda, W, part, ksplit, oscale=1.0, tile=-1, stream=None):
    _check(lib().qi21_op_gemm_split(M, N, K, kw, _p(A), lda, _p(W), _p(part), ksplit, oscale, tile, _stream(stream)))


def qi21_op_rowop_parts(rows, h, mode, x, y, nparts, pstride, xn, ldxn, mods, g_off, s_off, eps, oscale,
                        stream=None):
    _check(lib().qi21_op_rowop_parts(rows, h, mode, _p(x), _p(y), nparts, pstride, _p(xn), ldxn, _p(mods), g_off,
                                     s_off, eps, oscale, _stream(stream)))


def qi21_op_rowop(rows, h, mode, x, y, xn, ldxn, mods, g_off, s_off, eps, oscale, stream=None):
    _check(lib().qi21_op_rowop(rows, h, mode, _p(x), _p(y), _p(xn), ldxn, _p(mods), g_off, s_off, eps, oscale,
                               _stream(stream)))


def qi21_op_rowop_lo(fmt, rows, h, mode, x, y, nparts, pstride, xn, ldxn, xsc, mods, g_off, s_off, eps, oscale,
                     stream=None):
    _check(lib().qi21_op_rowop_lo(fmt, rows, h, mode, _p(x), _p(y), nparts, pstride, _p(xn), ldxn, _p(xsc), _p(mods),
                                  g_off, s_off, eps, oscale, _stream(stream)))


def qi21_op_gemm_lo(fmt, epi, M, N, K, A, lda, asc, W, ldw, wsc, out, ldo, gate=None, osc=None, ksplit=1,
                    oscale=1.0, inscale=1.0, stream=None):
    _check(lib().qi21_op_gemm_lo(fmt, epi, M, N, K, _p(A), lda, _p(asc), _p(W), ldw, _p(wsc), _p(out), ldo, _p(gate),
                                 _p(osc), ksplit, oscale, inscale, _stream(stream)))


def qi21_op_plane_lo(fmt, src_dtype, src, rows, cols, dst, ld, group, gstride, goff, stream=None):
    _check(lib().qi21_op_plane_lo(fmt, src_dtype, _p(src), rows, cols, _p(dst), ld, group, gstride, goff,
                                  _stream(stream)))


def qi21_op_plane_lo_fill(fmt, rows, cols, plane, ld, sc, stream=None):
    _check(lib().qi21_op_plane_lo_fill(fmt, rows, cols, _p(plane), ld, _p(sc), _stream(stream)))


def qi21_op_qkrope(rows, heads, panel, ldp, norm_q, norm_k, cos, sin, eps, kdst=None, ldk=0, stream=None):
    _check(lib().qi21_op_qkrope(rows, heads, _p(panel), ldp, _p(norm_q), _p(norm_k), _p(cos), _p(sin), eps, _p(kdst),
                                ldk, _stream(stream)))


def qi21_op_embed(rows, h, tok, img_in, x, stream=None):
    _check(lib().qi21_op_embed(rows, h, _p(tok), _p(img_in), _p(x), _stream(stream)))


def qi21_op_final(rows, h, x, fs, proj_out, eps, out, flag, stream=None):
    _check(lib().qi21_op_final(rows, h, _p(x), _p(fs), _p(proj_out), eps, _p(out), _p(flag), _stream(stream)))


def qi21_op_mods(h, mods, mods_dev, stream=None):
    _check(lib().qi21_op_mods(h, _p(mods), _p(mods_dev), _stream(stream)))


def qi21_op_plane(src_dtype, src, rows, cols, dst, group, gstride, goff, stream=None):
    _check(lib().qi21_op_plane(src_dtype, _p(src), rows, cols, _p(dst), group, gstride, goff, _stream(stream)))
