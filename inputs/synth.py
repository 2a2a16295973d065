"""Counter-based generator of seeded synthetic tensors.

Every element is a pure function of (seed, tensor id, flat index), so any
slice of any tensor can be regenerated anywhere, and the CPU copy (C code in
``csrc/synth.c``) and the device copy (torch integer ops below) give the same
bits.  The distribution is the Irwin-Hall(4) approximation of a normal
N(mean, sigma^2) described at the top of ``csrc/synth.c``.

Holds none of the denoiser's arithmetic.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_M32 = 0xFFFFFFFF
_lib = None


def build_native() -> str:
    """Compile the CPU generator (gcc, OpenMP) next to this file."""
    cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-o", _LIB + ".tmp", _SRC]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _native():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_native()
        lib = ctypes.CDLL(_LIB)
        lib.synth_fill_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_uint32, ctypes.c_double, ctypes.c_double,
                                       ctypes.c_int]
        lib.synth_fill_f32.restype = None
        lib.synth_mix32.argtypes = [ctypes.c_uint32]
        lib.synth_mix32.restype = ctypes.c_uint32
        _lib = lib
    return _lib


def _mix32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x21F0AAAD) & _M32
    x ^= x >> 15
    x = (x * 0x735A2D97) & _M32
    x ^= x >> 15
    return x


def tensor_key(seed: int, tid: int) -> int:
    """32-bit stream key of tensor ``tid`` under ``seed``."""
    return _mix32_int(_mix32_int(seed * 0x9E3779B1 + 0x7F4A7C15) ^ ((tid * 0x85EBCA6B) & _M32) ^ (tid >> 32))


def _scale(sigma: float) -> float:
    return float(sigma) * math.sqrt(3.0) / 131072.0


def host_array(seed: int, tid: int, shape, sigma: float = 1.0, mean: float = 0.0,
               bf16: bool = False, start: int = 0) -> np.ndarray:
    """float32 numpy array of the tensor (values bf16-rounded if ``bf16``).

    ``start`` offsets the flat index, so a slice of a large tensor can be
    produced without the rest.
    """
    shape = tuple(int(s) for s in np.atleast_1d(shape)) if not isinstance(shape, tuple) else shape
    count = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(count, dtype=np.float32)
    if count:
        _native().synth_fill_f32(out.ctypes.data, int(start), count, tensor_key(seed, tid),
                                 _scale(sigma), float(mean), int(bool(bf16)))
    return out.reshape(shape)


def _torch_mix32(x):
    x = x ^ (x >> 16)
    x = (x * 0x21F0AAAD) & _M32
    x = x ^ (x >> 15)
    x = (x * 0x735A2D97) & _M32
    x = x ^ (x >> 15)
    return x


def device_tensor(seed: int, tid: int, shape, sigma: float = 1.0, mean: float = 0.0,
                  bf16: bool = False, device="cuda", chunk: int = 1 << 24):
    """The same tensor generated with torch integer ops on ``device``.

    Returns float32, or bfloat16 when ``bf16`` (the values then equal
    ``host_array(..., bf16=True)`` exactly).  All products stay below 2^63
    (a value below 2^32 times a constant below 2^31), so int64 arithmetic
    reproduces the 32-bit wrap-around of the C code exactly.
    """
    import torch

    shape = tuple(int(s) for s in shape)
    count = int(np.prod(shape)) if len(shape) else 1
    key = tensor_key(seed, tid)
    scale = _scale(sigma)
    out = torch.empty(count, dtype=torch.bfloat16 if bf16 else torch.float32, device=device)
    for lo in range(0, count, chunk):
        n = min(chunk, count - lo)
        i = torch.arange(lo, lo + n, dtype=torch.int64, device=device)
        h1 = _torch_mix32(_torch_mix32((i & _M32) ^ key) ^ (i >> 32))
        h2 = _torch_mix32(h1 ^ 0x9E3779B9)
        s = (h1 & 0xFFFF) + (h1 >> 16) + (h2 & 0xFFFF) + (h2 >> 16)
        z = (2 * s + 4 - 262144).to(torch.float64) * scale
        z = z + float(mean)
        out[lo:lo + n] = z.to(torch.float32).to(out.dtype)
        del i, h1, h2, s, z
    return out.reshape(shape)
