"""qi21: the Qwen-Image-2.1 single-stream denoiser step on AMD MI355X (gfx950).

The product is ``libqi21.so`` (hand-written HIP kernels behind the C ABI of
``include/qi21.h``); ``qi21`` is its ctypes binding.
"""
from . import qi21  # noqa: F401
from .qi21 import Qi21Error  # noqa: F401
