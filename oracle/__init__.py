"""CPU oracle of the Qwen-Image-2.1 denoiser step -- test infrastructure only.

Only the tests, the package's smoke check and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU library.
"""
from . import qi21_oracle  # noqa: F401
from .model import SynthModel, workload_inputs  # noqa: F401
