"""Seeded synthetic inputs for the Qwen-Image-2.1 denoiser workloads.

Shared by the oracle's tests, the GPU parity tests and the benchmark.  This
package holds no arithmetic of the denoiser: only a counter-based random
generator, the workload definitions (shapes, seeds, distributions) and the
tensor naming scheme.
"""
from .synth import (  # noqa: F401
    build_native,
    host_array,
    device_tensor,
    tensor_key,
)
from .configs import CONFIGS, ModelSpec, Workload, model_spec  # noqa: F401
