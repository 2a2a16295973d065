"""The seeded generator: CPU (C) and torch copies agree bit for bit, and the moments are right."""
import numpy as np
import torch

import inputs


def test_c_and_torch_generators_agree_bitwise():
    for seed, tid, n, sig, mean, bf in [(7, 100, 70_001, 0.02, 0.0, True), (21, 107, 128, 0.02, 1.0, False),
                                        (1024, 11, 4096 * 64, 1.0, 0.0, False), (3, 12, 999, 0.1, 0.0, True)]:
        a = inputs.host_array(seed, tid, (n,), sig, mean=mean, bf16=bf)
        b = inputs.device_tensor(seed, tid, (n,), sig, mean=mean, bf16=bf, device="cpu", chunk=1 << 14)
        assert np.array_equal(a, b.float().numpy())


def test_slices_and_high_indices():
    a = inputs.host_array(5, 9, (3000,), 1.0)
    assert np.array_equal(inputs.host_array(5, 9, (1000,), 1.0, start=2000), a[2000:])
    hi = inputs.host_array(5, 9, (64,), 1.0, start=(1 << 33) + 5)
    assert np.all(np.isfinite(hi)) and not np.array_equal(hi, a[5:69])


def test_moments_and_bf16_rounding():
    a = inputs.host_array(1, 2, (1 << 20,), 0.02, bf16=True).astype(np.float64)
    assert abs(a.mean()) < 1e-4 and abs(a.std() - 0.02) < 2e-4
    assert np.abs(a).max() <= 0.02 * 2 * np.sqrt(3) * 1.01
    bits = inputs.host_array(1, 2, (4096,), 0.02, bf16=True).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    b = inputs.host_array(1, 3, (1 << 16,), 1.0, mean=1.0)
    assert abs(b.mean() - 1.0) < 0.02


def test_distinct_tensors_are_uncorrelated():
    a = inputs.host_array(7, 100, (1 << 16,), 1.0)
    b = inputs.host_array(7, 101, (1 << 16,), 1.0)
    c = inputs.host_array(8, 100, (1 << 16,), 1.0)
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.02 and abs(np.corrcoef(a, c)[0, 1]) < 0.02
    assert torch.tensor(0).item() == 0
