"""The stored full-size oracle outputs, ``tests/golden/oracle_v_*.npy``
(written by ``tests/golden/make_oracle_golden.py`` from the oracle alone).

Each file's name gives the workload, the prefix (program) index, the
storage mode and the row stride; its content must be that workload's
target rows at that stride by the 64 output channels, finite, and at the
scale the velocity has on these inputs (rms about 1.3 for every
workload).  This catches a file written for another workload, cut short
or damaged before a GPU test trusts it.
"""
import glob
import os
import re

import numpy as np
import pytest

from inputs import CONFIGS
from oracle import qi21_oracle as O

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FILES = sorted(glob.glob(os.path.join(GOLD, "oracle_v_*.npy")))


def test_the_full_size_workloads_have_stored_outputs():
    names = {re.match(r"oracle_v_(\w+?)_p\d", os.path.basename(f)).group(1) for f in FILES}
    assert {"512", "1024", "2048", "cond", "ragged", "cfg512"} <= names, names


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(f) for f in FILES])
def test_stored_output_matches_its_name(path):
    m = re.match(r"oracle_v_(\w+?)_p(\d+)(_f16)?_rows(\d+)\.npy$", os.path.basename(path))
    assert m, path
    name, prefix, stride = m.group(1), int(m.group(2)), int(m.group(4))
    w = CONFIGS[name]
    n = O.Layout(w.layout(prefix)).target_len
    v = np.load(path)  # no pickles: numpy's own format only
    assert v.dtype == np.float32
    assert v.shape == (-(-n // stride), 64), (v.shape, n, stride)  # 64 latent channels
    assert np.all(np.isfinite(v))
    rms = float(np.sqrt((v.astype(np.float64) ** 2).mean()))
    assert 0.8 < rms < 2.0, rms
