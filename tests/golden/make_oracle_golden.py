"""Write the CPU oracle's velocity for the full-size workloads.

    python tests/golden/make_oracle_golden.py [--f16] [512 1024 cond cfg512 ...]

Calls only the oracle (``oracle/``) and the seeded input generator
(``inputs/``): the stored values never come from the GPU path.  For each
workload the prefix is prefilled and one step is taken, exactly as the
GPU parity test does; every ``stride``-th target row of v is stored
(float32 .npy) with the row stride in the file name.  ``--f16`` runs the
oracle's ``storage="f16"`` mode (every activation the device design keeps
in float16 rounded to it) and stores ``..._f16_rows{stride}.npy``: the
error that storage alone costs, against which the device's single-f16
path is bounded.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from inputs import CONFIGS  # noqa: E402
from oracle import SynthModel, workload_inputs  # noqa: E402
from oracle import qi21_oracle as O  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
STRIDE = {"512": 1, "1024": 1, "cond": 4, "cfg512": 2, "2048": 16, "ragged": 4}


def golden_path(name: str, prefix: int = 0, storage=None) -> str:
    tag = "_f16" if storage == "f16" else ""
    return os.path.join(HERE, f"oracle_v_{name}_p{prefix}{tag}_rows{STRIDE[name]}.npy")


def make(name: str, storage=None) -> None:
    w = CONFIGS[name]
    model = SynthModel(w.model)
    for p in range(len(w.prefixes)):
        t0 = time.time()
        d = workload_inputs(w, p)
        lay = O.Layout(w.layout(p))
        pre = O.prefill(model, d["x_prefix"], lay, storage=storage)
        t1 = time.time()
        v = O.step(model, pre, d["tok"], d["mods"], d["final_scale"], storage=storage)
        np.save(golden_path(name, p, storage), np.ascontiguousarray(v[::STRIDE[name]]).astype(np.float32))
        print(f"{name} prefix {p} storage {storage}: prefill {t1 - t0:.0f} s, step {time.time() - t1:.0f} s, "
              f"|v| rms {float(np.sqrt((v.astype(np.float64) ** 2).mean())):.4f}", flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    st = "f16" if "--f16" in args else None
    names = [a for a in args if a != "--f16"]
    for n in names or ["512", "1024", "cond", "cfg512"]:
        make(n, st)
