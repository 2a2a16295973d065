"""The 16 x 16 x 32 GEMM kernel's main loops as compiled for gfx950.

The register allocator keeps the kernel's 256 accumulators in AGPRs, where
the MFMAs read and write them, only for some instruction orders and with the
kernel's AGPR pin at each loop head.  A change that makes it give the
loop-carried accumulators VGPR homes (copying all of them every iteration)
or spill costs much of the kernel's speed without changing any result, so
no parity test would notice.  This compiles gemm.hip to assembly (no GPU
needed) and checks every instance of the kernel.
"""
import collections
import os
import re
import subprocess

import pytest

from diffusion_transformer_denoiser_qi21_amd import build as B


def _kernels(asm: str, pattern: str):
    """(name, body lines, metadata text) of each kernel whose symbol holds pattern."""
    lines = asm.split("\n")
    for i, l in enumerate(lines):
        if re.match(r"^_Z\w*:", l) and pattern in l:
            e = i
            while "s_endpgm" not in lines[e]:
                e += 1
            yield l.split(":")[0], lines[i:e + 1], "\n".join(lines[e:e + 400])


def _loops(body):
    """Instruction counts of each loop: from a label marked as a loop header
    to the last branch back to it."""
    out = []
    for i, l in enumerate(body):
        m = re.match(r"^(\.LBB\w+):", l)
        if not (m and any("Loop Header" in x for x in body[i:i + 3])):
            continue
        lab = re.escape(m.group(1))
        back = [j for j, x in enumerate(body) if re.search(r"s_c?branch\w*\s+" + lab + r"\s*$", x)]
        if back:
            ops = [x.split()[0] for x in body[i:max(back) + 1]
                   if x.strip() and not x.strip().startswith(";") and not x.startswith(".")]
            out.append(collections.Counter(ops))
    return out


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    flags = [f for f in B.FLAGS if f not in ("-fPIC", "-Werror")]
    cmd = [B._hipcc()] + flags + ["--cuda-device-only", "-S", "-o", str(out), os.path.join(B.CSRC, "gemm.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_gemm16_main_loops_keep_accumulators_in_agprs(gemm_asm):
    seen = 0
    for name, body, meta in _kernels(gemm_asm, "gemm16_kernel"):
        seen += 1
        scratch = re.search(r";\s*ScratchSize:\s*(\d+)", meta)
        assert scratch and int(scratch.group(1)) == 0, f"{name} spills"
        loops = _loops(body)
        mfma_loops = [c for c in loops if sum(v for k, v in c.items() if "mfma" in k) > 0]
        assert mfma_loops, f"{name}: no main loop found"
        for c in mfma_loops:
            moves = sum(v for k, v in c.items() if k.startswith("v_accvgpr"))
            assert moves == 0, f"{name}: {moves} accumulator copies in the main loop"
    # the f16 forms of every epilogue but the 8-wave lo8 SwiGLU, and the lo4
    # forms of the FFN sites
    assert seen >= 12, seen
