"""The library's host logic under AddressSanitizer and UBSan (CPU only).

``tests/host_sanitize/host_checks.cpp`` drives the layout helpers, model
creation (including an allocator hook that refuses each request in turn),
the op entry points' refusals, the launch-shape choices and the per-thread
last error.  It is built here, together with the library's host sources
(``layout.cpp``, ``qi21_api.cpp``, ``tiles.cpp``) and stand-ins for the
device launchers, by ROCm's clang in host-only mode with
``-fsanitize=address,undefined`` and ``-Werror``, then run; any sanitizer
report or failed check fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_transformer_denoiser_qi21_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
OUT = os.path.join(ROOT, "_build", "host_sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

SOURCES = [os.path.join(CSRC, f) for f in ("layout.cpp", "qi21_api.cpp", "tiles.cpp")] + \
          [os.path.join(HERE, f) for f in ("launch_stubs.cpp", "host_checks.cpp")]
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-Wall", "-Wno-unused-function", "-Werror", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(not os.path.exists(CLANG) or shutil.which("ld") is None, reason="ROCm clang++ not found")
def test_host_logic_is_clean_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        rc, log = _run([CLANG] + FLAGS + ["-c", src, "-o", obj])
        assert rc == 0, f"compile {src}:\n{log}"
        objs.append(obj)
    exe = os.path.join(OUT, "host_checks")
    rc, log = _run([CLANG, "-fsanitize=address,undefined", "-o", exe] + objs +
                   ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
                    "-lpthread"])
    assert rc == 0, f"link:\n{log}"
    supp = os.path.join(OUT, "lsan.supp")
    with open(supp, "w") as f:  # the HIP runtime's own start-up allocations are not ours
        f.write("leak:libamdhip64\nleak:libhsa-runtime64\nleak:librocprofiler-register\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               LSAN_OPTIONS=f"suppressions={supp}", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, log = _run([exe], env=env, timeout=300)
    print(log)
    assert rc == 0, log
    assert "ERROR: AddressSanitizer" not in log and "runtime error" not in log
    assert "host checks:" in log
