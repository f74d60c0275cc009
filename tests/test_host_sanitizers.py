"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed).

The library sources are compiled with the library's own flags plus both
sanitizers on the host pass only (device code is built as usual and never
run) and linked into tests/abi_host_check.cpp, which
calls every entry point with each class of invalid argument (null, shape,
extent, alignment, alpha, ldo, workspace, row limits), the workspace queries
at the extreme accepted shapes (s up to 2^31 - 1, h up to I8MM_MAX_H) and
the status strings. Any out-of-bounds access, signed overflow or other
undefined behaviour on these paths aborts the run.
"""

import os
import shlex
import subprocess
from concurrent.futures import ThreadPoolExecutor

from int8_quantized_matmul_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_host_check.cpp")

# host pass only: -Xarch_host precedes each sanitizer option
SANITIZE = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=undefined -fno-omit-frame-pointer")


def test_abi_validation_under_host_sanitizers(tmp_path):
    hipcc = build._hipcc()
    flags = [*build.HIP_FLAGS, "-Wextra", "-Werror", "-g", *SANITIZE]

    def compile_one(src):
        path = src if os.path.isabs(src) else os.path.join(build.CSRC, src)
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        res = subprocess.run([hipcc, *flags, "-x", "hip", "-c", path, "-o", obj], capture_output=True, text=True)
        assert res.returncode == 0, res.stdout + res.stderr
        return obj

    with ThreadPoolExecutor(max_workers=len(build.SOURCES) + 1) as ex:
        objs = list(ex.map(compile_one, build.SOURCES + [DRIVER]))
    exe = str(tmp_path / "abi_host_check")
    res = subprocess.run([hipcc, "--offload-arch=gfx950", *SANITIZE, *objs, "-o", exe], capture_output=True,
                         text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "0 failed" in res.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
