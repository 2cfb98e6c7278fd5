"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer.

Every library source is compiled with both sanitizers on its host code (the device code
is built as usual but never launched) and linked with ``tests/native/abi_sanitize_check.cpp``,
which calls every entry point of ``include/nvfp4.h`` with arguments that fail validation
(null, misaligned and out-of-range values, bad shapes, short workspaces), with empty
problems, and the host-only queries (plans, workspace sizes, status strings) over a fuzz
of extreme shapes. No call reaches a kernel launch; the pointers are host addresses that
the library never dereferences. The sanitizers abort on any finding (overflow in a size
check, an out-of-bounds host access), and the program checks each call's status.

The test needs no GPU and refuses to run where one is visible.
"""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_02_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "abi_sanitize_check.cpp")
# host-only sanitizer flags (device code is not instrumented)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _gpu_visible() -> bool:
    return os.path.exists("/dev/kfd")


@pytest.mark.skipif(_gpu_visible(), reason="host-only check: a visible GPU could take real launches")
def test_abi_validation_under_sanitizers(tmp_path):
    from nvfp4_block_scaled_02_amd import build as B

    flags = [f for f in B.compile_flags() if f != "-O3"]
    hipcc = B.hipcc()

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [hipcc, *flags, *SAN]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        r = subprocess.run(cmd + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = [os.path.join(CSRC, s) for s in B.SOURCES] + [SRC]
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_sanitize_check")
    r = subprocess.run([hipcc, *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("checks ")]
    assert line and line[-1].endswith("failures 0"), r.stdout
    assert int(line[-1].split()[1]) > 10000
