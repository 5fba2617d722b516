"""The host side of the C-ABI library under AddressSanitizer and
UndefinedBehaviorSanitizer.

The library's sources are built a second time, the device code exactly as in
the product build and the host code instrumented (``-Xarch_host
-fsanitize=...``), and tests/test_abi_cpu.py runs again against that copy in a
child interpreter with the sanitizer runtime preloaded.  Every argument check,
workspace-size query and launch-plan computation those tests reach then runs
under the sanitizers; a report aborts the child and fails this test.  Needs
no GPU: nothing is launched."""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from selective_state_space_84_amd import build_lib

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(_runtime() is None or not os.path.exists(build_lib.HIPCC),
                    reason="hipcc or the clang sanitizer runtime is missing")
def test_abi_validation_clean_under_sanitizers(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        r = subprocess.run([build_lib.HIPCC, *build_lib.FLAGS, *SAN, "-c", os.path.join(build_lib.CSRC, src),
                            "-o", obj], capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, src + "\n" + r.stdout[-2000:] + r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, build_lib.SOURCES))
    lib = str(tmp_path / "libssm_scan_sanitized.so")
    subprocess.run([build_lib.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-shared-libsan",
                    "-o", lib, *objs], check=True, capture_output=True, timeout=300)
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, SSM_TEST_LIBRARY=lib, LD_PRELOAD=(_runtime() + (" " + pre if pre else "")),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(REPO, "tests", "test_abi_cpu.py")],
                       capture_output=True, text=True, timeout=600, env=env, cwd=REPO)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
