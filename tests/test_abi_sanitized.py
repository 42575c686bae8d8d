"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the library is rebuilt with both sanitizers on its host code only (device
code unchanged), and the host-only ABI tests (validation of every entry
point, workspace and ring sizing, descriptor checks, exported symbols) run
against it in a child process with the ASan runtime preloaded.  Any
out-of-bounds access, use after free or undefined behaviour in the
validation layer aborts the child.  Runs without a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_under_host_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from video_world_model_chunkwise_amd import build as B
    lib = B.build(out=str(tmp_path / "libkairos_asan.so"), sanitize=True)
    nm = shutil.which("nm")
    if nm:                                        # the host code really is instrumented
        syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_" in syms and "__ubsan_" in syms
    env = dict(os.environ)
    env["KAIROS_LIB"] = lib
    env["LD_PRELOAD"] = B.sanitizer_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""               # host-only: validation paths never launch
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, "ABI tests failed under the host sanitizers"
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
