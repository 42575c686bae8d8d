"""Build the gfx950 shared library ``libkairos.so`` in-tree with hipcc.

Usage: ``python -m video_world_model_chunkwise_amd.build`` (always rebuilds).
Sources: ``csrc/*.hip`` (kernels and the C ABI of ``include/kairos.h``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkairos.so")
ARCH = "gfx950"

SOURCES = ["gdn.hip", "window_attn.hip", "operands.hip", "ring.hip", "prologue.hip", "gates_check.hip",
           "kairos_abi.hip"]

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]

# per-source options: the gated delta rule keeps every MFMA result in
# architectural VGPRs (its chained products feed VALU work directly)
EXTRA = {
    "gdn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


# host-only sanitizers (the device code is built as usual): AddressSanitizer
# and UndefinedBehaviorSanitizer on the C ABI's validation and launch code
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime the sanitized library needs
    preloaded (it must be the process's first ASan-aware library)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/lib/llvm")
    return hits[-1]


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    hipcc = _hipcc()
    extra_flags = SANITIZE if sanitize else []
    with tempfile.TemporaryDirectory(prefix="kairos_build_") as tmp:
        objs = []
        jobs = []
        with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
            for src in SOURCES:
                obj = os.path.join(tmp, src.replace(".hip", ".o"))
                objs.append(obj)
                cmd = [hipcc, *CFLAGS, *extra_flags, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
                jobs.append(ex.submit(_run, cmd))
            for j in jobs:
                o = j.result()
                if verbose and o.strip():
                    print(o)
        tmp_lib = out + ".tmp"
        _run([hipcc, "-shared", f"--offload-arch={ARCH}", *extra_flags, *objs, "-o", tmp_lib])
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
