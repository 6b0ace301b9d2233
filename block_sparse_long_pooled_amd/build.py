"""Build libflashprefill.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m block_sparse_long_pooled_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "pool.hip", "select.hip", "attn.hip", "meancorr.hip"]
LIB_NAME = "libflashprefill.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
PEAKS_PATH = os.path.join(HERE, "libfppeaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU ops are switched off: ordinary float code must not be
# vectorised into v_pk_{add,mul,fma}_f32.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = COMMON_FLAGS + list(extra_flags)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        out = _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    # the peak microbenchmarks bench.py measures against (not part of the ABI)
    peaks_tmp = PEAKS_PATH + ".tmp"
    _run([HIPCC, *flags, "-shared", os.path.join(CSRC, "peaks.hip"), "-o", peaks_tmp])
    os.replace(peaks_tmp, PEAKS_PATH)
    if verbose:
        print(f"built {PEAKS_PATH}")
    # a stand-alone C++ consumer of the C ABI (run by the GPU tests)
    capi_src = os.path.join(ROOT, "tests", "capi", "capi_check.cpp")
    if os.path.exists(capi_src):
        capi_bin = os.path.join(ROOT, "tests", "capi", "capi_check")
        _run([HIPCC, f"--offload-arch={ARCH}", "-O2", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}",
              capi_src, "-o", capi_bin + ".tmp", f"-L{HERE}", "-lflashprefill", f"-Wl,-rpath,{HERE}",
              "-Wl,-rpath,$ORIGIN/../../block_sparse_long_pooled_amd"])
        os.replace(capi_bin + ".tmp", capi_bin)
        if verbose:
            print(f"built {capi_bin}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
