"""Build libxattn.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Run as ``python -m block_sparse_attention_strided_amd.build``; the library is
written next to this file so that it travels with the source tree.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/estimate.hip", "csrc/select.hip", "csrc/attention.hip", "csrc/abi.cpp", "csrc/prefill_static.hip"]
LIB = os.path.join(HERE, "libxattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-ffp-contract=fast",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + os.path.join(HERE, "csrc"),
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(HERE, src), "-o", obj] + FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs + [
        "-L" + os.path.join(ROCM, "lib"), "-lrocprofiler-sdk-roctx", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
