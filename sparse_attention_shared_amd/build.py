"""Build libcsa2.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

The library links against the HIP runtime that PyTorch ships (same soname as
the system one, found through an rpath to torch's lib directory) so that the
streams and device memory torch hands over belong to the runtime the kernels
run on.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libcsa2.so")

SOURCES = ["k_fp4.hip", "k_score.hip", "k_topk.hip", "k_prefill.hip", "k_attn.hip", "csa2_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions stay off: hipcc must not emit v_pk_{add,mul,fma}_f32.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + INCLUDE, "-I" + CSRC]


def _torch_lib_dir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("torch is required to locate its HIP runtime")
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


# Per-file code generation options: these kernels keep their MFMA accumulators
# in ordinary VGPRs, so reading a result costs no v_accvgpr_read.
FILE_FLAGS = {"k_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + FILE_FLAGS.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                         "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tl = _torch_lib_dir()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + [
        "-L" + tl, "-Wl,-rpath," + tl, "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
