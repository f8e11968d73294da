"""Build liblinattn.so (the C-ABI library) from csrc/ with hipcc for gfx950.

Usage:  python -m weight_sequence_mixing_amd.build   (or build() from Python)

The library is linked against the HIP runtime that PyTorch ships
(torch/lib/libamdhip64.so), so that a process that has imported torch holds a
single HIP runtime and torch's device pointers and streams are valid in the
library.  Objects are compiled in parallel into _build/ next to this file; the
shared library is written next to this file.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblinattn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

SOURCES = [
    "la_inst_bf16_elu.hip",
    "la_inst_bf16_rf.hip",
    "la_inst_f32.hip",
    "la_inst_bf16_relu.hip",
    "la_inst_f32_relu.hip",
    "la_inst_bwd_bf16.hip",
    "la_inst_bwd_f32.hip",
    "la_scan.hip",
    "la_inst_ident_bf16.hip",
    "la_inst_ident_f32.hip",
    "la_rf_grad.hip",
    "la_scratch.hip",
    "la_api.cpp",
]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the kernels scale and mask
    # them with vector ALU code, which cannot read AGPRs directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def torch_lib_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("PyTorch is required: the library links torch's HIP runtime")
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), out))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link liblinattn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tl = torch_lib_dir()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [CLANG, "-shared", "-fPIC", "-o", tmp] + objs + [
        "-L" + tl, "-l:libamdhip64.so", "-Wl,-rpath," + tl, "-Wl,--no-undefined", "-lstdc++", "-lm"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), r.stdout))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
