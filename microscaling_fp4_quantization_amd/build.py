"""Build libfp4q.so (HIP kernels for gfx950 plus the C ABI) in-tree.

    python -m microscaling_fp4_quantization_amd.build

Kernels are compiled with hipcc for gfx950 only; the ABI layer is plain host
C++.  Flags that matter for the arithmetic:
  -ffp-contract=off      no fusing of a*b+c: every binary32 operation is the
                         one written (explicit fmaf() where fusion is meant)
  -fno-gpu-flush-denormals-to-zero, no fast-math: IEEE binary32 and binary64
                         with subnormals and correctly rounded division
  -target-feature -packed-fp32-ops: no packed-FP32 instructions
The GEMM source also takes -amdgpu-mfma-vgpr-form: matrix-core accumulators
in ordinary VGPRs, which keeps them in place across the K loop.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfp4q.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
FILE_FLAGS = {"fp4q_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = [ln for ln in r.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libfp4q.so; returns its path."""
    tmp = tempfile.mkdtemp(prefix="fp4q_build_")
    try:
        sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
        objs, jobs = [], []
        for f in sources:
            o = os.path.join(tmp, f[:-4] + ".o")
            objs.append(o)
            jobs.append([HIPCC, *HIP_FLAGS, *FILE_FLAGS.get(f, []), "-c", os.path.join(CSRC, f), "-o", o])
        a_obj = os.path.join(tmp, "fp4q_abi.o")
        objs.append(a_obj)
        jobs.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "fp4q_abi.cpp"), "-o", a_obj])
        with ThreadPoolExecutor(len(jobs)) as ex:
            list(ex.map(_run, jobs))
        tmp_out = out + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_out, *objs])
        os.replace(tmp_out, out)
        if verbose:
            print("built", out)
        return out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
