"""Build libtq.so (HIP, gfx950) in the package directory.

    python -m vector_quantization_tq_amd.build

Runs hipcc once over all sources: host C++ (precompute), the C ABI and the
kernels.  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
SOURCES = ["tq_host.cpp", "tq_api.hip", "tq_encode.hip", "tq_scores.hip", "tq_attend.hip", "tq_topk.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def hipcc_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
            # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix-core accumulators in ordinary VGPRs: the kernels scale and
            # read them with vector ALU ops, which cannot address AGPRs
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def build(verbose: bool = False) -> str:
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        srcs += (["-x", "hip", p] if s.endswith(".hip") else ["-x", "c++", p])
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + hipcc_flags() + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l and "ignoring feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
