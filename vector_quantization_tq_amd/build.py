"""Build libtq.so (HIP, gfx950) in the package directory.

    python -m vector_quantization_tq_amd.build [--define NAME ...] [--out DIR]

Compiles every source to an object with hipcc (in parallel, objects under
_build/ next to this file), then links them into libtq.so.  Always
recompiles.  --define adds a preprocessor macro and --out puts the libraries
(and objects) in DIR instead: a variant for A/B measurements, loaded by
setting TQ_LIBRARY=DIR/libtq.so (TQ_NO_WHT_ENCODE: Hadamard-rotation values
and MSE-only keys on the dense +-1 matrix-core encoder instead of the
Walsh-Hadamard butterflies).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtq.so")
SOURCES = ["tq_host.cpp", "tq_api.hip", "tq_encode.hip", "tq_scores.hip", "tq_attend.hip", "tq_attend_d64.hip",
           "tq_attend_d96.hip", "tq_attend_d256.hip", "tq_topk.hip"]
# the benchmark's streaming-ceiling kernel, in a library of its own
STREAM_LIB = os.path.join(HERE, "libtq_stream.so")
STREAM_SOURCES = ["tq_stream.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
NOISE = ("is not a recognized feature for this target", "ignoring feature")


def hipcc_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix-core accumulators in ordinary VGPRs: the kernels scale and
            # read them with vector ALU ops, which cannot address AGPRs
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if not any(n in l for n in NOISE))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, defines=(), out_dir: str | None = None) -> str:
    obj_dir = os.path.join(out_dir, "_build") if out_dir else OBJ
    lib_path = os.path.join(out_dir, "libtq.so") if out_dir else LIB
    stream_path = os.path.join(out_dir, "libtq_stream.so") if out_dir else STREAM_LIB
    os.makedirs(obj_dir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    jobs = []
    for s in SOURCES + STREAM_SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
        lang = "hip" if s.endswith(".hip") else "c++"
        jobs.append((s, obj, [HIPCC] + hipcc_flags() + extra + ["-c", "-x", lang, src, "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, cmd, verbose) for _, _, cmd in jobs]:
            f.result()
    for lib, srcs in ((lib_path, SOURCES), (stream_path, STREAM_SOURCES)):
        tmp = lib + ".tmp"
        objs = [o for s, o, _ in jobs if s in srcs]
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, lib)
    return lib_path


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--define", action="append", default=[], help="preprocessor macro (NAME or NAME=VALUE)")
    ap.add_argument("--out", default=None, help="directory for a variant build (default: in-tree)")
    a = ap.parse_args()
    print(build(verbose=True, defines=a.define, out_dir=a.out))
