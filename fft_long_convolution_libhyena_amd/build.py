"""Build libhyena.so (HIP, gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-FP32 instructions
disabled, into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhyena.so")
SOURCES = ["hyena_api.hip", "hyena_backward.hip", "hyena_operator.hip", "fourstep.hip", "fourstep_backward.hip", "implicit_filter.hip", "kernel_synthesis.hip", "inproj.hip", "outproj.hip", "conv2d.hip", "conv3d.hip", "partitioned.hip", "lds_path_a.hip", "lds_path_b.hip", "lds_path_c.hip",
           "lds_path_d.hip", "lds_backward_a.hip", "lds_backward_b.hip", "lds_backward_c.hip", "lds_backward_d.hip",
           "lds_backward_e.hip", "lds_backward_f.hip"]
HEADERS = ["fft_core.hpp", "kernels.hpp", "pair.hpp", "plan.hpp", "tables.hpp", "conv_nd.hpp", "lds_path.hpp", "fourstep.hpp", "backward.hpp",
           "lds_backward.hpp", "outproj.hpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libhyena")
    return path


def build(verbose: bool = False, jobs: int = 4, out: str = LIB, defines=()) -> str:
    """Compile every source to an object in parallel, then link libhyena.so
    (or `out`, with extra -D tuning defines)."""
    objdir = os.path.join(os.path.dirname(os.path.abspath(out)), "_build" + ("_" + "_".join(
        d.replace("=", "") for d in defines) if defines else ""))
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc(), *HIPCC_FLAGS, *["-D" + d for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        text = log.decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp,
           "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
