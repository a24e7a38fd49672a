"""Compile libtq.so (the HIP kernels and the C ABI) in-tree for gfx950.

``python -m ternary_quantized_amd.build`` builds the library next to this
file; every call recompiles.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
BUILD = os.path.join(HERE, "_build")

HIP_SOURCES = ["tq_hadamard.hip", "tq_gemv.hip", "tq_gemv_quads.hip", "tq_gemm.hip",
               "tq_transcode.hip", "tq_q2g64.hip", "tq_head.hip", "tq_measure.hip",
               "tq_gemv_f4.hip"]
HOST_SOURCES = ["tq_host.cpp", "tq_container.cpp"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError("build failed:\n%s\n%s" % (" ".join(cmd), proc.stdout))
    return proc.stdout


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c",
                     os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    outs.append(_run(link))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


# The host-only build: the C ABI's host sources (validation, geometry, host
# packer, container parser) under AddressSanitizer and
# UndefinedBehaviorSanitizer, linked with tq_host_only.cpp in place of the
# kernels.  It needs no GPU; the CPU tests run against it with
#   TQ_LIBRARY=<this .so> LD_PRELOAD="<libasan.so> <libubsan.so>"
#   ASAN_OPTIONS=detect_leaks=0 python -m pytest tests -m "not gpu"
SANITIZE_LIB = os.path.join(BUILD, "libtq_host_sanitize.so")
SANITIZE_SOURCES = ["tq_host.cpp", "tq_container.cpp", "tq_host_only.cpp"]


def build_sanitize():
    os.makedirs(BUILD, exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fPIC", "-shared", "-Wall",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(rocm, "include"),
           *[os.path.join(CSRC, f) for f in SANITIZE_SOURCES],
           "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-o", SANITIZE_LIB]
    _run(cmd)
    return SANITIZE_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitize())
    else:
        print(build(verbose="-v" in sys.argv))
