"""Build liblvq.so in-tree: hipcc for the gfx950 kernels, g++ for the host expander.

    python dequant_gemv_lvq_amd/build.py        # or __graft_entry__.build()

(Run it as a file: importing it through the package would first load the
library it is about to build.)

Objects go to dequant_gemv_lvq_amd/_build/, the library to
dequant_gemv_lvq_amd/liblvq.so.  Every call recompiles.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblvq.so")
ARCH = os.environ.get("LVQ_OFFLOAD_ARCH", "gfx950")

HIP_SOURCES = ["lvq_gemv.hip", "fp16_gemv.hip", "bpdq_gemv.hip", "trellis_gemv.hip",
               "rotate.hip", "unfold.hip", "measure.hip"]
HOST_SOURCES = ["expand.cpp", "index.cpp"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # packed fp32 VALU forms stay off (plain fp32 ops only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall"]


def _hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return cand


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), p.stdout))
    return p.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    hipcc = _hipcc()
    cxx = shutil.which("g++") or "g++"
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, src.replace(".hip", ".o"))
        jobs.append([hipcc] + HIPCC_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, src.replace(".cpp", ".o"))
        jobs.append([cxx] + CXX_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        logs = list(ex.map(_run, jobs))
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
