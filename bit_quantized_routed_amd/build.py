"""Build libmoe.so (hipcc, gfx950) in-tree.

    python -m bit_quantized_routed_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libmoe.so")

HIP_SOURCES = ["route.hip", "ffn.hip", "prefill.hip", "decode.hip", "cache.hip", "probe.hip", "api.hip"]
# plain host C++ (the quantizer); built at -O2 as C++: clang's -O3 loop
# optimisation of the codebook search does not terminate in reasonable time
HOST_SOURCES = ["pack.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


CXX = os.environ.get("MOE_CXX", "/opt/rocm/llvm/bin/clang++")
HOST_FLAGS = ["-x", "c++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
              "-I" + os.path.join(ROOT, "include")]
_NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    out = "\n".join(l for l in r.stdout.splitlines() if _NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".host.o")
        jobs.append(([CXX] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        jobs.append(([HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    # one compiler process per source, a few at a time
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1), 8))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    objs = [o for _, o in jobs]
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp, "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
