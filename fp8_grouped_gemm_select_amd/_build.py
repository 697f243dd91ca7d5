"""Builds libmoe.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")

SOURCES = ["abi.hip", "select_experts.hip", "router.hip", "pre_reorder.hip", "grouped_gemm.hip",
           "act_requant.hip", "post_reorder.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


# the benchmark's on-box ceilings (streaming copy / read, FP8 MFMA loop): a
# library of their own, outside the layer's ABI
CEIL_SOURCES = ["ceilings.hip"]
CEIL_LIB = os.path.join(HERE, "libmoe_ceilings.so")
# the tests' device evaluation of the library's fixed-sequence math, likewise
PROBE_SOURCES = ["probe_math.hip"]
PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEIL_SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEIL_SOURCES], CEIL_LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
