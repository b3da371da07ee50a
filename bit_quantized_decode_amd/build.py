"""Build libnvfp4.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Run as `python -m bit_quantized_decode_amd.build` or call build().  The
library is written next to this file so that it travels with the source tree.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libnvfp4.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["pack.hip", "quantize.hip", "gemv.hip", "skinny.hip", "prefill.hip", "moe.hip", "w4a4.hip", "abi.cpp"]
# The benchmark's ceiling probes: a library of their own, not part of the product.
PROBES_SRC = "probes.hip"
PROBES_LIB = os.path.join(HERE, "libnvfp4_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # No packed-fp32 VALU instructions anywhere in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src):
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, 6)) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBES_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBES_LIB)
    if verbose:
        print(f"built {LIB} and {PROBES_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
