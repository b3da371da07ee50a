"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code, on
the CPU: the oracle (every function, small inputs in exactly sized buffers)
and the C ABI (every entry point, with arguments it must refuse before any
launch, and the host-only calls).  The library's HIP sources are compiled in
full, with the sanitizers on their host side only (-Xarch_host)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "bit_quantized_decode_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)} failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11", "-g", "-O1", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-o", exe, "-lm"])
    r = run([exe], env=ENV)
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    import torch
    if torch.cuda.device_count() != 0:
        pytest.skip("a GPU is visible: the driver's placeholder pointers are for a machine without one")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    srcs = [os.path.join(CSRC, f) for f in ("pack.hip", "quantize.hip", "gemv.hip", "skinny.hip", "prefill.hip",
                                            "moe.hip", "w4a4.hip", "abi.cpp")]
    srcs.append(os.path.join(HERE, "abi_driver.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        run([HIPCC, *flags, "-c", src, "-o", obj])
        return obj
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_driver")
    run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         *objs, "-o", exe])
    r = run([exe], env=ENV)
    assert r.stdout.strip().endswith("ok"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
