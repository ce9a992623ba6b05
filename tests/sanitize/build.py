"""Host-side sanitizer builds, for the CPU test suite (tests/test_sanitizers.py).

  * the fp64 oracle (oracle/zl_oracle.c) with gcc's AddressSanitizer and
    UndefinedBehaviorSanitizer;
  * the attention library (mla_attention_amd/csrc) with the same two
    sanitizers on its HOST code only: every hipcc line puts -Xarch_host before
    each -fsanitize=, so the gfx950 device code is compiled as usual.  No GPU
    is involved: the tests that use it (the C-ABI argument checks) return
    before any HIP call.

A shared library built this way needs the sanitizer runtime preloaded into
the Python process that loads it: runtime_preload() names it.  Outputs go to
tests/sanitize/_build/.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "_build")
CSRC = os.path.join(ROOT, "mla_attention_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

ORACLE_LIB = os.path.join(OUT, "liboracle_asan.so")
ZL_LIB = os.path.join(OUT, "libzl_attn_asan.so")

GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build_oracle(src: str = os.path.join(ROOT, "oracle", "zl_oracle.c"), out: str = ORACLE_LIB) -> str:
    """gcc build of an oracle source with ASan + UBSan (OpenMP kept)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-O1", "-g", *GCC_SAN, "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_library(out: str = ZL_LIB) -> str:
    """hipcc build of the whole library, sanitizers on the host code only."""
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "zl_api.cpp")]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, *HOST_SAN]

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        subprocess.run([HIPCC, *common, "-c", src, "-o", obj], check=True, stderr=subprocess.DEVNULL)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, *objs, "-o", out + ".tmp"],
                   check=True)
    os.replace(out + ".tmp", out)
    return out


def runtime_preload(kind: str) -> str:
    """LD_PRELOAD value for a library built by gcc ('gcc') or by hipcc ('clang')."""
    if kind == "gcc":
        libs = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                               check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
        return ":".join(libs)
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("clang AddressSanitizer runtime not found under /opt/rocm/llvm")
    return found[-1]


if __name__ == "__main__":
    print(build_oracle())
    print(build_library())
