"""Build libzl_attn.so (gfx950 HIP kernels + C ABI) in-tree with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzl_attn.so")
SOURCES = ["decode_attn.hip", "decode_mla.hip", "split_merge.hip", "attn_combine.hip", "int8_codec.hip", "prefill_attn.hip",
           "hbm_read.hip", "no_alloc.hip", "zl_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler away from packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    # MFMA accumulators in ordinary VGPRs (no AGPR round trips for the
    # per-tile softmax rescale)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source (one hipcc per file, in parallel) and link
    them into mla_attention_amd/libzl_attn.so."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    incs = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [HIPCC, *compile_flags, *incs, "-c", os.path.join(CSRC, s), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: _run(j[1], verbose), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
