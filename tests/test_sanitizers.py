"""Host-side sanitizer runs, on the CPU.

  * The oracle pin suite (and the codec pins) against the oracle built with
    gcc's AddressSanitizer + UndefinedBehaviorSanitizer.
  * The C-ABI argument checks (tests/test_abi.py) against the attention
    library built with the same sanitizers on its host code.
Both run in a child process with the sanitizer runtime preloaded, and any
report fails them (halt_on_error; recovery off).  A planted slip in a copy of
the oracle (its score buffer allocated one query row short) shows that the
oracle build does report a heap overflow, and the library build is checked
for the sanitizer's instrumentation.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from tests.sanitize import build as sb

ROOT = sb.ROOT
ASAN = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
UBSAN = "halt_on_error=1:print_stacktrace=1"
# (the child pytest runs with -s, so that a report is not swallowed by its
# output capture when the sanitizer ends the process)


def child(args, env_extra, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def reports(r):
    return "AddressSanitizer" in r.stderr or "runtime error" in r.stderr


def why(r):
    """The report lines first, then the tails of the child's output."""
    keys = ("runtime error", "ERROR: AddressSanitizer", "SUMMARY:")
    lines = [ln for ln in r.stderr.splitlines() if any(k in ln for k in keys)]
    return "\n".join(lines[:12]) + "\n--- stdout tail:\n" + r.stdout[-1500:] + "\n--- stderr tail:\n" + r.stderr[-1500:]


@pytest.fixture(scope="module")
def oracle_env():
    lib = sb.build_oracle()
    return {"LD_PRELOAD": sb.runtime_preload("gcc"), "ASAN_OPTIONS": ASAN, "UBSAN_OPTIONS": UBSAN,
            "ZL_ORACLE_LIBRARY": lib}


def test_oracle_pins_under_asan_and_ubsan(oracle_env):
    r = child(["-c", "import oracle; print(oracle._load()._name)"], oracle_env)
    assert r.returncode == 0 and r.stdout.strip() == sb.ORACLE_LIB, r.stderr[-2000:]
    r = child(["-m", "pytest", "tests/test_oracle_pins.py", "tests/test_oracle_codec.py", "-x", "-q", "-s",
               "-p", "no:cacheprovider"], oracle_env)
    assert r.returncode == 0 and not reports(r), why(r)


def test_planted_overflow_in_the_oracle_is_reported(oracle_env, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "zl_oracle.c")).read()
    old = "malloc(sizeof(double) * ((size_t)max_len + (size_t)dk))"
    assert old in src
    planted = tmp_path / "zl_oracle_planted.c"
    planted.write_text(src.replace(old, "malloc(sizeof(double) * ((size_t)max_len))", 1))
    lib = sb.build_oracle(str(planted), str(tmp_path / "liboracle_planted.so"))
    code = ("import numpy as np, oracle\n"
            "rng = np.random.default_rng(0)\n"
            "q = rng.integers(0, 0x3c00, (2, 4, 64), dtype=np.uint16)\n"
            "k = rng.integers(0, 0x3c00, (40, 1, 64), dtype=np.uint16)\n"
            "cu = np.array([0, 7, 40], dtype=np.int32)\n"
            "oracle.gqa_decode(q, k, k, cu, 1, 0.125, oracle.F16)\n")
    r = child(["-c", code], dict(oracle_env, ZL_ORACLE_LIBRARY=lib), timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_abi_checks_under_asan_and_ubsan():
    lib = sb.build_library()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host code is not instrumented"
    env = {"LD_PRELOAD": sb.runtime_preload("clang"), "ASAN_OPTIONS": ASAN, "UBSAN_OPTIONS": UBSAN,
           "ZL_ATTN_LIBRARY": lib}
    r = child(["-c", "import mla_attention_amd as z; z.library(); print(z.LIB_PATH)"], env)
    assert r.returncode == 0 and r.stdout.strip().endswith(os.path.basename(lib)), r.stderr[-2000:]
    r = child(["-m", "pytest", "tests/test_abi.py", "-x", "-q", "-s", "-p", "no:cacheprovider"], env)
    assert r.returncode == 0 and not reports(r), why(r)
