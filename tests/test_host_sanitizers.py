"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The float64 oracle (oracle/etp_oracle.c) is rebuilt with
   -fsanitize=address,undefined and the oracle's pin tests run against that
   build in a child process (ORACLE_LIB points the wrapper at it; the ASan
   runtime is preloaded into the interpreter, leak checks off, any report
   aborts the child).
2. The library's plan-table code (csrc/etp_tables.hpp) is evaluated at run
   time in a sanitized g++ build of tests/sanitize_tables.cpp and compared
   field by field with the compile-time table the kernels use.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _gcc_lib(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", *SAN, "-std=c11", "-fopenmp", "-shared", "-fPIC",
                           os.path.join(ROOT, "oracle", "etp_oracle.c"), "-o", lib, "-lm"])
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=_gcc_lib("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_sh_cg.py", "test_oracle_conv.py", "test_oracle_radial.py", "test_oracle_edge_tp.py",
              "test_oracle_forces.py", "test_oracle_mix.py", "test_oracle_neighbors.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


def test_plan_tables_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_tables")
    subprocess.check_call(["g++", *SAN, "-std=c++20", "-fconstexpr-ops-limit=4000000000",
                           "-fconstexpr-loop-limit=100000000",
                           "-I", os.path.join(ROOT, "equivariant_interatomic_potentials_amd", "csrc"),
                           os.path.join(ROOT, "tests", "sanitize_tables.cpp"), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("mismatches=0") == 5, r.stdout
