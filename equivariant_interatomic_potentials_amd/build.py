"""Build libetp.so (HIP, gfx950) in-tree.

Each kernel source is compiled once per l_max (-DETP_L=0..4) so the
translation units compile in parallel; the objects are linked into
``equivariant_interatomic_potentials_amd/libetp.so``.

    python -m equivariant_interatomic_potentials_amd.build [--force] [-j N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libetp.so")
ARCH = os.environ.get("ETP_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    f"--offload-arch={ARCH}", "-std=c++20", "-O3", "-fPIC", "-fvisibility=hidden",
    "-fconstexpr-steps=100000000",
    # packed FP32 stays off: the kernels use plain scalar FMAs
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def units():
    """(source, object, extra flags) for every translation unit."""
    out = []
    for name in ("etp_api", "etp_sh", "etp_graph", "etp_mix", "etp_forces", "etp_neighbors", "etp_node_product"):
        out.append((os.path.join(CSRC, name + ".hip"), os.path.join(BUILD, name + ".o"), []))
    for L in range(5):
        out.append((os.path.join(CSRC, "etp_edge_tp.hip"), os.path.join(BUILD, f"etp_edge_tp_L{L}.o"),
                    [f"-DETP_L={L}"]))
    for name, modes in (("etp_dst", (0, 1, 2, 3)), ("etp_src", (0, 1, 2, 3, 4, 5)), ("etp_bwd", (0, 1))):
        for L in range(5):
            for xt in (0, 1):
                for mode in modes:
                    out.append((os.path.join(CSRC, name + ".hip"),
                                os.path.join(BUILD, f"{name}_L{L}_X{xt}_M{mode}.o"),
                                [f"-DETP_L={L}", f"-DETP_XT={xt}", f"-DETP_MODE={mode}"]))
    return out


_INCLUDE = re.compile(r'^\s*#\s*include\s+"([^"]+)"', re.M)


def _deps(path, seen=None):
    """The file and every quoted header it includes, recursively."""
    seen = set() if seen is None else seen
    path = os.path.normpath(path)
    if path in seen or not os.path.exists(path):
        return seen
    seen.add(path)
    with open(path) as f:
        text = f.read()
    for inc in _INCLUDE.findall(text):
        _deps(os.path.join(os.path.dirname(path), inc), seen)
    return seen


def _stale(src, obj):
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(t < os.path.getmtime(d) for d in _deps(src))


def _compile(job):
    src, obj, extra = job
    t0 = time.time()
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(obj + ".tmp", obj)
    return obj, time.time() - t0


def build(force: bool = False, jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    todo = [u for u in units() if force or _stale(u[0], u[1])]
    # biggest units first so the slowest ones start early
    todo.sort(key=lambda u: ("_L4" not in u[1], "_L3" not in u[1]))
    if jobs is None:
        jobs = max(1, min(len(todo) or 1, os.cpu_count() or 1, 16))
    t0 = time.time()
    if todo:
        with cf.ThreadPoolExecutor(jobs) as ex:
            for obj, dt in ex.map(_compile, todo):
                if verbose:
                    print(f"[etp build] {os.path.basename(obj)} {dt:.1f}s", flush=True)
    objs = [u[1] for u in units()]
    if todo or not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(o) for o in objs):
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, LIB)
    if verbose:
        print(f"[etp build] {LIB} ({time.time() - t0:.1f}s)", flush=True)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    a = ap.parse_args(argv)
    build(force=a.force, jobs=a.jobs)


if __name__ == "__main__":
    sys.exit(main())
