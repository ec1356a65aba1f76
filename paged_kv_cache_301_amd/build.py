"""Build libpa_decode.so: the HIP kernels and the C ABI, for gfx950 only.

Usage: ``python -m paged_kv_cache_301_amd.build [-v] [--save-temps DIR]``.
Objects go to ``<repo>/_build/`` (not committed); the library is written next
to this file, where ``binding.load()`` looks for it.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpa_decode.so")

ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile every source for gfx950 and link the shared library."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIP_FLAGS, "-x", "hip", "-c", src, "-o", obj]
        if save_temps:
            os.makedirs(save_temps, exist_ok=True)
            cmd.insert(1, f"-save-temps={'obj'}")
        objs.append(obj)
        cmds.append(cmd)

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True,
                           cwd=save_temps or BUILD_DIR)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, flush=True)

    workers = min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(run, cmds))
    tmp = LIB_PATH + ".tmp"
    link = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--save-temps", default=None, help="keep ISA / IR in this directory")
    args = ap.parse_args()
    print(build(args.verbose, args.save_temps))


if __name__ == "__main__":
    main()
