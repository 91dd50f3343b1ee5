"""Build libfa.so in-tree for gfx950 with hipcc.

Usage: python -m io_aware_tiled_03_amd.build [-j JOBS] [-v]

Every HIP source is compiled with
  hipcc --offload-arch=gfx950 -O3 -fPIC -std=c++17
        -Xclang -target-feature -Xclang -packed-fp32-ops
(the last option keeps the compiler from emitting packed fp32 instructions;
hipcc's host pass warns that it does not know the feature, which is harmless)
and linked into io_aware_tiled_03_amd/libfa.so.  Objects go to
io_aware_tiled_03_amd/_build/.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_plan.cpp", "fa_fwd.hip", "fa_f32.hip", "fa_decode.hip", "fa_bwd.hip",
           "fa_noalloc.hip", "fa_calib.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature name; drop that line.
    out = "\n".join(x for x in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in x)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    if out.strip() and verbose:
        print(out)
    return out


def build(jobs: int = 4, verbose: bool = False, defines=(), out: str = LIB) -> str:
    """Compile every source and link the library (default libfa.so); returns its path.

    `defines` are extra -D macros (tile and launch parameters) for tuning builds,
    which should go to another `out` path."""
    if out == LIB:
        obj_dir = OUT_DIR
    else:   # objects of a tuning build sit beside that library
        obj_dir = os.path.join(os.path.dirname(out), "_build",
                               hashlib.sha1(out.encode()).hexdigest()[:8])
    os.makedirs(obj_dir, exist_ok=True)
    dflags = ["-D" + d for d in defines]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC] + FLAGS + dflags + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="extra preprocessor define for a tuning build")
    ap.add_argument("-o", "--out", default=LIB, help="library path (default: in-tree libfa.so)")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose, args.defines, os.path.abspath(args.out)))


if __name__ == "__main__":
    sys.exit(main())
