"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_attention_slot_amd.build [--verbose]

Object files go to _build/ at the repository root; the shared library is
written next to this file.  Every call recompiles every source.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIP_SOURCES = ["kv_append.hip", "decode.hip", "decode_mfma.hip", "decode_q8.hip", "chunk.hip", "verify.hip", "gather.hip", "attend.hip"]
HOST_SOURCES = ["host_alloc.cpp"]

# Packed-fp32 instructions are kept out of the generated code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False, jobs: int | None = None, defines=(), out: str | None = None,
          build_dir: str | None = None) -> str:
    """Compile every source and link the library.  `defines` (NAME=VALUE)
    override tuning constants; `out`/`build_dir` place a variant build."""
    hipcc = _hipcc()
    bdir = build_dir or BUILD_DIR
    lib_path = out or LIB_PATH
    os.makedirs(bdir, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC] + [f"-D{d}" for d in defines]
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        cmds.append([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        cmds.append(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for fut in [ex.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    tmp = lib_path + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib_path)
    return lib_path


PROBE_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes")
# Standalone measurement executables (not part of the library): the decode
# access pattern's HBM read rate, and the softmax instructions' issue cost
# beside the matrix cores.
PROBES = ("tile_read_probe", "valu_mfma_cost_probe")


def build_probe(out: str | None = None, verbose: bool = False, name: str | None = None) -> list[str]:
    """Compile the probe executables (all of them, or `name`; `out` names the
    executable when one is built) under the build directory and return their
    paths."""
    names = [name] if name else list(PROBES)
    exes = []
    for n in names:
        exe = out if (out and len(names) == 1) else os.path.join(BUILD_DIR, n)
        os.makedirs(os.path.dirname(exe), exist_ok=True)
        _run([_hipcc(), *[f for f in HIP_FLAGS if f not in ("-fPIC", "-Wall")], "-o", exe,
              os.path.join(PROBE_DIR, n + ".hip")], verbose)
        exes.append(exe)
    return exes


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("-D", dest="defines", action="append", default=[], help="NAME=VALUE tuning override")
    ap.add_argument("--out", default=None, help="write the library here instead of the package")
    ap.add_argument("--build-dir", default=None)
    ap.add_argument("--probe", action="store_true", help="build only the probe executables")
    a = ap.parse_args()
    if a.probe:
        print("\n".join(build_probe(out=a.out, verbose=a.verbose)))
    else:
        print(build(verbose=a.verbose, defines=a.defines, out=a.out, build_dir=a.build_dir))
