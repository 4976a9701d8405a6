"""Builds libpkv.so in-tree: host C++ (radix tree, allocator, C ABI) plus HIP kernels for gfx950.

    python -m prefix_shared_kv_match_amd.build [--debug] [--sanitize]

The host sources are compiled with g++, the .hip sources with hipcc for gfx950 only,
and everything is linked by hipcc into prefix_shared_kv_match_amd/libpkv.so.

--debug defines PKV_DEBUG (kv_scatter then checks its slot list on the host before each
launch) and adds debug info.  --sanitize builds the host sources (radix tree, plans, C ABI
argument checks) with AddressSanitizer and UndefinedBehaviorSanitizer into
_build/sanitize/libpkv.so, leaving the in-tree library alone; the CPU tests run against it
with

    PKV_LIBRARY=_build/sanitize/libpkv.so LD_PRELOAD=$(g++ -print-file-name=libasan.so) \
        ASAN_OPTIONS=detect_leaks=0 python -m pytest tests -m "not gpu"

(the GPU code is not instrumented; the sanitizers cover the host library only).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")

HOST_SOURCES = ["common.cpp", "radix_tree.cpp", "decode_plan.cpp"]
HIP_SOURCES = ["kv_scatter.hip", "extend_attention.hip", "decode_attention.hip", "hbm_probe.hip"]

ARCH = "gfx950"
# Packed-FP32 instructions are switched off for every HIP file.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]
# The attention kernels never see NaN inputs; without this flag every fmaxf in their softmax
# costs an extra canonicalising instruction on the vector ALU, which bounds the extend loop.
HIP_FILE_FLAGS = {"extend_attention.hip": ["-fno-honor-nans"], "decode_attention.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def source_hash() -> str:
    """sha256 over every source the library is built from (kernels, host code, the C ABI header)."""
    import hashlib
    h = hashlib.sha256()
    for d, names in ((CSRC, sorted(os.listdir(CSRC))), (INCLUDE, ["pkv.h"])):
        for n in names:
            if n.endswith((".cpp", ".h", ".hip")):
                h.update(n.encode())
                with open(os.path.join(d, n), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def build(debug: bool = False, verbose: bool = False, sanitize: bool = False) -> str:
    out_dir = os.path.join(BUILD, "sanitize") if sanitize else BUILD
    os.makedirs(out_dir, exist_ok=True)
    hc = hipcc()
    extra = ["-DPKV_DEBUG=1", "-g"] if debug else []
    extra = extra + [f'-DPKV_SOURCE_HASH="{source_hash()}"']
    jobs = []
    objs = []
    for s in HOST_SOURCES:
        o = os.path.join(out_dir, s + ".o")
        objs.append(o)
        jobs.append(["g++", *HOST_FLAGS, *(SANITIZE_FLAGS + ["-g"] if sanitize else []), *extra, "-I", INCLUDE,
                     "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o])
    for s in HIP_SOURCES:
        o = os.path.join(out_dir, s + ".o")
        objs.append(o)
        jobs.append([hc, *HIP_FLAGS, *HIP_FILE_FLAGS.get(s, []), *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    lib_path = os.path.join(out_dir, "libpkv.so") if sanitize else LIB
    tmp = lib_path + ".tmp"
    # the sanitizer runtimes of the host compiler, linked as plain libraries
    _run([hc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, *(["-lasan", "-lubsan"] if sanitize else []),
          "-o", tmp])
    os.replace(tmp, lib_path)
    return lib_path


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="host sources with ASan/UBSan into _build/sanitize/libpkv.so")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.debug, a.verbose, a.sanitize))


if __name__ == "__main__":
    sys.exit(main())
