"""Build libbsp.so for gfx950 with hipcc, in-tree (next to this file).

Usage: ``python -m beam_search_shared_amd.build [--jobs N]``. Every call
recompiles every source: the library is small and the build is the check.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libbsp.so")
BUILD = os.path.join(HERE, "_build")

SOURCES = ["bsp_host.cpp", "write_kv.hip", "merge.hip", "merge_row.hip", "tail_attn.hip",
           "prefix_attn.hip", "naive_attn.hip", "static_ws.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}",
          # keep the compiler away from packed-FP32 instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs:
        print(f"[{src}]\n" + "\n".join(msgs), file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = True) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


HOST_ONLY_SOURCES = ["bsp_host.cpp", "host_only_stubs.cpp"]
SANITIZE = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]


def build_host_sanitized(out_dir: str) -> str:
    """Build the host planner alone (no GPU code: every launcher is a stub) with a
    plain C++ compiler and the address and undefined-behaviour sanitizers, for the
    CPU tests of the host logic. Returns the path of the shared library; load it
    with the sanitizer runtimes preloaded (``sanitizer_runtimes()``)."""
    cxx = os.environ.get("CXX", "g++")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in HOST_ONLY_SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".san.o")
        cmd = [cxx, "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__",
               "-I/opt/rocm/include", *SANITIZE, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        objs.append(obj)
    out = os.path.join(out_dir, "libbsp_host_sanitized.so")
    cmd = [cxx, "-shared", *SANITIZE, *objs, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
           "-lamdhip64", "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return out


def sanitizer_runtimes() -> list:
    """The compiler's address and undefined-behaviour sanitizer runtimes (to preload
    into an uninstrumented Python that loads the sanitized library)."""
    cxx = os.environ.get("CXX", "g++")
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        path = subprocess.run([cxx, f"-print-file-name={name}"], capture_output=True,
                              text=True).stdout.strip()
        if not os.path.isabs(path) or not os.path.exists(path):
            raise RuntimeError(f"{name} not found for {cxx}")
        libs.append(path)
    return libs


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args()
    build(args.jobs)


if __name__ == "__main__":
    main()
