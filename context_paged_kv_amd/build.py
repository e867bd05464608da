"""Build libdcpkv.so (the C-ABI library) in-tree for gfx950.

    python -m context_paged_kv_amd.build          # compile every source, link
    python -m context_paged_kv_amd.build --jobs 4

Every HIP source is compiled with hipcc for gfx950 only, with packed fp32
instructions disabled; host-only C++ goes through the same driver without
device code.  The library lands next to this file.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdcpkv.so")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result", "-fvisibility=hidden",
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-fvisibility=hidden"]
# Per-source additions.  The MLA kernel runs two wavefronts per SIMD (256 registers
# each); with accumulators in VGPRs the whole budget is one class, where the default
# would split it evenly between VGPRs and AGPRs and spill.
EXTRA_FLAGS = {"mla_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    out = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip") or f.endswith(".cpp"):
            out.append(os.path.join(CSRC, f))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE,
               "-I", CSRC, "-c", src, "-o", obj]
    else:
        cmd = [hipcc(), *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip())
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def build(jobs: int = 0, verbose: bool = True) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2) - 1), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


HOST_ASAN_LIB = os.path.join(BUILD, "libdcpkv_host_asan.so")
# the host part (page map, block tables, filters, checks) alone, with the address and
# undefined-behaviour sanitizers, for the host tests; plain g++, no device code
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build_host_asan() -> str:
    """Compile csrc/host.cpp with g++ and the sanitizers into a host-only shared library."""
    os.makedirs(BUILD, exist_ok=True)
    gxx = shutil.which("g++") or "/usr/bin/g++"
    tmp = HOST_ASAN_LIB + ".tmp"
    cmd = [gxx, "-std=c++17", "-fPIC", "-shared", "-Wall", *SANITIZE_FLAGS, "-I", INCLUDE, "-I", CSRC,
           os.path.join(CSRC, "host.cpp"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host sanitizer build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, HOST_ASAN_LIB)
    return HOST_ASAN_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    a = ap.parse_args()
    build(a.jobs)
