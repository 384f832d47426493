"""Build libhcattn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m head_chunked_context_amd.build   (or call build())

Every HIP source compiles for gfx950 only, with packed-fp32 instructions
disabled in device code (v_pk_fma_f32 and friends are left to no one).
Objects are compiled in parallel and linked into
head_chunked_context_amd/libhcattn.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libhcattn.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["fwd.hip", "bwd.hip", "aux.hip", "gemm.hip", "scratch.hip", "hcattn.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# per-source code-generation options: the backward kernels keep their MFMA
# accumulators in VGPRs (measured faster than letting the register allocator
# shuttle them through AGPRs); the forward kernel is scheduled for
# instruction-level parallelism rather than occupancy (it runs at a fixed two
# waves per SIMD; measured 2-3% faster, while the backward kernels lose with it)
FLAGS = {"bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + FLAGS.get(src, []) + list(extra) + lang + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if err:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    """Compile every source and link the shared library at `out` (default: the
    in-tree libhcattn.so the package loads); returns its path.  `extra_flags`
    are added to every compile (for experiments with code-generation options)."""
    build_dir = BUILD_DIR if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra_flags), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
