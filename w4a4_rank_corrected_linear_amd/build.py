"""Builds libsvdq.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m w4a4_rank_corrected_linear_amd.build [-v]

Every HIP source under csrc/ is compiled for gfx950 only and linked into
w4a4_rank_corrected_linear_amd/libsvdq.so.  build_asan() links a second copy,
_build/asan/libsvdq_asan.so, whose C-ABI source (svdq_api.hip) has its host code built
with AddressSanitizer; it is for the CPU tests of the host-side argument validation
and loads only into a process that preloads the ASan runtime (asan_runtime()).
Compile flags:

  -ffp-contract=off           no implicit FMA contraction: the quantizer's rounding
                              decisions rely on the exact operation sequence
  -mllvm -amdgpu-mfma-vgpr-form
                              MFMA results land in ordinary VGPRs, so the per-group
                              rescale is one v_fmac per element (no accvgpr moves)
  -target-feature -packed-fp32-ops
                              no packed-FP32 VALU instructions
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
BUILD_ASAN = os.path.join(BUILD, "asan")
LIB_ASAN = os.path.join(BUILD_ASAN, "libsvdq_asan.so")
API_SRC = "svdq_api.hip"
# host-only instrumentation: each -fsanitize is scoped to the host pass
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
LIB = os.path.join(PKG, "libsvdq.so")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _compile(src: str, verbose: bool, extra=(), out_dir: str = BUILD) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                    and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libsvdq.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload into the test process)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the ASan runtime libclang_rt.asan-x86_64.so was not found")
    return path


def build_asan(verbose: bool = False) -> str:
    """Link _build/asan/libsvdq_asan.so: svdq_api.hip with host ASan, the kernel
    sources as in build() (their objects are rebuilt when missing)."""
    os.makedirs(BUILD_ASAN, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    api = [x for x in srcs if os.path.basename(x) == API_SRC]
    rest = [x for x in srcs if os.path.basename(x) != API_SRC]
    if len(api) != 1:
        raise RuntimeError(f"{API_SRC} not found")

    def obj_for(src):
        o = os.path.join(BUILD, os.path.basename(src) + ".o")
        if os.path.exists(o) and os.path.getmtime(o) >= os.path.getmtime(src):
            return o
        os.makedirs(BUILD, exist_ok=True)
        return _compile(src, verbose)

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        fut_api = ex.submit(_compile, api[0], verbose, ASAN_FLAGS, BUILD_ASAN)
        objs = list(ex.map(obj_for, rest))
        objs.append(fut_api.result())
    tmp = LIB_ASAN + ".tmp"
    # the ASan runtime is not linked in: the loading process preloads it
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_ASAN)
    return LIB_ASAN


if __name__ == "__main__":
    print(build_asan(verbose="-v" in sys.argv) if "--asan" in sys.argv
          else build(verbose="-v" in sys.argv))
