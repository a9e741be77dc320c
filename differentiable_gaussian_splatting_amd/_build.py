"""Build libgsmi.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgsmi.so")
SOURCES = ["gs_api.cpp", "scan.hip", "radix.hip", "project.hip", "binning.hip", "raster.hip", "planner.hip",
           "loss.hip", "adam.hip", "gate.cpp"]
HEADERS = ["gs_device.h", "gs_internal.h"]

# Float discipline of the forward path: no contraction of a*b+c into fma (only
# explicit fmaf), correctly rounded f32 division and square root, IEEE
# denormals.  Packed-f32 instructions are left out of the code generator.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc"] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd = ["hipcc"] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return out


TORCH_ALLOC = os.path.join(HERE, "libgsmi_torchalloc.so")


def build_torch_alloc() -> str | None:
    """libgsmi_torchalloc.so: C allocator callbacks over PyTorch's HIP caching
    allocator (host code only, linked against libc10_hip), for the binding.
    None when torch is not importable."""
    try:
        import torch
    except ImportError:
        return None
    tp = os.path.dirname(torch.__file__)
    tmp = TORCH_ALLOC + ".tmp"
    cmd = ["hipcc", "-std=c++17", "-O2", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__=1", "-DUSE_ROCM=1",
           "-I" + os.path.join(tp, "include"), "-I" + os.path.join(tp, "include", "torch", "csrc", "api", "include"),
           os.path.join(CSRC, "torch_alloc.cpp"), "-L" + os.path.join(tp, "lib"), "-lc10_hip", "-lc10",
           "-Wl,-rpath," + os.path.join(tp, "lib"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on torch_alloc.cpp:\n{r.stderr}")
    os.replace(tmp, TORCH_ALLOC)
    return TORCH_ALLOC


def build(force: bool = True, jobs: int = 8) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(CSRC, h) for h in HEADERS] + \
        [os.path.join(ROOT, "include", "gs.h")]
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(p) for p in srcs):
        return LIB
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, check=True)
    os.replace(tmp, LIB)
    build_torch_alloc()
    return LIB


if __name__ == "__main__":
    print(build())
