"""Build libmoe.so in-tree with hipcc for gfx950.

    python -m routing_fp8_grouped_amd.build

Every translation unit is compiled to an object under ``_build/`` (in
parallel), then linked into ``routing_fp8_grouped_amd/libmoe.so``.  HIP code is
compiled with the packed-FP32 feature disabled (``-packed-fp32-ops``).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

SOURCES = ["api.cpp", "quant.hip", "route.hip", "permute.hip", "gemm.hip", "gemm_small.hip",
           "combine.hip", "balance.hip", "backward.hip", "wgrad.hip", "roofs.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")
    return p


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-I", INCLUDE, "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA results in VGPRs: the FP32 promotion reads them without
           # v_accvgpr_read copies
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wno-unused-command-line-argument",
           "-c", os.path.join(CSRC, src), "-o", obj] + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{out}")
    return obj, out


def build(verbose=False, extra=()):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (_, out), s in zip(results, SOURCES):
            if out.strip():
                print(f"[{s}]\n{out}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_c_program(src, out):
    """Compile a C program that calls the library through include/moe.h only
    (a plain C compiler, HIP's runtime API for device memory), linked against
    the in-tree libmoe.so."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rpath_lib = os.path.relpath(PKG, os.path.dirname(os.path.abspath(out)))
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), src, "-o", out,
           "-L", PKG, "-lmoe", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rpath_lib}", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
