"""Build libpa.so in-tree with hipcc for gfx950.

Usage: python -m paged_kv_cache_167_amd.build   (or call build()).
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "pa_kernels.hip"), os.path.join(HERE, "csrc", "pa_blocks.hip"),
           os.path.join(HERE, "csrc", "pa_vkv.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libpa.so")


def command(out: str = LIB) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed-FP32 VALU forms are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix products accumulate in ordinary vector registers: every kernel fits in them,
        # and accumulators kept in the accumulation registers were copied to vector registers
        # and back on each tile wherever vector instructions also touch them (the rescale)
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", "-o", out, *SOURCES,
    ]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
