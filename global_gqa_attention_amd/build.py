"""Compile the HIP sources into libg4attn.so (gfx950), in place next to this file.

Every HIP translation unit is built with
  -ffp-contract=off       no implicit fused multiply-adds: the rounding points of the
                          numerical contract are the ones written in the source;
  packed-fp32-ops off     scalar fp32 instructions only;
  amdgpu-mfma-vgpr-form   matrix instructions accumulate in ordinary vector registers
                          where the register file allows (the attention kernels keep
                          O in the accumulation registers and the scores in vector
                          registers; without it the compiler shuttles between them).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libg4attn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["attention.hip", "backward.hip", "prologue.hip", "g4attn_api.cpp"]
ARCH = os.environ.get("G4ATTN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", INCLUDE, "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link libg4attn.so; returns the library path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="g4attn_build_") as tmp:
        objs = []

        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            if verbose:
                sys.stderr.write(r.stderr)
            return obj

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
