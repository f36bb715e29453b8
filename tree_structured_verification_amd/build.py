"""Build libtsv.so (the HIP library behind include/tsv.h) for gfx950, in-tree.

    python -m tree_structured_verification_amd.build [--verbose]

Flags that matter for correctness:
  -ffp-contract=off                 no fused multiply-add where the method's
                                    arithmetic must round step by step
  -fno-gpu-flush-denormals-to-zero  fp32 denormals are kept
  -mno-packed-fp32 (target feature) no packed fp32 instructions are emitted
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtsv.so")
SOURCES = ["api.hip", "topk.hip", "tree.hip", "attn.hip", "walk.hip", "commit.hip", "fit.hip", "budget.hip", "chains.hip", "compress.hip"]
ARCH = os.environ.get("TSV_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the tsv library needs ROCm to build")


def command(out: str = LIB, extra=()):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix instructions start in the VGPR form; the register allocator
        # then moves the large accumulators into AGPRs.  Without it, a kernel
        # allowed more than 256 registers puts every accumulator in AGPRs
        # (the latent attention kernel's score tiles then no longer fit)
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-result",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out, *extra,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("building libtsv.so failed")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
