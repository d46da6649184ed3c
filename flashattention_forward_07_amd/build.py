"""Build libfa355.so in-tree with hipcc for gfx950.

    python -m flashattention_forward_07_amd.build [-v] [--resource-usage]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa355.so")
SOURCES = ["fa355_api.hip", "fa_fwd_kernel.hip", "fa_fwd_pipe.hip", "fa_fwd_ksplit.hip",
           "fa_fwd_f32.hip", "fa_naive.hip", "fa_decode.hip", "fa_small.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are switched off for all device code.  Matrix-core
# builtins keep their accumulators in VGPRs even in kernels that hold other
# accumulators in AGPRs through inline products (the pipelined kernel's scores
# feed the vector ALU directly).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]


def command(out: str = LIB, extra=()) -> list:
    return ([HIPCC, *DEVICE_FLAGS, "-O3", "-std=c++20", "-fPIC", "-shared",
             "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
            + [os.path.join(CSRC, s) for s in SOURCES] + list(extra) + ["-o", out])


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    tmp = LIB + ".tmp"
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, resource_usage="--resource-usage" in sys.argv)
    print(LIB)
