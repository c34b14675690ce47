"""Build libmoe_prefill.so (HIP for gfx950 + the host runtime) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_prefill.so")
MICRO_LIB = os.path.join(HERE, "libmoe_micro.so")   # measurement kernels (roofline denominators)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["moe_kernels.hip", "moe_runtime.cpp", "moe_pack.cpp", "moe_pool_plan.cpp"]

# -ffp-contract=off: no fused multiply-adds beyond the ones written out.
# No fast-math: IEEE division (correctly rounded), fp32 denormals kept.
# -packed-fp32-ops: keep the compiler off the packed fp32 VALU instructions.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Wno-inline-asm",   # M0 is clobbered on purpose by the direct-to-LDS loads (no compiler use of M0 there)
]


def _hipcc(sources, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC] + FLAGS + [os.path.join(CSRC, s) for s in sources] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _hipcc(SOURCES, LIB, verbose)
    _hipcc(["moe_micro.hip"], MICRO_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
