"""Build libfsstate.so (gfx950) in-tree with hipcc.

    python -m fsdp_sharded_state_amd.build

The library is one hipcc link of the host planner (fs_plan.cpp) and the
kernels plus launchers (fs_kernels.hip).  Flags:
  --offload-arch=gfx950          CDNA4 only, no other targets
  -ffp-contract=off              no FMA contraction: every + and * rounds once,
                                 as the documented update formulas say
  -target-feature -packed-fp32-ops
                                 no packed-fp32 instructions in device code
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfsstate.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "fs_plan.cpp"), os.path.join(CSRC, "fs_kernels.hip")]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Compile every source into libfsstate.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libfsstate.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
