"""Build the gfx950 libraries in-tree with hipcc.

  libdcr.so        the delta encode / apply library (C-ABI in include/dcr.h)
  libdcr_synth.so  the seeded synthetic input generator (test / bench inputs)

Run ``python -m bit_exact_xor_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")

LIB_DCR = os.path.join(HERE, "libdcr.so")
LIB_SYNTH = os.path.join(HERE, "libdcr_synth.so")

ARCH = os.environ.get("DCR_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# packed fp32 instructions stay off in all HIP code built here
COMMON = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-I", INCLUDE, "-I", CSRC]


def _compile(out: str, sources: list[str], extra: list[str] | None = None) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, *COMMON, *(extra or []), "-o", tmp, *sources]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = True) -> None:
    _compile(LIB_DCR, [os.path.join(CSRC, "dcr_plan.cpp"), os.path.join(CSRC, "dcr_kernels.hip"),
                       os.path.join(CSRC, "dcr_transcode.hip"), os.path.join(CSRC, "dcr_pack.hip")])
    _compile(LIB_SYNTH, [os.path.join(CSRC, "synth.hip")])
    if verbose:
        print(f"built {LIB_DCR} and {LIB_SYNTH} for {ARCH}")


if __name__ == "__main__":
    build()
    sys.exit(0)
