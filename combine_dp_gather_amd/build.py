"""Build the HIP library libmoe_hip.so (gfx950) in-tree with hipcc.

    python -m combine_dp_gather_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe_hip.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def command(out: str):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # no packed fp32 instructions anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            *sources(), "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device feature flag: drop that one warning
    err = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
