"""Build the C consumer of the ABI (ep_c_smoke.c) next to itself: plain C against
include/ep.h and the HIP runtime, linked with libep.so and, as the reference it checks
against, the oracle library (TEST INFRASTRUCTURE). Run by __graft_entry__.build()."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "ep_c_smoke")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "combine_ep_get_03_amd")
    orc = os.path.join(ROOT, "oracle")
    rpath = "$ORIGIN/../../combine_ep_get_03_amd:$ORIGIN/../../oracle:" + os.path.join(ROCM, "lib")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", orc, "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "ep_c_smoke.c"), "-o", BIN + ".tmp",
           "-L", pkg, "-lep", "-L", orc, "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + rpath]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
