"""Builds libccl.so (the HIP kernels and the C ABI of include/ccl.h) for gfx950,
in-tree next to this file."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("ccl_kernels.hip", "ccl_api.hip", "ccl_large.hip")]
LIB_PATH = os.path.join(HERE, "libccl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere (there is no float arithmetic here either)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        # the host pass does not know the packed-fp32 feature (it only applies
        # to the gfx950 code) and says so once per source; that line is dropped
        print("\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
