"""Builds libqgemv.so, the gfx950 HIP library behind include/qgemv.h, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "qg_api.hip")
DEPS = [os.path.join(HERE, "csrc", f) for f in
        ("qg_api.hip", "qg_kernels.hpp", "qg_formats.hpp", "qg_device.hpp", "qg_mfma.hpp", "qg_q8act.hpp")] + \
       [os.path.join(ROOT, "include", "qgemv.h")]
LIB = os.path.join(HERE, "libqgemv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile the library (always when force, else only when sources are newer)."""
    if not force and not stale():
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
