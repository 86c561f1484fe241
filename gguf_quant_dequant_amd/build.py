"""Builds libqgemv.so, the gfx950 HIP library behind include/qgemv.h, in-tree.

The host code is split into several translation units (per batch width of
the VALU GEMV, per batch tile of the matrix-core GEMV, the int8-activation
GEMV, the MoE chain, and the C ABI), compiled in parallel to objects and
linked into one shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def deps() -> list:
    return sources() + sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + \
        [os.path.join(ROOT, "include", "qgemv.h")]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in deps())


def _filter(out: str) -> list:
    noise = "is not a recognized feature for this target"
    return [l for l in out.splitlines() if noise not in l]


def _compile(src: str, extra: list) -> tuple:
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    cmd = ["hipcc", *HIPCC_FLAGS, *extra, "-c", "-o", obj, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return obj, r.returncode, _filter(r.stdout + r.stderr)


def build(force: bool = True, verbose: bool = False, extra: list | None = None,
          jobs: int | None = None) -> str:
    """Compile the library (always when force, else only when sources are newer).

    extra: additional hipcc flags (e.g. -D tuning knobs)."""
    if not force and not stale():
        return LIB
    extra = list(extra or [])
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), srcs))
    msgs = []
    for obj, rc, m in results:
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(obj)}:\n" + "\n".join(m))
        msgs += m
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[r[0] for r in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(_filter(r.stdout + r.stderr)))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
