"""Build libmra.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage:  python -m block_sparse_approximate_amd.build [--force]
Objects go to block_sparse_approximate_amd/_build/, the library next to this
file.  The selection-deciding translation units (pooling, logits and
selection) are compiled with -ffp-contract=off so that their fp32 operations
are exactly the ones written; every unit disables packed fp32 instructions.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmra.so")
ARCH = os.environ.get("MRA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
# translation unit -> extra flags
UNITS = {
    "mra_pool": ["-ffp-contract=off"],
    "mra_select": ["-ffp-contract=off"],
    "mra_attn": [],
    "mra_bwd": [],
    "mra_api": [],
}
HEADERS = ["mra_common.h", "mra_pool_unit.h", os.path.join("..", "..", "include", "mra.h")]


def _stale(target: str, deps: list[str]) -> bool:
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(d) > t for d in deps)


def _compile(unit: str, force: bool) -> str:
    src = os.path.join(CSRC, unit + ".hip")
    obj = os.path.join(BUILD, unit + ".o")
    deps = [src] + [os.path.join(CSRC, h) for h in HEADERS]
    if force or _stale(obj, deps):
        cmd = [HIPCC, *COMMON, *UNITS[unit], "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (unit, "\n".join(msgs)))
    return obj


def build(force: bool = True) -> str:
    """Compile every unit (force=True recompiles even when up to date) and link."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(UNITS)) as ex:
        objs = list(ex.map(lambda u: _compile(u, force), UNITS))
    if force or _stale(LIB, objs):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
