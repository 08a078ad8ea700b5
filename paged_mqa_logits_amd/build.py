"""Build libpml.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Every ``csrc/*.hip`` is compiled on its own (in parallel) and the objects are
linked into ``paged_mqa_logits_amd/libpml.so``. Packed-fp32 VALU instructions
are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libpml.so"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature; that note is harmless
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l and "hip-link" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(jobs: int | None = None, verbose: bool = False) -> Path:
    """Compile every kernel source and link libpml.so; returns its path."""
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip"))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    objs = [BUILD / (s.stem + ".o") for s in srcs]
    jobs = jobs or min(8, os.cpu_count() or 1)

    def compile_one(pair):
        src, obj = pair
        return _run([HIPCC, *CFLAGS, "-c", str(src), "-o", str(obj)])

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(compile_one, zip(srcs, objs)):
            if verbose and out.strip():
                print(out)
    tmp = LIB.with_suffix(".so.tmp")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
