"""Build libsgc.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m structured_grid_cfd_amd.build

Compiles every ``csrc/*.hip`` with hipcc into ``structured_grid_cfd_amd/libsgc.so``.
Flags that matter for results:

* ``-ffp-contract=off``: no fused multiply-add anywhere, so each operation is
  one IEEE round-to-nearest, matching the CPU oracle bit for bit;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed FP32 math;
* no fast-math, FP32 denormals kept (hipcc's default).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libsgc.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsgc.so)")


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip"))


def build(verbose: bool = False) -> Path:
    """Compile and link libsgc.so; always rebuilds."""
    objdir = PKG / "_build"
    objdir.mkdir(exist_ok=True)
    cc = hipcc()
    objs = []
    procs = []
    for src in sources():
        obj = objdir / (src.stem + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-c", str(src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 target feature; that
        # warning is expected and harmless.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src.name)
            print(text, file=sys.stderr)
        elif lines and verbose:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
