"""Compile the HIP library ``libspecverify.so`` for gfx950, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRC = PKG / "csrc" / "spec_verify.hip"
LIB = PKG / "libspecverify.so"
# reference kernels for the benchmark's context figures (empty launch, plain read stream)
BENCH_SRC = PKG / "csrc" / "bench_context.hip"
BENCH_LIB = PKG / "libspecbench.so"
INCLUDE = ROOT / "include"

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(path).exists():
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def _compile(src: Path, out: Path, extra_flags=()) -> Path:
    tmp = out.with_name(out.name + ".tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, f"-I{INCLUDE}", str(src), "-o", str(tmp)]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(extra_flags=(), out: Path | None = None) -> Path:
    """Always recompiles (the library, then the benchmark's reference kernels); writes
    atomically so a running process never sees half a file."""
    lib = _compile(SRC, LIB if out is None else Path(out), extra_flags)
    if out is None:
        _compile(BENCH_SRC, BENCH_LIB, extra_flags)
    return lib


if __name__ == "__main__":
    print(build())
