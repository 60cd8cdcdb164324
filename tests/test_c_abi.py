"""The C ABI from plain C: a program that includes the header and links the library, with
no Python in between (tests/c_abi/abi_check.c).  Host part on the CPU; the device part (HIP
runtime buffers, a greedy call checked against the target argmax and a sampling call with
the draft equal to the target) on the GPU, in a child process."""
import subprocess
from pathlib import Path

import pytest

import speculative_sampling_verification_spec_amd as sv

ROOT = Path(__file__).resolve().parent.parent
SRC = ROOT / "tests" / "c_abi" / "abi_check.c"
ROCM_LIB = "/opt/rocm/lib"


def _build(tmp_path: Path) -> Path:
    pkg = sv.LIB_PATH.parent
    assert sv.LIB_PATH.exists(), "build the HIP library first"
    exe = tmp_path / "abi_check"
    subprocess.run(["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-I", str(ROOT / "include"),
                    str(SRC), "-o", str(exe), "-L", str(pkg), "-lspecverify", "-L", ROCM_LIB,
                    "-lamdhip64", f"-Wl,-rpath,{pkg}", f"-Wl,-rpath,{ROCM_LIB}"], check=True)
    return exe


def _run(exe: Path, mode: str):
    r = subprocess.run([str(exe), mode], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed: 0 failure(s)" in r.stdout


def test_c_abi_from_plain_c_host(tmp_path):
    _run(_build(tmp_path), "host")


@pytest.mark.gpu
def test_c_abi_from_plain_c_on_the_device(tmp_path):
    _run(_build(tmp_path), "gpu")
