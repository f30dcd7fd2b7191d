"""The C ABI driven from plain C++ (tests/c_client/pkv_client.cpp): HIP
runtime calls and libpkv.so only, checked against the float64 oracle.

On a machine without a GPU the client must still load (its libraries resolve)
and report that no device is present; on a GPU it runs a mixed step in bf16
and fp32 and checks pool bytes, outputs and error codes."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_client", "pkv_client")


def _exe():
    # __graft_entry__.build() builds it; a tree holding only the library gets it here
    if not os.path.exists(EXE):
        from tests.c_client import build as client_build
        client_build.build()
    return EXE


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="a GPU driver is present: the GPU test runs the client")
def test_client_loads_without_a_device():
    res = subprocess.run([_exe()], capture_output=True, text=True, timeout=120)
    assert res.returncode == 2 and "no HIP device" in res.stdout, res.stdout + res.stderr


@pytest.mark.gpu
def test_client_runs_a_mixed_step_through_the_c_abi():
    print(f"c client: {EXE}", flush=True)
    res = subprocess.run([_exe()], capture_output=True, text=True, timeout=120)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all checks passed" in res.stdout
