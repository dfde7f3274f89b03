"""The library used from a plain C program (tests/c_abi/abi_check.c) through
include/dit.h alone. Without a GPU the program runs its argument-validation
checks (the library validates before touching the device) and stops; with one
it also runs attention, modulate and Euler on device buffers against closed
forms."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "abi_check")


def _run():
    if not os.path.exists(EXE):
        import importlib.util
        spec = importlib.util.spec_from_file_location("abi_build", os.path.join(HERE, "c_abi", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build_abi_check()
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    return r


def test_c_program_argument_checks():
    r = _run()
    assert r.returncode == 0, r.stdout + r.stderr
    lines = [l for l in r.stdout.splitlines() if "rejected" in l]
    assert len(lines) == 5 and all(l.rstrip().endswith("(max err 0)") and " ok " in l for l in lines)


@pytest.mark.gpu
def test_c_program_on_device():
    from gpu_util import need_gpu
    need_gpu()
    r = _run()
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout, r.stdout
