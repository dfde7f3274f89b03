"""The FP8 kernels' per-head scale decisions (the library's dit_fp8.hpp,
compiled into a host program that makes no GPU call) against the oracle: the
score-scale exponent n and q's float32 multiplier, bit for bit, over amax pairs
from 1e-30 to 1e30, zeros, and the neighbours of powers of two."""
import os
import shutil
import struct
import subprocess

import pytest

from oracle import fp8

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi", "fp8_scale_dump.cpp")
EXE = os.path.join(ROOT, "_build", "fp8_scale_dump")


def _f(bits):
    return struct.unpack("<f", struct.pack("<I", bits))[0]


@pytest.fixture(scope="module")
def rows():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = [hipcc, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "diffusion_transformer_video_amd", "csrc"), SRC,
           "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=60, check=True).stdout
    return [tuple(int(v) for v in l.split()[1:]) for l in out.splitlines() if l.startswith("S ")]


def test_exponent_and_multiplier_bit_exact(rows):
    assert len(rows) > 10000
    for aqb, akb, n, gb in rows:
        aq, ak = _f(aqb), _f(akb)
        assert n == fp8.score_exponent(aq, ak, 128), (aq, ak)
        g = fp8.q_multiplier(aq, ak, 128)
        assert struct.unpack("<I", struct.pack("<f", float(g)))[0] == gb, (aq, ak, float(g), _f(gb))


def test_cases_cover_the_range_ends(rows):
    ns = {n for _, _, n, _ in rows}
    assert 127 in ns                           # the upper clamp
    assert any(gb == 0 and aqb == 0 for aqb, _, _, gb in rows)   # zero amax -> multiplier 0
    # scores below 2^-127 (both amax nonzero): codes 0, n = 0
    assert any(gb == 0 and n == 0 and aqb != 0 and akb != 0 for aqb, akb, n, gb in rows)
