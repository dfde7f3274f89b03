"""The persistent attention launch's XCD ranges and split-tail plan, as the
library computes them (its own host/device functions, compiled into a host
program that makes no GPU call), against the plan the GPU tests use to find
split work items (tests/gpu_util.py), plus the invariants the kernel's
scratch layout relies on."""
import os
import shutil
import subprocess

import pytest

from gpu_util import split_plan, xcd_slice

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi", "split_plan_dump.cpp")
EXE = os.path.join(ROOT, "_build", "split_plan_dump")


@pytest.fixture(scope="module")
def dump():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "diffusion_transformer_video_amd", "csrc"), SRC, "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=60, check=True).stdout
    rows = [l.split() for l in out.splitlines()]
    return ([tuple(int(v) for v in r[1:]) for r in rows if r[0] == "P"],
            [tuple(int(v) for v in r[1:]) for r in rows if r[0] == "X"],
            [tuple(int(v) for v in r[1:]) for r in rows if r[0] == "K"][0])


def test_split_plan_matches_the_tests_mirror(dump):
    plans, _, _ = dump
    assert len(plans) == 40 * 401
    for C, ln, T, s, units in plans:
        assert (T, s) == split_plan(ln, C), (C, ln)
        assert units == ln - T + T * s


def test_xcd_ranges_match_and_partition_the_items(dump):
    _, ranges, _ = dump
    by_total = {}
    for total, x, start, ln in ranges:
        assert (start, ln) == xcd_slice(total, x)
        by_total.setdefault(total, []).append((start, ln))
    for total, parts in by_total.items():
        pos = 0
        for start, ln in parts:   # XCDs 0..7 in order: contiguous, covering [0, total)
            assert start == pos and ln >= 0
            pos += ln
        assert pos == total
        assert max(l for _, l in parts) - min(l for _, l in parts) <= 1


def test_split_plan_fits_the_scratch(dump):
    """Every split item's pieces fit the kernel's slots: T s <= 2C <= 2 kSplitC
    partial slots per XCD (8 XCDs x 2 kSplitC = kSplitPieces), T <= C counters per
    XCD, 2 <= s <= kSplitMaxS, and the plan never lengthens the last round."""
    plans, _, (split_c, max_s, pieces) = dump
    assert pieces == 8 * 2 * split_c
    for C, ln, T, s, _ in plans:
        if T == 0:
            assert s == 1
            continue
        assert C <= split_c and ln >= 2 * C
        assert 2 <= s <= max_s and T * s <= 2 * C and T <= C
        # the tail's rounds of pieces, ceil(T s / C) / s of an item, never exceed one item
        assert -(-(T * s) // C) <= s
