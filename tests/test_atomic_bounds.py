"""Atomic-dQ addressing on the CPU: the index arithmetic of the atomic-dQ
key-owner pass (hstu_jagged_masked_amd/csrc/atomic_dq.h, the functions the
kernel calls) replayed for every residue of L mod 128, several batch sizes and
head counts: the LDS exchange writes tile each half's buffer exactly once and
every transpose read stays inside it; the K gather and the atomics touch only
the sequence's own rows; each dQ element receives exactly one atomic per key
tile.  A replay with a planted mistake (the second half's row offset dropped)
must fail.  No kernel runs here."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "atomic_bounds.cpp")
CSRC = os.path.join(ROOT, "hstu_jagged_masked_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    tmp = str(tmp_path_factory.mktemp("atomic_bounds"))
    exes = []
    for plant in (False, True):
        exe = os.path.join(tmp, "atomic_bounds_planted" if plant else "atomic_bounds")
        cmd = [HIPCC, "-O1", "-std=c++17", "-I", CSRC, SRC, "-o", exe]
        if plant:
            cmd.insert(1, "-DPLANT_DROP_HALF_OFFSET")
        subprocess.run(cmd, check=True, capture_output=True, cwd=tmp)
        exes.append(exe)
    yield exes
    shutil.rmtree(tmp, ignore_errors=True)


def _cases():
    rng = np.random.default_rng(64)
    out = []
    for r in range(0, 128, 3):
        B = 1 + r % 5
        H = 1 + (r // 5) % 4
        others = [int(x) for x in rng.integers(0, 400, size=B - 1)]
        out.append((H, others + [128 * int(rng.integers(0, 4)) + r]))
    out += [(2, [1, 0, 3, 0]), (1, [4700, 130]), (4, [2663])]
    return out


def _run(exe, H, lengths):
    return subprocess.run([exe, str(H)] + [str(x) for x in lengths], capture_output=True,
                          text=True)


def test_every_atomic_access_in_bounds_and_complete(harness):
    exe, _ = harness
    for H, lengths in _cases():
        p = _run(exe, H, lengths)
        assert p.returncode == 0 and p.stdout.strip().endswith("ok"), \
            f"H={H} lengths={lengths}: {p.stdout}{p.stderr}"


def test_planted_half_offset_mistake_is_caught(harness):
    _, planted = harness
    p = _run(planted, 2, [700, 129])
    assert p.returncode == 1 and "not added once per key tile" in p.stdout, p.stdout
