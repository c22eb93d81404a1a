"""Stored-P addressing on the CPU: every access the key-owner pass (stores)
and the dQ pass (loads) can make, replayed through the layout functions the
kernels themselves call (hstu_jagged_masked_amd/csrc/pstore.h), stays inside
the caller's buffer and inside its own key tile's blocks, for every residue of
L mod 128, several batch sizes (B <= 8) and head counts (H <= 4), with a buffer
of exactly hstu_attn_pstore_bytes bytes and with one a block short.

The dQ pass's waves past the end of a sequence (its last 128-row query tile
with L mod 128 in [1, 96]) still issue their loads; the replay checks that
these land past their tile's range check and read zeros.  The same replay with
plain unchecked addressing must find an access past the buffer, which shows
the sweep reaches those waves.  No kernel runs here.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "pstore_bounds.cpp")
CSRC = os.path.join(ROOT, "hstu_jagged_masked_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _build(tmp, flat):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = os.path.join(tmp, "pstore_bounds_flat" if flat else "pstore_bounds")
    cmd = [HIPCC, "-O1", "-std=c++17", "-I", CSRC, SRC, "-o", exe]
    if flat:
        cmd.insert(1, "-DFLAT_ADDRESSING")
    subprocess.run(cmd, check=True, capture_output=True, cwd=tmp)
    return exe


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("pstore_bounds"))
    yield _build(tmp, False), _build(tmp, True)
    shutil.rmtree(tmp, ignore_errors=True)


def _cases():
    """(H, lengths): each residue r of L mod 128 in a batch of its own, with
    B from 1 to 8 and H from 1 to 4, the residue's sequence last (whose
    blocks end the buffer), plus zero-length and one-row sequences."""
    rng = np.random.default_rng(128)
    out = []
    for r in range(128):
        B = 1 + r % 8
        H = 1 + (r // 8) % 4
        others = [int(x) for x in rng.integers(0, 700, size=B - 1)]
        last = 128 * int(rng.integers(0, 6)) + r
        if last == 0:
            last = 128
        out.append((H, others + [last]))
    out += [(2, [1, 0, 3, 0]), (4, [0, 0, 5]), (1, [4700, 130, 4160]), (3, [2663])]
    return out


def _run(exe, H, lengths):
    return subprocess.run([exe, str(H)] + [str(x) for x in lengths], capture_output=True,
                          text=True)


def test_every_access_stays_in_bounds(harness):
    exe, _ = harness
    for H, lengths in _cases():
        p = _run(exe, H, lengths)
        assert p.returncode == 0, f"H={H} lengths={lengths}: {p.stdout}{p.stderr}"
        assert p.stdout.strip().endswith("ok")


def test_buffer_size_matches_library(harness):
    """The replay's buffer size (sum of pstore_seq_blocks) is the size the
    library's hstu_attn_pstore_bytes reports for the same offsets."""
    import ctypes

    import hstu_jagged_masked_amd as hj

    if not os.path.exists(hj.LIBRARY):
        pytest.skip("library not built")
    lib = hj.library()
    exe, _ = harness
    for H, lengths in _cases()[::7]:
        off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        got = lib.hstu_attn_pstore_bytes(off.ctypes.data_as(ctypes.c_void_p), len(lengths),
                                         int(off[-1]), H)
        p = _run(exe, H, lengths)
        need = int(p.stdout.split("need=")[1].split()[0])
        assert got == need, (H, lengths)


def test_idle_waves_are_reached(harness):
    """Residues 1..96 leave idle dQ waves in the last query tile: the replay
    counts their loads, and unchecked addressing would take them past the end
    of the buffer."""
    exe, flat = harness
    for r in (1, 3, 32, 64, 65, 96):
        lengths = [256, 128 * 3 + r]
        p = _run(exe, 2, lengths)
        assert p.returncode == 0 and int(p.stdout.split("past_end=")[1].split()[0]) > 0
        q = _run(flat, 2, lengths)
        assert q.returncode == 1 and "load past the buffer" in q.stdout, q.stdout
    # residues 97..127 and 0 have no idle wave in the last tile
    p = _run(exe, 1, [128 * 2 + 100])
    assert p.returncode == 0 and int(p.stdout.split("past_end=")[1].split()[0]) == 0
