"""The forward entry point that allocates nothing (hstu_attn_fwd_noalloc, its
workspace a fixed per-device array in the library) against hstu_attn_fwd with
a caller workspace: the same kernels, so the outputs must be identical bit for
bit.  Two calls in a row, the second on a smaller input (the array keeps the
first call's contents), full-length and targets-only, called through the C ABI
(ctypes)."""
import ctypes

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda"


@pytest.fixture(scope="module")
def hj():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hstu_jagged_masked_amd as hj

    hj.library()
    return hj


def _inputs(lengths, H, seed, targets=False):
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    rows_q = len(lengths) if targets else T
    out = []
    for i, rows in enumerate((rows_q, T, T)):
        bits, _ = wl.normal_bf16((rows, H, 128), seed + i)
        out.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV))
    off = torch.from_numpy(wl.offsets_from_lengths(lengths)).to(DEV)
    func = torch.from_numpy(wl.func_causal(lengths, 5)).to(DEV)
    tr = torch.from_numpy(wl.targets_last(lengths)).to(DEV) if targets else None
    return out, off, func, tr


def _noalloc(hj, q, k, v, off, func, alpha, max_len, tr):
    """Direct C-ABI call of hstu_attn_fwd_noalloc into a preallocated output."""
    lib = hj.library()
    o = torch.empty_like(q)
    P = ctypes.c_void_p
    st = lib.hstu_attn_fwd_noalloc(
        hj.HSTU_BF16, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()),
        P(off.data_ptr()), off.numel() - 1, k.shape[0], k.shape[1], k.shape[2],
        P(func.data_ptr()), func.shape[0], float(alpha), int(max_len),
        P(tr.data_ptr()) if tr is not None else None,
        P(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.hstu_last_error().decode()
    return o


@pytest.mark.parametrize("targets", [False, True])
def test_noalloc_matches_workspace_forward(hj, targets):
    alpha = 1 / np.sqrt(128)
    for lengths, H, seed in (([700, 64, 1300, 1, 257], 4, 41), ([300, 129], 2, 43)):
        (q, k, v), off, func, tr = _inputs(lengths, H, seed, targets)
        max_len = max(lengths)
        got = _noalloc(hj, q, k, v, off, func, alpha, max_len, tr)
        want = hj.attn_fwd(q, k, v, off, func, alpha, max_len, tr)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, want), f"lengths {lengths}: outputs differ"
