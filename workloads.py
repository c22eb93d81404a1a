"""Seeded synthetic inputs for HSTU jagged masked attention.

This module builds *inputs only*: sequence lengths, jagged offsets, func
(interval-mask) tensors and random q/k/v/dO tensors.  It holds none of the
operator's arithmetic (no interval decoding, no SiLU, no products), so both the
fp64 oracle and the HIP path may take their inputs from here.

Conventions (shared by every consumer):

* ``seq_offsets`` is int64 ``[B+1]`` with a leading 0 and the running sum of
  the lengths (the "complete cumsum" the MLCommons DLRMv4 page mentions for its
  jagged inputs).
* ``func`` is int32 ``[nfunc, total]``: column ``t`` holds the bounds for global
  row ``t``.  Row 0 of it is the end of interval 0 (which starts at 0); rows
  ``2j-1, 2j`` are the start and end of interval ``j`` (TorchEasyRec PR #670,
  "What changed": the interleaved layout, and the pad rule that repeats the last
  bound so a pad interval has ``max <= min``).  All bounds are sequence-local.
* Random tensors are standard normal, drawn in float32 with numpy's PCG64 and
  (for bf16 workloads) rounded to bfloat16 with round-to-nearest-even.  Large
  workloads draw on the device with torch's seeded generator instead, since
  drawing billions of samples on the host takes minutes.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# lengths and offsets
# ---------------------------------------------------------------------------


def lengths_uniform(batch: int, length: int) -> np.ndarray:
    return np.full(batch, int(length), dtype=np.int64)


def lengths_ragged(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Lengths drawn uniformly from the integers in [lo, hi] (both inclusive)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=batch, dtype=np.int64)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def local_rows(lengths) -> np.ndarray:
    """Sequence-local row index of every global row (0..L_b-1 per sequence)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    total = int(lengths.sum())
    if total == 0:
        return np.zeros(0, dtype=np.int64)
    starts = np.repeat(offsets_from_lengths(lengths)[:-1], lengths)
    return np.arange(total, dtype=np.int64) - starts


def seq_length_per_row(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.repeat(lengths, lengths)


# ---------------------------------------------------------------------------
# func tensors (the caller-side encoding of each row's visible intervals)
# ---------------------------------------------------------------------------


def _pack(rows, nfunc: int) -> np.ndarray:
    """Stack bound rows into ``[nfunc, total]`` int32, padding empty intervals.

    ``rows`` holds the first ``len(rows)`` bounds.  Remaining rows repeat the
    last given bound, which makes every pad interval ``[x, x)`` -- empty.
    """
    if nfunc < 1 or nfunc % 2 == 0:
        raise ValueError("nfunc must be odd and >= 1")
    if len(rows) > nfunc:
        raise ValueError(f"{len(rows)} bounds do not fit nfunc={nfunc}")
    out = [np.asarray(r, dtype=np.int64) for r in rows]
    while len(out) < nfunc:
        out.append(out[-1])
    return np.ascontiguousarray(np.stack(out).astype(np.int32))


def func_causal(lengths, nfunc: int = 5) -> np.ndarray:
    """Row i sees [0, i+1); every other interval padded empty by repeating i+1."""
    i = local_rows(lengths)
    return _pack([i + 1], nfunc)


def func_sla(lengths, k1: int, k2: int, nfunc: int = 5) -> np.ndarray:
    """Two-interval SLA mask: a global prefix of k2 columns plus a causal window of k1.

    interval 0 = [0, min(k2, i+1)); interval 1 = [max(k2, i-k1+1), i+1); the
    rest padded empty.  With k1 >= L and k2 = 0 the rows are
    [0, 0, i+1, i+1, i+1], i.e. plain causal (TorchEasyRec PR #670 test thread).
    """
    if nfunc < 3:
        raise ValueError("SLA needs two intervals (nfunc >= 3)")
    i = local_rows(lengths)
    f0 = np.minimum(k2, i + 1)
    f1 = np.maximum(k2, i - k1 + 1)
    f2 = i + 1
    return _pack([f0, f1, f2], nfunc)


def func_partition(lengths, s1: int = 2, s2: int = 5, nfunc: int = 5) -> np.ndarray:
    """Causal row split into three adjacent chunks [s1,s1,s2,s2,i+1].

    With s1' = min(s1, i+1) and s2' = min(s2, i+1) the union of
    [0,s1'), [s1',s2'), [s2',i+1) is again [0, i+1) (TorchEasyRec PR #670, the
    test that decodes every interval).
    """
    if nfunc < 5:
        raise ValueError("the partition uses three intervals (nfunc >= 5)")
    i = local_rows(lengths)
    a = np.minimum(s1, i + 1)
    b = np.minimum(s2, i + 1)
    return _pack([a, a, b, b, i + 1], nfunc)


def func_three_interval(lengths, n_blocks: int = 32, block: int = 8, nfunc: int = 5) -> np.ndarray:
    """Prefix + own-candidate-block + task-token masks (three intervals).

    Each sequence ends with ``n_blocks`` candidate blocks of ``block`` rows and a
    final task-token row; the history is ``h = L - 1 - n_blocks*block`` rows.
    History row i sees [0, i+1) and the task token; a row of candidate block c
    sees the whole history, its own block [h+8c, h+8c+8) and the task token; the
    task-token row sees the history and itself.  Sequences too short for the
    blocks fall back to plain causal rows.
    """
    if nfunc < 5:
        raise ValueError("three intervals need nfunc >= 5")
    lengths = np.asarray(lengths, dtype=np.int64)
    i = local_rows(lengths)
    L = seq_length_per_row(lengths)
    h = L - 1 - n_blocks * block
    f = np.zeros((5, i.size), dtype=np.int64)
    hist = i < h
    cand = (i >= h) & (i < L - 1)
    last = i == L - 1
    short = h < 1
    # history rows
    f[0] = np.where(hist, i + 1, h)
    c = np.where(cand, (i - h) // block, 0)
    f[1] = np.where(cand, h + block * c, f[0])
    f[2] = np.where(cand, h + block * c + block, f[0])
    f[3] = L - 1
    f[4] = L
    # task-token row: history then itself (interval 1 empty)
    f[1] = np.where(last, f[0], f[1])
    f[2] = np.where(last, f[0], f[2])
    # short sequences: plain causal
    f[0] = np.where(short, i + 1, f[0])
    f[1] = np.where(short, i + 1, f[1])
    f[2] = np.where(short, i + 1, f[2])
    f[3] = np.where(short, i + 1, f[3])
    f[4] = np.where(short, i + 1, f[4])
    return _pack(list(f), nfunc)


def onerank_lengths(history, n_candidates, k_tasks: int = 3) -> np.ndarray:
    """Sequence lengths of the OneRank layout: history plus, per candidate, the
    candidate token followed by its K task tokens (groups of K + 1)."""
    history = np.asarray(history, dtype=np.int64)
    n_candidates = np.asarray(n_candidates, dtype=np.int64)
    return history + n_candidates * (k_tasks + 1)


def func_onerank(lengths, n_candidates, k_tasks: int = 3, nfunc: int = 5) -> np.ndarray:
    """OneRank task-private masks (TorchEasyRec PR #670 follow-up commit, the
    build_onerank_func_tensor note).

    Sequence b holds a history of H_b = L_b - n_b (K + 1) rows, then n_b groups
    of K + 1 rows: candidate e_i followed by task tokens t_1..t_K.  Task token
    t_k of group i sees [0, H_b), e_i and itself -- three intervals, because the
    other task tokens of the group lie between e_i and t_k.  Readings (the note
    states only the task tokens' set): history rows are causal, [0, r+1); a
    candidate sees the history and itself.  K = 3 matches the note's length
    examples (148 -> 132, 26 -> 18, 2328 -> 2208 when each candidate stops
    being replicated once per task token).
    """
    if nfunc < 5:
        raise ValueError("task tokens need three intervals (nfunc >= 5)")
    lengths = np.asarray(lengths, dtype=np.int64)
    n_candidates = np.broadcast_to(np.asarray(n_candidates, dtype=np.int64), lengths.shape)
    hist = lengths - n_candidates * (k_tasks + 1)
    if np.any(hist < 0):
        raise ValueError("a sequence is shorter than its candidate groups")
    i = local_rows(lengths)
    H = np.repeat(hist, lengths)
    in_hist = i < H
    g = np.where(in_hist, 0, (i - H) // (k_tasks + 1))        # group of a candidate row
    pos = np.where(in_hist, 0, (i - H) % (k_tasks + 1))       # 0 = candidate, k = task k
    cand = H + g * (k_tasks + 1)                              # the group's candidate row
    f0 = np.where(in_hist, i + 1, H)
    f1 = np.where(in_hist, f0, cand)
    f2 = np.where(in_hist, f0, cand + 1)
    is_task = (~in_hist) & (pos > 0)
    f3 = np.where(is_task, i, f2)
    f4 = np.where(is_task, i + 1, f2)
    return _pack([f0, f1, f2, f3, f4], nfunc)


def func_random(lengths, nfunc: int, seed: int, spread: int = 4) -> np.ndarray:
    """Arbitrary int32 bounds, including negative, past-the-end, reversed and
    overlapping pairs, for decode tests on small inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = seq_length_per_row(lengths)
    f = rng.integers(-spread, L + spread + 1, size=(nfunc, L.size))
    return np.ascontiguousarray(f.astype(np.int32))


def targets_last(lengths) -> np.ndarray:
    """Candidate row of each sequence = its last row (L_b - 1)."""
    return np.asarray(lengths, dtype=np.int64).astype(np.int32) - 1


# ---------------------------------------------------------------------------
# random tensors
# ---------------------------------------------------------------------------


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(shape, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(size=shape, dtype=np.float32)


def normal_bf16(shape, seed: int):
    """Standard normal rounded to bf16: returns (bits uint16, values float32)."""
    bits = round_to_bf16_bits(normal_f32(shape, seed))
    return bits, bf16_bits_to_f32(bits)


def normal_device(shape, seed: int, dtype, device="cuda"):
    """Standard normal drawn on the device with torch's seeded generator."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


# ---------------------------------------------------------------------------
# named workloads (the shapes the pages measure on)
# ---------------------------------------------------------------------------

SLA_K1 = 256  # window width
SLA_K2 = 32   # global prefix width


def workload(name: str):
    """Return a dict describing a named workload: lengths, func builder, H, D,
    dtype, alpha, max_len, and seeds.

    Names:
      tiny_fp32      B=2 lengths 37 and 64, H=2, D=32, fp32, causal nfunc=5
      sla_1k         B=32 S=1024 H=4 D=128 bf16, two-interval SLA, nfunc=5
      sla_2k         B=16 S=2048 H=8 D=128 bf16, same SLA (nfunc=5 and 3)
      hstu_2663      B=1024 L=2663 H=4 D=128 bf16 causal, last row candidate
      hstu_ragged    B=1024 L~U{1332..3994} (seed 41), otherwise as hstu_2663
      hstu_4086      B=1024 L=4086, otherwise as hstu_2663
      three_interval B=256 L~U{512..4096} (seed 5) H=4 D=128 bf16, 3 intervals
      onerank        B=256, 60 candidates x (1 + 3 task tokens) after a history
                     H~U{272..3856} (seed 6), H=4 D=128 bf16, the OneRank layout
    """
    if name == "tiny_fp32":
        lengths = np.array([37, 64], dtype=np.int64)
        return dict(name=name, lengths=lengths, H=2, D=32, dtype="fp32",
                    func=lambda ls, nf=5: func_causal(ls, nf), nfunc=5,
                    alpha=1.0 / np.sqrt(32.0), max_len=64, seed=1)
    if name == "sla_1k":
        lengths = lengths_uniform(32, 1024)
        return dict(name=name, lengths=lengths, H=4, D=128, dtype="bf16",
                    func=lambda ls, nf=5: func_sla(ls, SLA_K1, SLA_K2, nf), nfunc=5,
                    alpha=1.0 / np.sqrt(128.0), max_len=1024, seed=2)
    if name == "sla_2k":
        lengths = lengths_uniform(16, 2048)
        return dict(name=name, lengths=lengths, H=8, D=128, dtype="bf16",
                    func=lambda ls, nf=5: func_sla(ls, SLA_K1, SLA_K2, nf), nfunc=5,
                    alpha=1.0 / np.sqrt(128.0), max_len=2048, seed=3)
    if name in ("hstu_2663", "hstu_ragged", "hstu_4086"):
        if name == "hstu_2663":
            lengths, seed = lengths_uniform(1024, 2663), 4
        elif name == "hstu_ragged":
            lengths, seed = lengths_ragged(1024, 1332, 3994, 41), 41
        else:
            lengths, seed = lengths_uniform(1024, 4086), 42
        return dict(name=name, lengths=lengths, H=4, D=128, dtype="bf16",
                    func=lambda ls, nf=5: func_causal(ls, nf), nfunc=5,
                    alpha=1.0 / np.sqrt(128.0), max_len=int(lengths.max()), seed=seed)
    if name == "three_interval":
        lengths = lengths_ragged(256, 512, 4096, 5)
        return dict(name=name, lengths=lengths, H=4, D=128, dtype="bf16",
                    func=lambda ls, nf=5: func_three_interval(ls, 32, 8, nf), nfunc=5,
                    alpha=1.0 / np.sqrt(128.0), max_len=int(lengths.max()), seed=5)
    if name == "onerank":
        hist = lengths_ragged(256, 272, 3856, 6)
        n_cand = np.full(256, 60, dtype=np.int64)
        lengths = onerank_lengths(hist, n_cand, 3)
        return dict(name=name, lengths=lengths, H=4, D=128, dtype="bf16",
                    func=lambda ls, nf=5: func_onerank(ls, n_cand, 3, nf), nfunc=5,
                    alpha=1.0 / np.sqrt(128.0), max_len=int(lengths.max()), seed=6)
    raise KeyError(name)


WORKLOADS = ("tiny_fp32", "sla_1k", "sla_2k", "hstu_2663", "hstu_ragged", "hstu_4086",
             "three_interval", "onerank")
