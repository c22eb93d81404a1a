"""Input generators (CPU): the func layouts encode the visible sets their
docstrings define."""
import numpy as np

import oracle
import workloads as wl
from tests.oracle_pins import _dense_mask


def _onerank_sets(history, n_cand, k_tasks):
    """Visible sets of the OneRank layout written from its definition."""
    L = history + n_cand * (k_tasks + 1)
    sets = []
    for i in range(L):
        if i < history:
            sets.append(set(range(i + 1)))
            continue
        cand = history + (i - history) // (k_tasks + 1) * (k_tasks + 1)
        s = set(range(history)) | {cand, i}
        sets.append(s)
    return sets


def test_onerank_layout_sets():
    history, n_cand, k = np.array([2, 5, 0, 7]), np.array([4, 2, 1, 0]), 3
    lengths = wl.onerank_lengths(history, n_cand, k)
    func = wl.func_onerank(lengths, n_cand, k, 5)
    masks = _dense_mask(lengths, func)
    for b in range(len(lengths)):
        want = _onerank_sets(int(history[b]), int(n_cand[b]), k)
        got = [set(np.nonzero(row)[0].tolist()) for row in masks[b]]
        assert got == want, f"sequence {b}"
    # a task token never sees the other task tokens of its group
    t1 = int(history[0]) + 1  # first task token of group 0 in sequence 0
    assert not masks[0][t1 + 1][t1]


def test_onerank_counts_closed_form():
    # the note's length examples: 132 = 100 + 8*4, 18 = 2 + 4*4, 2208 = 1968 + 60*4
    history, n_cand = np.array([100, 2, 1968]), np.array([8, 4, 60])
    lengths = wl.onerank_lengths(history, n_cand, 3)
    assert lengths.tolist() == [132, 18, 2208]
    counts, total = oracle.default().visible_counts(wl.offsets_from_lengths(lengths),
                                                    wl.func_onerank(lengths, n_cand, 3, 5))
    want, want_total = [], 0
    for H, n in zip(history, n_cand):
        H, n = int(H), int(n)
        row = list(range(1, H + 1)) + [H + 1, H + 2, H + 2, H + 2] * n
        want += row
        want_total += H * (H + 1) // 2 + n * (H + 1) + 3 * n * (H + 2)
    assert counts.tolist() == want
    assert total == want_total
