"""Pins that tie the fp64 oracle to facts outside itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises ``AssertionError``
when the oracle disagrees with a value or property fixed by the pages or by
mathematics: hand-derived closed forms, closed-form visible counts, the mask
invariants the TorchEasyRec PR #670 tests state, the targets-only equivalence of
MLCommons training PR #903, gradients from torch autograd and from central finite
differences, and special cases that reduce to a plain matrix product.

``tests/test_oracle.py`` runs every pin against the oracle; the mutation test runs
them against deliberately broken copies of the oracle (built on the CPU) and
requires each copy to fail at least one pin.  Run as a script,
``python tests/oracle_pins.py LIB`` prints the names of the pins that fail for the
oracle library at path LIB.
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402


def _silu(x):
    return x / (1.0 + math.exp(-x))


def _dsilu(x):
    s = 1.0 / (1.0 + math.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def _eval(expr):
    return float(eval(expr, {"__builtins__": {}}, {"silu": _silu, "dsilu": _dsilu}))


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    lim = atol + rtol * (np.max(np.abs(b)) if b.size else 0.0)
    assert err <= lim, f"{what}: max err {err:.3e} > {lim:.3e}"


def _rand_problem(lengths, H, D, seed, func=None, nfunc=5):
    lengths = np.asarray(lengths, dtype=np.int64)
    off = wl.offsets_from_lengths(lengths)
    T = int(off[-1])
    q = wl.normal_f32((T, H, D), seed).astype(np.float64)
    k = wl.normal_f32((T, H, D), seed + 1000).astype(np.float64)
    v = wl.normal_f32((T, H, D), seed + 2000).astype(np.float64)
    do = wl.normal_f32((T, H, D), seed + 3000).astype(np.float64)
    if func is None:
        func = wl.func_random(lengths, nfunc, seed + 4000)
    return off, q, k, v, do, func


def _dense_mask(lengths, func):
    """Visible[i][j] for each sequence, by testing every column against every
    interval (a dense membership test, not a walk over intervals)."""
    off = wl.offsets_from_lengths(lengths)
    nfunc = func.shape[0]
    masks = []
    for b in range(len(lengths)):
        L = int(lengths[b])
        m = np.zeros((L, L), dtype=bool)
        for i in range(L):
            t = off[b] + i
            bounds = [(0, int(func[0, t]))]
            bounds += [(int(func[2 * j - 1, t]), int(func[2 * j, t]))
                       for j in range(1, (nfunc - 1) // 2 + 1)]
            for j in range(L):
                m[i, j] = any(lo <= j < hi for lo, hi in bounds)
        masks.append(m)
    return masks


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------


def pin_hand_examples(orc):
    with open(os.path.join(HERE, "golden", "hand_examples.json")) as f:
        data = json.load(f)
    for ex in data["examples"]:
        lengths = np.array(ex["lengths"], dtype=np.int64)
        off = wl.offsets_from_lengths(lengths)
        H, D = ex["H"], ex["D"]
        func = np.array(ex["func"], dtype=np.int32)
        tr = ex.get("target_rows")
        tr = None if tr is None else np.array(tr, dtype=np.int32)
        q = np.array(ex["q"], dtype=np.float64).reshape(-1, H, D)
        k = np.array(ex["k"], dtype=np.float64).reshape(-1, H, D)
        v = np.array(ex["v"], dtype=np.float64).reshape(-1, H, D)
        do = np.array(ex["dout"], dtype=np.float64).reshape(-1, H, D)
        counts, total = orc.visible_counts(off, func, tr)
        assert list(counts) == ex["counts"], f"{ex['name']}: counts {list(counts)}"
        assert total == sum(ex["counts"]), f"{ex['name']}: total pairs"
        o = orc.fwd(q, k, v, off, func, ex["alpha"], ex["max_len"], tr)
        dq, dk, dv = orc.bwd(q, k, v, do, off, func, ex["alpha"], ex["max_len"], tr)
        for name, got in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
            want = np.array([[_eval(e) for e in row] for row in ex[name]]).reshape(got.shape)
            _close(got, want, what=f"{ex['name']}.{name}")


def pin_counts_closed_forms(orc):
    # causal: row i sees i+1 columns; a sequence of L rows has L(L+1)/2 pairs.
    lengths = np.array([1, 5, 64, 2663], dtype=np.int64)
    off = wl.offsets_from_lengths(lengths)
    counts, total = orc.visible_counts(off, wl.func_causal(lengths, 5))
    assert np.array_equal(counts, wl.local_rows(lengths) + 1), "causal counts"
    assert total == int(sum(L * (L + 1) // 2 for L in lengths)), "causal total"
    # 2663 rows: 3,547,116 pairs per sequence and head
    c1, t1 = orc.visible_counts(wl.offsets_from_lengths([2663]), wl.func_causal([2663], 1))
    assert t1 == 3547116, "causal 2663"
    # SLA with a prefix of 32 and a window of 256:
    # |V_i| = min(32, i+1) + max(0, i+1 - max(32, i-255)).
    for S, want_total in ((1024, 253584), (2048, 548496)):
        lengths = np.array([S], dtype=np.int64)
        for nfunc in (3, 5):
            counts, total = orc.visible_counts(wl.offsets_from_lengths(lengths),
                                               wl.func_sla(lengths, 256, 32, nfunc))
            i = np.arange(S)
            want = np.minimum(32, i + 1) + np.maximum(0, i + 1 - np.maximum(32, i - 255))
            assert np.array_equal(counts, want), f"SLA counts S={S} nfunc={nfunc}"
            assert total == want_total, f"SLA total S={S}: {total}"
    # the three-chunk partition of a causal row is causal again
    lengths = np.array([1, 2, 3, 6, 9, 17], dtype=np.int64)
    off = wl.offsets_from_lengths(lengths)
    counts, _ = orc.visible_counts(off, wl.func_partition(lengths))
    assert np.array_equal(counts, wl.local_rows(lengths) + 1), "partition counts"
    # every interval of the nfunc=9 layout is read: five disjoint unit intervals
    lengths = np.array([12], dtype=np.int64)
    f = np.array([[1], [2], [3], [4], [5], [6], [7], [8], [9]], dtype=np.int32) * 1
    f = np.repeat(f, 12, axis=1)
    counts, _ = orc.visible_counts(wl.offsets_from_lengths(lengths), f)
    # [0,1) u [2,3) u [4,5) u [6,7) u [8,9) -> 5 columns
    assert np.all(counts == 5), "nfunc=9 intervals"


def pin_decode_bruteforce(orc):
    """Random bounds (negative, past-the-end, reversed, overlapping): the visible
    set must equal a dense membership test.  The forward with v = identity
    (D = L, v_j = e_j) exposes each row's visible columns as its nonzero outputs."""
    for nfunc in (1, 3, 5, 7):
        for seed, lengths in ((11, [7, 0, 13, 1, 9]), (12, [16, 5]), (13, [3, 3, 3])):
            lengths = np.array(lengths, dtype=np.int64)
            off = wl.offsets_from_lengths(lengths)
            func = wl.func_random(lengths, nfunc, seed * 10 + nfunc)
            masks = _dense_mask(lengths, func)
            counts, total = orc.visible_counts(off, func)
            want = np.concatenate([m.sum(axis=1) for m in masks]) if masks else []
            assert np.array_equal(counts, want), f"counts nfunc={nfunc} seed={seed}"
            assert total == int(np.sum(want)), "total"
            # targets-only counts
            tr = np.array([max(int(L) - 1 - (b % 2), 0) if L else 0 for b, L in enumerate(lengths)],
                          dtype=np.int32)
            tc, _ = orc.visible_counts(off, func, tr)
            for b, L in enumerate(lengths):
                if L:
                    assert tc[b] == masks[b][tr[b]].sum(), "targets-only counts"
            # mask through the forward, one sequence at a time (D = L)
            for b, L in enumerate(lengths):
                L = int(L)
                if L == 0:
                    continue
                sub_off = np.array([0, L], dtype=np.int64)
                fsub = np.ascontiguousarray(func[:, off[b]:off[b + 1]])
                q = np.ones((L, 1, L))
                k = np.ones((L, 1, L))
                v = np.eye(L).reshape(L, 1, L)
                o = orc.fwd(q, k, v, sub_off, fsub, 1.0 / L, 1.0)
                # P = 1 for every pair, so a visible pair shows silu(1) at o[i, j]
                want_o = masks[b] * _silu(1.0)
                _close(o[:, 0, :], want_o, what=f"identity-v mask nfunc={nfunc} seq={b}")


def pin_invariants(orc):
    rng_lengths = np.array([17, 40, 1, 33], dtype=np.int64)
    H, D = 2, 8
    off, q, k, v, do, _ = _rand_problem(rng_lengths, H, D, seed=21)
    alpha, max_len = 0.3, 40.0
    causal = wl.func_causal(rng_lengths, 5)

    def both(func):
        return (orc.fwd(q, k, v, off, func, alpha, max_len),) + \
            orc.bwd(q, k, v, do, off, func, alpha, max_len)

    ref = both(causal)
    # partition [s1,s1,s2,s2,i+1] reproduces causal exactly (same columns, same order)
    for a, b in zip(both(wl.func_partition(rng_lengths)), ref):
        assert np.array_equal(a, b), "partition != causal"
    # SLA with the window spanning the sequence and no prefix is causal
    for a, b in zip(both(wl.func_sla(rng_lengths, 10**6, 0, 5)), ref):
        assert np.array_equal(a, b), "full-window SLA != causal"
    # a causal func is the lower triangle: compare with the dense tril mask
    for a, b in zip(both(causal[:1]), ref):
        assert np.array_equal(a, b), "nfunc=1 causal != nfunc=5 causal"
    masks = _dense_mask(rng_lengths, causal)
    for m in masks:
        assert np.array_equal(m, np.tril(np.ones_like(m))), "causal mask is not tril"
    # padding SLA to nfunc=5 reproduces the nfunc=3 result bit for bit
    sla3 = wl.func_sla(rng_lengths, 8, 3, 3)
    sla5 = wl.func_sla(rng_lengths, 8, 3, 5)
    assert np.array_equal(sla5[:3], sla3)
    for a, b in zip(both(sla5), both(sla3)):
        assert np.array_equal(a, b), "nfunc=5 padded != nfunc=3"
    # extra empty intervals of any encoding ([x,x), reversed) change nothing
    pad = np.concatenate([sla3, np.array([[0], [0]]) * np.ones((2, sla3.shape[1]), int),
                          np.array([[9], [2]]) * np.ones((2, sla3.shape[1]), int)]).astype(np.int32)
    for a, b in zip(both(pad), both(sla3)):
        assert np.array_equal(a, b), "empty pads not inert"
    # jagged independence: each sequence alone gives the same rows
    func = wl.func_random(rng_lengths, 5, 77)
    o = orc.fwd(q, k, v, off, func, alpha, max_len)
    dq, dk, dv = orc.bwd(q, k, v, do, off, func, alpha, max_len)
    for b in range(len(rng_lengths)):
        s, e = off[b], off[b + 1]
        so = np.array([0, e - s])
        fs = np.ascontiguousarray(func[:, s:e])
        ob = orc.fwd(q[s:e], k[s:e], v[s:e], so, fs, alpha, max_len)
        gb = orc.bwd(q[s:e], k[s:e], v[s:e], do[s:e], so, fs, alpha, max_len)
        assert np.array_equal(ob, o[s:e]), "jagged independence (fwd)"
        for a, g in zip(gb, (dq, dk, dv)):
            assert np.array_equal(a, g[s:e]), "jagged independence (bwd)"
    # targets-only row equals the full-length row at the candidate; its
    # gradients equal the full-length gradients with dO zero except there
    tr = np.array([16, 0, 0, 20], dtype=np.int32)
    rows = off[:-1] + tr
    o_t = orc.fwd(q[rows], k, v, off, func, alpha, max_len, tr)
    _close(o_t, o[rows], rtol=0, atol=0, what="targets-only fwd")
    do_masked = np.zeros_like(do)
    do_masked[rows] = do[rows]
    fdq, fdk, fdv = orc.bwd(q, k, v, do_masked, off, func, alpha, max_len)
    tdq, tdk, tdv = orc.bwd(q[rows], k, v, do[rows], off, func, alpha, max_len, tr)
    _close(tdq, fdq[rows], rtol=1e-13, atol=1e-15, what="targets-only dq")
    _close(tdk, fdk, rtol=1e-13, atol=1e-15, what="targets-only dk")
    _close(tdv, fdv, rtol=1e-13, atol=1e-15, what="targets-only dv")


def pin_autograd(orc):
    """Gradients vs torch autograd in float64 on the dense masked formulation."""
    import torch

    lengths = np.array([9, 1, 14], dtype=np.int64)
    H, D = 2, 5
    for seed, nfunc in ((31, 5), (32, 3), (33, 1)):
        off, q, k, v, do, func = _rand_problem(lengths, H, D, seed, nfunc=nfunc)
        alpha, max_len = 0.7, 14.0
        o = orc.fwd(q, k, v, off, func, alpha, max_len)
        dq, dk, dv = orc.bwd(q, k, v, do, off, func, alpha, max_len)
        masks = _dense_mask(lengths, func)
        for b in range(len(lengths)):
            s, e = off[b], off[b + 1]
            for h in range(H):
                tq = torch.tensor(q[s:e, h], requires_grad=True)
                tk = torch.tensor(k[s:e, h], requires_grad=True)
                tv = torch.tensor(v[s:e, h], requires_grad=True)
                m = torch.tensor(masks[b], dtype=torch.float64)
                sc = torch.nn.functional.silu(alpha * (tq @ tk.T)) / max_len * m
                to = sc @ tv
                to.backward(torch.tensor(do[s:e, h]))
                _close(o[s:e, h], to.detach().numpy(), what="autograd o")
                _close(dq[s:e, h], tq.grad.numpy(), what="autograd dq")
                _close(dk[s:e, h], tk.grad.numpy(), what="autograd dk")
                _close(dv[s:e, h], tv.grad.numpy(), what="autograd dv")


def pin_finite_differences(orc):
    """dL/dx of L = sum(O * dO) by central differences equals the oracle's bwd."""
    lengths = np.array([5, 7], dtype=np.int64)
    H, D = 2, 3
    off, q, k, v, do, func = _rand_problem(lengths, H, D, seed=41, nfunc=5)
    alpha, max_len = 0.9, 7.0
    dq, dk, dv = orc.bwd(q, k, v, do, off, func, alpha, max_len)
    eps = 1e-6

    def loss(q_, k_, v_):
        return float(np.sum(orc.fwd(q_, k_, v_, off, func, alpha, max_len) * do))

    rng = np.random.Generator(np.random.PCG64(5))
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in grad.shape)
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][idx] += eps
            up = loss(args["q"], args["k"], args["v"])
            args[name][idx] -= 2 * eps
            dn = loss(args["q"], args["k"], args["v"])
            fd = (up - dn) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 + 1e-6 * abs(fd), \
                f"finite difference d{name}{idx}: {fd} vs {grad[idx]}"


def pin_special_cases(orc):
    lengths = np.array([6, 11], dtype=np.int64)
    H, D = 1, 4
    off, q, k, v, do, func = _rand_problem(lengths, H, D, seed=51, nfunc=5)
    # alpha = 0: every score is silu(0) = 0 -> O = 0, dV = 0; dQ, dK carry alpha -> 0
    o = orc.fwd(q, k, v, off, func, 0.0, 11.0)
    assert np.all(o == 0.0), "alpha=0 fwd"
    dq, dk, dv = orc.bwd(q, k, v, do, off, func, 0.0, 11.0)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0), "alpha=0 bwd"
    # linear in v
    v2 = wl.normal_f32(v.shape, 52).astype(np.float64)
    o1 = orc.fwd(q, k, v, off, func, 0.5, 11.0)
    o2 = orc.fwd(q, k, v2, off, func, 0.5, 11.0)
    o12 = orc.fwd(q, k, v + 2.0 * v2, off, func, 0.5, 11.0)
    _close(o12, o1 + 2.0 * o2, rtol=1e-13, what="linearity in v")
    # large positive scores: silu(x) = x up to exp(-x) < 1e-17 and silu'(x) = 1,
    # so the op reduces to masked matrix products
    L = 10
    qa = 2.0 + np.abs(wl.normal_f32((L, 1, 3), 53).astype(np.float64))
    ka = 2.0 + np.abs(wl.normal_f32((L, 1, 3), 54).astype(np.float64))
    va = wl.normal_f32((L, 1, 3), 55).astype(np.float64)
    da = wl.normal_f32((L, 1, 3), 56).astype(np.float64)
    f = wl.func_sla(np.array([L]), 4, 2, 3)
    m = _dense_mask(np.array([L]), f)[0].astype(np.float64)
    alpha, max_len = 10.0, 5.0
    Q, K, V, G = qa[:, 0], ka[:, 0], va[:, 0], da[:, 0]
    P = alpha * (Q @ K.T) * m
    o = orc.fwd(qa, ka, va, np.array([0, L]), f, alpha, max_len)
    _close(o[:, 0], P @ V / max_len, rtol=1e-14, what="linear regime o")
    dq, dk, dv = orc.bwd(qa, ka, va, da, np.array([0, L]), f, alpha, max_len)
    dP = (G @ V.T) * m / max_len
    _close(dq[:, 0], alpha * dP @ K, rtol=1e-13, what="linear regime dq")
    _close(dk[:, 0], alpha * dP.T @ Q, rtol=1e-13, what="linear regime dk")
    _close(dv[:, 0], P.T @ G / max_len, rtol=1e-14, what="linear regime dv")
    # large negative scores: silu(x) -> 0 and silu'(x) -> 0
    o = orc.fwd(qa, -ka, va, np.array([0, L]), f, alpha, max_len)
    assert np.max(np.abs(o)) < 1e-30, "negative regime o"
    # a row with no visible column has zero outputs and zero gradient
    f0 = np.zeros((1, 4), dtype=np.int32)
    z = orc.fwd(qa[:4], ka[:4], va[:4], np.array([0, 4]), f0, 1.0, 1.0)
    assert np.all(z == 0.0)
    # empty batch entries and an all-empty batch
    lz = np.array([0, 0], dtype=np.int64)
    e = orc.fwd(np.zeros((0, 1, 3)), np.zeros((0, 1, 3)), np.zeros((0, 1, 3)),
                wl.offsets_from_lengths(lz), np.zeros((5, 0), dtype=np.int32), 1.0, 1.0)
    assert e.shape == (0, 1, 3)


PINS = [pin_hand_examples, pin_counts_closed_forms, pin_decode_bruteforce, pin_invariants,
        pin_autograd, pin_finite_differences, pin_special_cases]


def failing_pins(orc):
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except Exception as exc:  # a broken oracle may also raise on bad args
            failed.append(f"{pin.__name__}: {type(exc).__name__}: {str(exc)[:120]}")
    return failed


if __name__ == "__main__":
    import oracle

    lib = sys.argv[1] if len(sys.argv) > 1 else oracle.LIBRARY
    for line in failing_pins(oracle.Oracle(lib)):
        print(line)
