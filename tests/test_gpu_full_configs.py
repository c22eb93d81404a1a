"""GPU parity at the full workload sizes, through the same entry points and
launch configuration bench.py times.

Every output of a sequence (O, dQ, dK, dV of its rows) depends only on that
sequence's rows, so the oracle run on 32 whole sequences gives exact expected
values for them (the longest, the shortest, the median and the rest spread
over the batch); the small SLA workloads are checked in full, and the
targets-only mode on every candidate.  Both backward paths (recompute and
stored P) are checked on every shape whose timing is reported.
Visible counts are checked for every row against closed forms where the
mask has one, else against the oracle on the sampled sequences.
"""
import numpy as np
import pytest

import oracle
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


def device_inputs(cfg, targets=False):
    lengths = cfg["lengths"]
    off = wl.offsets_from_lengths(lengths)
    T = int(off[-1])
    B, H, D = len(lengths), cfg["H"], cfg["D"]
    seed = cfg["seed"]
    rq = B if targets else T
    dt = torch.bfloat16
    t = {
        "off": torch.from_numpy(off).to(DEV),
        "k": wl.normal_device((T, H, D), seed * 10 + 1, dt, DEV),
        "v": wl.normal_device((T, H, D), seed * 10 + 2, dt, DEV),
        "q": wl.normal_device((rq, H, D), seed * 10 + (5 if targets else 0), dt, DEV),
        "do": wl.normal_device((rq, H, D), seed * 10 + (6 if targets else 3), dt, DEV),
    }
    return t, off


def check(name, got, want):
    got = got.float().cpu().numpy().astype(np.float64)
    assert got.shape == want.shape, name
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    scale = float(np.max(np.abs(want))) if want.size else 0.0
    assert err <= 2e-2 * max(1.0, scale), f"{name}: max abs err {err:.3e}"
    assert err <= 2e-2 * scale, f"{name}: rel err {err / scale:.3e}"
    print(f"  {name}: max abs err {err:.3e}, rel {err / max(scale, 1e-30):.3e}", flush=True)


def to64(x):
    return x.float().cpu().numpy().astype(np.float64)


def run_full(hj, cfg, func_np, seqs, nfunc_label="", repeat=False, pstore=False, atomic=False):
    """fwd+bwd on the whole workload; oracle on the sequences `seqs`.  With
    `repeat`, a second fwd+bwd must reproduce every output bit for bit (each
    output element is written by one workgroup in a fixed order, so any
    difference is a race).  With `pstore`, the stored-P backward runs too (after
    the default one, on the same inputs) and is checked against the same
    oracle values, and its dk, dv must equal the default path's bit for bit;
    run over a buffer of about a seventh of the batch's stored P, in runs of
    sequences, it must reproduce its own outputs bit for bit.  With `atomic`,
    the atomic-dQ backward runs too: dk, dv bitwise the default path's, dq
    against the oracle."""
    t, off = device_inputs(cfg)
    func = torch.from_numpy(func_np).to(DEV)
    o = hj.attn_fwd(t["q"], t["k"], t["v"], t["off"], func, cfg["alpha"], cfg["max_len"])
    dq, dk, dv = hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], func, cfg["alpha"],
                             cfg["max_len"])
    if repeat:
        o2 = hj.attn_fwd(t["q"], t["k"], t["v"], t["off"], func, cfg["alpha"], cfg["max_len"])
        g2 = hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], func, cfg["alpha"],
                         cfg["max_len"])
        for nm, a, b in zip(("o", "dq", "dk", "dv"), (o, dq, dk, dv), (o2,) + tuple(g2)):
            assert torch.equal(a, b), f"{cfg['name']}.{nm}: second run differs"
        del o2, g2
    gp = None
    if pstore:
        ps = torch.empty(hj.pstore_bytes(t["off"], cfg["H"]), dtype=torch.uint8, device=DEV)
        gp = hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], func, cfg["alpha"],
                         cfg["max_len"], pstore=ps)
        if repeat:
            ps.fill_(0xFF)  # stale bytes must not reach dq
            gp2 = hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], func, cfg["alpha"],
                              cfg["max_len"], pstore=ps)
            for nm, a, b in zip(("dq", "dk", "dv"), gp, gp2):
                assert torch.equal(a, b), f"{cfg['name']}.pstore.{nm}: second run differs"
            del gp2
        # the same backward in runs of sequences sharing a buffer of about a
        # seventh of the batch's need: bit for bit the one-run outputs
        need = ps.numel()
        del ps
        per_seq = max(-(-int(L) // 128) * -(-int(L) // 32) * 8192 * cfg["H"]
                      for L in cfg["lengths"])
        budget = max(per_seq, need // 7) // 256 * 256 + 256
        ps = torch.empty(budget, dtype=torch.uint8, device=DEV)
        gc = hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], func, cfg["alpha"],
                         cfg["max_len"], pstore=ps, host_offsets=torch.from_numpy(off))
        for nm, a, b in zip(("dq", "dk", "dv"), gp, gc):
            assert torch.equal(a, b), f"{cfg['name']}.pstore chunked ({budget} B).{nm} differs"
        del ps, gc
        assert torch.equal(gp[1], dk) and torch.equal(gp[2], dv), "stored-P dk/dv differ"
    ga = None
    if atomic:
        ga = hj.attn_bwd_atomic(t["q"], t["k"], t["v"], t["do"], t["off"], func, cfg["alpha"],
                                cfg["max_len"])
        assert torch.equal(ga[1], dk) and torch.equal(ga[2], dv), "atomic-dQ dk/dv differ"
    torch.cuda.synchronize()
    rows, sub_off = oracle.subset(off, seqs)
    rows_t = torch.from_numpy(rows).to(DEV)
    pick = lambda x: to64(x.index_select(0, rows_t))  # noqa: E731
    q, k, v, do = (pick(t[n]) for n in ("q", "k", "v", "do"))
    f_sub = np.ascontiguousarray(func_np[:, rows])
    want_o = oracle.fwd(q, k, v, sub_off, f_sub, cfg["alpha"], cfg["max_len"])
    want = oracle.bwd(q, k, v, do, sub_off, f_sub, cfg["alpha"], cfg["max_len"])
    for nm, got, w in zip(("o", "dq", "dk", "dv"), (o, dq, dk, dv), (want_o,) + want):
        check(f"{cfg['name']}{nfunc_label}.{nm}", got.index_select(0, rows_t), w)
    if gp is not None:
        check(f"{cfg['name']}{nfunc_label}.pstore.dq", gp[0].index_select(0, rows_t), want[0])
    if ga is not None:
        check(f"{cfg['name']}{nfunc_label}.atomic.dq", ga[0].index_select(0, rows_t), want[0])
    return (o, dq, dk, dv), t, off


def sample_seqs(lengths, n=32):
    """n sequences: the longest, the shortest, the median, the rest spread
    evenly over the batch."""
    order = np.argsort(lengths, kind="stable")
    picks = {int(order[-1]), int(order[0]), int(order[len(order) // 2])}
    for i in np.linspace(0, len(lengths) - 1, n):
        if len(picks) >= n:
            break
        picks.add(int(i))
    return sorted(picks)


def test_sla_1k_full(hj):
    cfg = wl.workload("sla_1k")
    ls = cfg["lengths"]
    f = cfg["func"](ls, 5)
    run_full(hj, cfg, f, list(range(len(ls))))
    off_t = torch.from_numpy(wl.offsets_from_lengths(ls)).to(DEV)
    counts, tot = hj.visible_counts(off_t, torch.from_numpy(f).to(DEV), int(ls.sum()))
    i = wl.local_rows(ls)
    want = np.minimum(32, i + 1) + np.maximum(0, i + 1 - np.maximum(32, i - 255))
    assert np.array_equal(counts.cpu().numpy(), want)
    assert int(tot.item()) == 32 * 253584


def test_sla_2k_full_and_nfunc3_bitwise(hj):
    cfg = wl.workload("sla_2k")
    ls = cfg["lengths"]
    out5, t, off = run_full(hj, cfg, cfg["func"](ls, 5), list(range(len(ls))), atomic=True)
    f3 = torch.from_numpy(cfg["func"](ls, 3)).to(DEV)
    o3 = hj.attn_fwd(t["q"], t["k"], t["v"], t["off"], f3, cfg["alpha"], cfg["max_len"])
    g3 = hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], f3, cfg["alpha"], cfg["max_len"])
    for a, b in zip(out5, (o3,) + tuple(g3)):
        assert torch.equal(a, b), "nfunc=5 padded differs from nfunc=3"
    _, tot = hj.visible_counts(t["off"], f3, int(off[-1]))
    assert int(tot.item()) == 16 * 548496


@pytest.mark.parametrize("name", ["hstu_2663", "hstu_ragged", "hstu_4086"])
def test_hstu_layer_shapes_sampled(hj, name):
    """The production layer shapes: both backward paths (recompute and stored
    P, whose buffer is 59 / 60 / 137 GB here), 32 sequences against the
    oracle, every output repeated bit for bit, exact causal counts."""
    cfg = wl.workload(name)
    ls = cfg["lengths"]
    f = cfg["func"](ls, 5)
    run_full(hj, cfg, f, sample_seqs(ls), repeat=True, pstore=True, atomic=name == "hstu_2663")
    off_t = torch.from_numpy(wl.offsets_from_lengths(ls)).to(DEV)
    counts, tot = hj.visible_counts(off_t, torch.from_numpy(f).to(DEV), int(ls.sum()))
    assert np.array_equal(counts.cpu().numpy(), wl.local_rows(ls) + 1), "causal counts"
    assert int(tot.item()) == int(np.sum(ls * (ls + 1) // 2))
    torch.cuda.empty_cache()


def test_three_interval_sampled(hj):
    cfg = wl.workload("three_interval")
    ls = cfg["lengths"]
    f = cfg["func"](ls, 5)
    seqs = sample_seqs(ls)
    run_full(hj, cfg, f, seqs, pstore=True)
    off = wl.offsets_from_lengths(ls)
    off_t = torch.from_numpy(off).to(DEV)
    counts, _ = hj.visible_counts(off_t, torch.from_numpy(f).to(DEV), int(off[-1]))
    counts = counts.cpu().numpy()
    rows, sub_off = oracle.subset(off, seqs)
    want, _ = oracle.visible_counts(sub_off, np.ascontiguousarray(f[:, rows]))
    assert np.array_equal(counts[rows], want)


def test_onerank_sampled(hj):
    cfg = wl.workload("onerank")
    ls = cfg["lengths"]
    f = cfg["func"](ls, 5)
    seqs = sample_seqs(ls)
    run_full(hj, cfg, f, seqs, pstore=True)
    off = wl.offsets_from_lengths(ls)
    off_t = torch.from_numpy(off).to(DEV)
    counts, tot = hj.visible_counts(off_t, torch.from_numpy(f).to(DEV), int(off[-1]))
    H = ls - 240
    want = sum(int(h) * (int(h) + 1) // 2 + 60 * (int(h) + 1) + 180 * (int(h) + 2) for h in H)
    assert int(tot.item()) == want


def test_hstu_2663_targets_only_all_candidates(hj):
    """Targets-only at the production shape: o and dq of all 1024 candidates
    and dk, dv of every row of every sequence against the oracle (in chunks
    of 128 sequences)."""
    cfg = wl.workload("hstu_2663")
    ls = cfg["lengths"]
    f_np = cfg["func"](ls, 5)
    t, off = device_inputs(cfg, targets=True)
    func = torch.from_numpy(f_np).to(DEV)
    tr_np = wl.targets_last(ls)
    tr = torch.from_numpy(tr_np).to(DEV)
    o = hj.attn_fwd(t["q"], t["k"], t["v"], t["off"], func, cfg["alpha"], cfg["max_len"], tr)
    dq, dk, dv = hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], func, cfg["alpha"],
                             cfg["max_len"], tr)
    torch.cuda.synchronize()
    for c0 in range(0, len(ls), 128):
        seqs = list(range(c0, min(c0 + 128, len(ls))))
        rows, sub_off = oracle.subset(off, seqs)
        rows_t = torch.from_numpy(rows).to(DEV)
        seq_t = torch.tensor(seqs, device=DEV)
        k = to64(t["k"].index_select(0, rows_t))
        v = to64(t["v"].index_select(0, rows_t))
        q = to64(t["q"].index_select(0, seq_t))
        do = to64(t["do"].index_select(0, seq_t))
        f_sub = np.ascontiguousarray(f_np[:, rows])
        tr_sub = tr_np[seqs]
        want_o = oracle.fwd(q, k, v, sub_off, f_sub, cfg["alpha"], cfg["max_len"], tr_sub)
        wq, wk, wv = oracle.bwd(q, k, v, do, sub_off, f_sub, cfg["alpha"], cfg["max_len"],
                                tr_sub)
        for nm, got, want in (("o", o.index_select(0, seq_t), want_o),
                              ("dq", dq.index_select(0, seq_t), wq),
                              ("dk", dk.index_select(0, rows_t), wk),
                              ("dv", dv.index_select(0, rows_t), wv)):
            check(f"targets[{c0}:{c0 + len(seqs)}].{nm}", got, want)
    counts, tot = hj.visible_counts(t["off"], func, int(off[-1]), tr)
    assert np.array_equal(counts.cpu().numpy(), ls.astype(np.int32))
    assert int(tot.item()) == int(ls.sum())
