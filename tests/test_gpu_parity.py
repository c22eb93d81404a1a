"""GPU parity: the HIP path (through the C ABI binding) against the fp64 oracle.

Tolerances: fp32 inputs -> max|gpu - oracle| / max|oracle| <= 1e-5 per tensor;
bf16 inputs -> max|gpu - oracle| <= 2e-2 and, additionally, max|err| / max|ref|
<= 2e-2 per tensor (outputs of unit-scale inputs are ~1e-2 in size, so the
absolute bound alone would be weak).  The absolute bound is stated for outputs of
unit scale; cases whose outputs exceed 1 in magnitude (a tiny max_len) apply it
to err / max(1, max|ref|).  Visible counts are compared bit for bit.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def hj():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hstu_jagged_masked_amd as hj

    hj.library()  # raises if the HIP library was not built
    return hj


DEV = "cuda"


def make_inputs(lengths, H, D, dtype, seed, targets=None):
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    rows_q = len(lengths) if targets is not None else T
    out = {}
    for name, shape, s in (("q", (rows_q, H, D), seed), ("k", (T, H, D), seed + 1),
                           ("v", (T, H, D), seed + 2), ("do", (rows_q, H, D), seed + 3)):
        if dtype == "bf16":
            bits, vals = wl.normal_bf16(shape, s)
            t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
            out[name] = (t, vals.astype(np.float64))
        else:
            vals = wl.normal_f32(shape, s)
            out[name] = (torch.from_numpy(vals).to(DEV), vals.astype(np.float64))
    return out


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if want.size == 0:
        return 0.0, 0.0
    err = float(np.max(np.abs(got - want)))
    scale = float(np.max(np.abs(want)))
    return err, err / scale if scale > 0 else err


def assert_parity(name, got_t, want, dtype):
    got = got_t.float().cpu().numpy().astype(np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err, rel = rel_err(got, want)
    if dtype == "fp32":
        assert rel <= 1e-5, f"{name}: rel err {rel:.3e} (abs {err:.3e})"
    else:
        scale = float(np.max(np.abs(want))) if want.size else 0.0
        assert err <= 2e-2 * max(1.0, scale), f"{name}: max abs err {err:.3e}"
        assert rel <= 2e-2, f"{name}: rel err {rel:.3e} (abs {err:.3e})"
    return err, rel


def pstore_for(hj, off_t, H):
    return torch.empty(max(hj.pstore_bytes(off_t, H), 256), dtype=torch.uint8, device=DEV)


def run_case(hj, lengths, H, D, dtype, func, alpha, max_len, seed=7, targets=None, bwd=True,
             pstore=False):
    lengths = np.asarray(lengths, dtype=np.int64)
    off = wl.offsets_from_lengths(lengths)
    inp = make_inputs(lengths, H, D, dtype, seed, targets)
    off_t = torch.from_numpy(off).to(DEV)
    func_t = torch.from_numpy(np.ascontiguousarray(func)).to(DEV)
    tr_t = None if targets is None else torch.from_numpy(np.asarray(targets, np.int32)).to(DEV)
    (q, qn), (k, kn), (v, vn), (do, don) = inp["q"], inp["k"], inp["v"], inp["do"]
    o = hj.attn_fwd(q, k, v, off_t, func_t, alpha, max_len, tr_t)
    torch.cuda.synchronize()
    want_o = oracle.fwd(qn, kn, vn, off, func, alpha, max_len, targets)
    res = {"o": assert_parity("o", o, want_o, dtype)}
    if bwd:
        ps = pstore_for(hj, off_t, q.shape[1]) if pstore else None
        dq, dk, dv = hj.attn_bwd(q, k, v, do, off_t, func_t, alpha, max_len, tr_t, pstore=ps)
        torch.cuda.synchronize()
        wq, wk, wv = oracle.bwd(qn, kn, vn, don, off, func, alpha, max_len, targets)
        res["dq"] = assert_parity("dq", dq, wq, dtype)
        res["dk"] = assert_parity("dk", dk, wk, dtype)
        res["dv"] = assert_parity("dv", dv, wv, dtype)
    counts, total = hj.visible_counts(off_t, func_t, int(off[-1]), tr_t)
    want_c, want_total = oracle.visible_counts(off, func, targets)
    assert np.array_equal(counts.cpu().numpy(), want_c), "visible counts differ"
    assert int(total.item()) == want_total, "total pairs differ"
    return res


# --- the small fp32 configuration: B=2 lengths 37 and 64, H=2, D=32 --------


def test_tiny_fp32_causal(hj):
    cfg = wl.workload("tiny_fp32")
    ls = cfg["lengths"]
    run_case(hj, ls, cfg["H"], cfg["D"], "fp32", cfg["func"](ls), cfg["alpha"], cfg["max_len"],
             seed=1)


def test_tiny_fp32_targets_only(hj):
    cfg = wl.workload("tiny_fp32")
    ls = cfg["lengths"]
    run_case(hj, ls, cfg["H"], cfg["D"], "fp32", cfg["func"](ls), cfg["alpha"], cfg["max_len"],
             seed=1, targets=wl.targets_last(ls))


@pytest.mark.parametrize("D", [32, 64, 128])
def test_fp32_random_func(hj, D):
    ls = np.array([5, 0, 40, 1, 70])
    run_case(hj, ls, 3, D, "fp32", wl.func_random(ls, 7, 99, spread=6), 0.2, 70, seed=3)


# --- bf16 ----------------------------------------------------------------

RAGGED = [1, 37, 64, 130, 257, 300, 0, 129]


@pytest.mark.parametrize("D", [32, 64, 128])
def test_bf16_causal_ragged(hj, D):
    ls = np.array(RAGGED)
    run_case(hj, ls, 2, D, "bf16", wl.func_causal(ls, 5), 1 / np.sqrt(D), int(ls.max()), seed=11)


def test_bf16_sla_nfunc5_equals_nfunc3(hj):
    ls = np.array([600, 333, 1000])
    H, D = 2, 128
    r5 = run_case(hj, ls, H, D, "bf16", wl.func_sla(ls, 256, 32, 5), 1 / np.sqrt(D), 1000,
                  seed=12)
    r3 = run_case(hj, ls, H, D, "bf16", wl.func_sla(ls, 256, 32, 3), 1 / np.sqrt(D), 1000,
                  seed=12)
    for key in r5:
        assert r5[key] == r3[key], f"{key}: nfunc=5 and nfunc=3 differ"


def test_bf16_sla_padded_bitwise(hj):
    """Padding empty intervals onto the 2-interval func gives identical bits."""
    ls = np.array([700, 128, 900])
    H, D = 2, 128
    off = wl.offsets_from_lengths(ls)
    inp = make_inputs(ls, H, D, "bf16", 13)
    off_t = torch.from_numpy(off).to(DEV)
    outs = []
    for nf in (3, 5, 9):
        f = torch.from_numpy(wl.func_sla(ls, 256, 32, nf)).to(DEV)
        o = hj.attn_fwd(inp["q"][0], inp["k"][0], inp["v"][0], off_t, f, 0.09, 900)
        g = hj.attn_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t, f, 0.09, 900)
        outs.append((o,) + tuple(g))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    for a, b in zip(outs[0], outs[2]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("mask", ["causal", "sla"])
def test_bf16_long_sequences_several_list_windows(hj, mask):
    """Sequences past 64 row blocks / key tiles (4096 rows): the kernels walk
    their tile lists in several windows of 64 blocks."""
    ls = np.array([4700, 130, 4160])
    f = wl.func_causal(ls, 5) if mask == "causal" else wl.func_sla(ls, 1200, 32, 5)
    run_case(hj, ls, 1, 128, "bf16", f, 1 / np.sqrt(128), 4700, seed=21)


def test_bf16_three_interval(hj):
    ls = np.array([300, 520, 270, 100])
    run_case(hj, ls, 2, 128, "bf16", wl.func_three_interval(ls, 32, 8, 5), 1 / np.sqrt(128),
             520, seed=14)


def test_bf16_onerank(hj):
    """OneRank task-private masks: history, then candidate + 3 task tokens per
    group; each task token sees the history, its candidate and itself."""
    n_cand = np.array([8, 4, 60, 1, 30])
    ls = wl.onerank_lengths([100, 2, 1968, 0, 300], n_cand, 3)
    run_case(hj, ls, 2, 128, "bf16", wl.func_onerank(ls, n_cand, 3, 5), 1 / np.sqrt(128),
             int(ls.max()), seed=22)


@pytest.mark.parametrize("nfunc", [1, 3, 5, 9])
def test_bf16_random_func(hj, nfunc):
    ls = np.array([5, 0, 77, 200, 64, 65])
    run_case(hj, ls, 2, 128, "bf16", wl.func_random(ls, nfunc, 100 + nfunc, spread=20), 0.1, 200,
             seed=15)


@pytest.mark.parametrize("path", ["default", "pstore", "targets"])
def test_bf16_max_heads(hj, path):
    """The largest head count the library accepts (255): row strides of
    255 * 128 * 2 bytes, ragged lengths with partial tiles, a random mask."""
    ls = np.array([130, 1, 257, 0, 64])
    f = wl.func_random(ls, 5, 255, spread=12)
    tr = wl.targets_last(ls) if path == "targets" else None
    run_case(hj, ls, 255, 128, "bf16", f, 0.09, 257, seed=255, targets=tr,
             pstore=path == "pstore")


def test_bf16_targets_only(hj):
    ls = np.array([300, 1, 129, 700, 0, 64])
    tr = np.array([299, 0, 5, 699, 0, 63], dtype=np.int32)
    run_case(hj, ls, 4, 128, "bf16", wl.func_causal(ls, 5), 1 / np.sqrt(128), 700, seed=16,
             targets=tr)


def test_bf16_targets_only_sla(hj):
    ls = np.array([1000, 513, 64])
    run_case(hj, ls, 2, 128, "bf16", wl.func_sla(ls, 256, 32, 5), 1 / np.sqrt(128), 1000,
             seed=17, targets=wl.targets_last(ls))


def test_empty_and_single_rows(hj):
    run_case(hj, np.array([1]), 1, 128, "bf16", wl.func_causal([1], 5), 0.5, 1, seed=18)
    run_case(hj, np.array([0, 3, 0]), 1, 128, "bf16", wl.func_causal([0, 3, 0], 5), 0.5, 3,
             seed=19)
    run_case(hj, np.array([0, 0]), 2, 64, "bf16", np.zeros((5, 0), np.int32), 0.5, 1, seed=20)


def test_unseen_key_rows_get_zero_grad(hj):
    """Key rows no query sees must come back with dK = dV = 0 exactly: every
    row sees [0, min(i+1, 50)), so local columns >= 50 are never seen."""
    ls = np.array([200, 150, 30])
    local = wl.local_rows(ls)
    f = np.minimum(local + 1, 50).astype(np.int32)[None, :]
    H, D = 2, 128
    inp = make_inputs(ls, H, D, "bf16", 21)
    off_t = torch.from_numpy(wl.offsets_from_lengths(ls)).to(DEV)
    dq, dk, dv = hj.attn_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t,
                             torch.from_numpy(f).to(DEV), 0.1, 200)
    unseen = torch.from_numpy(local >= 50).to(DEV)
    seen = ~unseen
    assert int(unseen.sum()) == 150 + 100
    assert torch.all(dk[unseen] == 0) and torch.all(dv[unseen] == 0)
    assert torch.any(dk[seen] != 0) and torch.any(dv[seen] != 0)


def test_dk_dv_bitwise_repeatable(hj):
    ls = np.array([700, 300, 1000, 64])
    H, D = 2, 128
    off = wl.offsets_from_lengths(ls)
    inp = make_inputs(ls, H, D, "bf16", 22)
    off_t = torch.from_numpy(off).to(DEV)
    ft = torch.from_numpy(wl.func_causal(ls, 5)).to(DEV)
    ref = hj.attn_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t, ft, 0.09, 1000)
    for _ in range(10):
        g = hj.attn_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t, ft, 0.09,
                        1000)
        for a, b in zip(ref, g):
            assert torch.equal(a, b)


def test_stored_p_bitwise_repeatable(hj):
    """The stored-P backward (P written by the key-owner pass, dQ from it)
    gives the same bits on every replay, dQ included."""
    ls = np.array([700, 300, 1000, 64])
    H, D = 2, 128
    off = wl.offsets_from_lengths(ls)
    inp = make_inputs(ls, H, D, "bf16", 23)
    off_t = torch.from_numpy(off).to(DEV)
    ft = torch.from_numpy(wl.func_causal(ls, 5)).to(DEV)
    ps = torch.empty(hj.pstore_bytes(off_t, H), dtype=torch.uint8, device=DEV)
    args = (inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t, ft, 0.09, 1000)
    ref = hj.attn_bwd(*args, pstore=ps)
    for _ in range(10):
        ps.fill_(0xFF)  # stale bytes from an earlier call must not leak into dQ
        g = hj.attn_bwd(*args, pstore=ps)
        for a, b in zip(ref, g):
            assert torch.equal(a, b)


ATOMIC_CASES = {
    "causal_ragged": ([700, 1, 300, 0, 1000, 64, 129], 3, lambda ls: wl.func_causal(ls, 5)),
    "long_windows": ([4700, 300], 1, lambda ls: wl.func_causal(ls, 5)),
    "sla": ([1024, 777, 2048], 2, lambda ls: wl.func_sla(ls, 256, 32, 5)),
    "random_nfunc9": ([500, 333, 64], 2, lambda ls: wl.func_random(ls, 9, 91, spread=20)),
    "three_interval": ([900, 611], 2, lambda ls: wl.func_three_interval(ls, 16, 8, 5)),
}


@pytest.mark.parametrize("case", sorted(ATOMIC_CASES))
def test_bf16_atomic_dq(hj, case):
    """The atomic-dQ backward (dQ added with fp32 atomics by the key-owner
    pass): dq within the bf16 bound of the oracle and close to attn_bwd's, dk
    and dv bitwise those of attn_bwd (the same key-owner arithmetic), and the
    accumulator's previous contents (NaN here) never reach dq."""
    lengths, H, make_func = ATOMIC_CASES[case]
    ls = np.asarray(lengths, dtype=np.int64)
    f = make_func(ls)
    off = wl.offsets_from_lengths(ls)
    inp = make_inputs(ls, H, 128, "bf16", 31)
    (q, qn), (k, kn), (v, vn), (do, don) = inp["q"], inp["k"], inp["v"], inp["do"]
    off_t = torch.from_numpy(off).to(DEV)
    ft = torch.from_numpy(np.ascontiguousarray(f)).to(DEV)
    alpha, max_len = 0.11, int(ls.max()) + 1
    args = (q, k, v, do, off_t, ft, alpha, max_len)
    acc = torch.full((int(off[-1]), H, 128), float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = hj.attn_bwd_atomic(*args, dq_accum=acc)
    rq, rk, rv = hj.attn_bwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(dk, rk) and torch.equal(dv, rv)
    wq, _, _ = oracle.bwd(qn, kn, vn, don, off, f, alpha, max_len, None)
    assert_parity("dq", dq, wq, "bf16")
    scale = max(1.0, float(rq.float().abs().max().item()))
    assert float((dq.float() - rq.float()).abs().max().item()) <= 2e-2 * scale


@pytest.mark.parametrize("targets", [False, True])
def test_autograd_wrapper_matches_entry_points(hj, targets):
    """hstu_attention (torch.autograd.Function): the forward and the gradients
    autograd hands back are bitwise those of attn_fwd / attn_bwd."""
    ls = np.array([200, 0, 77, 131])
    off = wl.offsets_from_lengths(ls)
    off_t = torch.from_numpy(off).to(DEV)
    f = torch.from_numpy(wl.func_sla(ls, 64, 16, 5)).to(DEV)
    tr = torch.from_numpy(wl.targets_last(ls)).to(DEV) if targets else None
    inp = make_inputs(ls, 2, 128, "bf16", 41, wl.targets_last(ls) if targets else None)
    q, k, v, do = (inp[n][0] for n in ("q", "k", "v", "do"))
    o_ref = hj.attn_fwd(q, k, v, off_t, f, 0.1, 200, tr)
    g_ref = hj.attn_bwd(q, k, v, do, off_t, f, 0.1, 200, tr)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = hj.hstu_attention(qa, ka, va, off_t, f, 0.1, 200, tr)
    o.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for nm, got, want in zip(("dq", "dk", "dv"), (qa.grad, ka.grad, va.grad), g_ref):
        assert torch.equal(got, want), nm
    if targets:
        return
    # the stored-P backward through autograd, over a whole-batch and a small buffer
    ps = pstore_for(hj, off_t, 2)
    g_p = hj.attn_bwd(q, k, v, do, off_t, f, 0.1, 200, pstore=ps)
    small = torch.empty(max(-(-int(L) // 128) * -(-int(L) // 32) * 8192 * 2 for L in ls),
                        dtype=torch.uint8, device=DEV)
    for buf, host in ((ps, None), (small, torch.from_numpy(off))):
        qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
        hj.hstu_attention(qa, ka, va, off_t, f, 0.1, 200, pstore=buf,
                          host_offsets=host).backward(do)
        torch.cuda.synchronize()
        for nm, got, want in zip(("dq", "dk", "dv"), (qa.grad, ka.grad, va.grad), g_p):
            assert torch.equal(got, want), "stored-P " + nm


def random_case(seed):
    """One random configuration: 1-8 sequences of 0-700 rows (empty, single-row
    and every tail residue occur), 1-5 heads, a causal, SLA, three-interval or
    arbitrary-bounds mask with nfunc 1-9, random alpha and max_len, and one of
    the paths (default, stored P, stored P in runs over a small buffer,
    targets-only with random candidates)."""
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    B = int(rng.integers(1, 9))
    ls = rng.integers(0, 701, size=B)
    ls[rng.random(B) < 0.15] = 0
    ls[rng.random(B) < 0.1] = 1
    H = int(rng.integers(1, 6))
    kind = ["causal", "sla", "three", "random"][int(rng.integers(0, 4))]
    if kind == "random":
        nfunc = int(rng.choice([1, 3, 5, 7, 9]))
    else:
        nfunc = int(rng.choice([5, 9] if kind == "three" else [3, 5, 9]))
    if kind == "causal":
        f = wl.func_causal(ls, nfunc)
    elif kind == "sla":
        f = wl.func_sla(ls, int(rng.integers(1, 400)), int(rng.integers(0, 64)), nfunc)
    elif kind == "three":
        f = wl.func_three_interval(ls, int(rng.integers(1, 40)), int(rng.integers(1, 12)), nfunc)
    else:
        f = wl.func_random(ls, nfunc, 2000 + seed, spread=int(rng.integers(1, 40)))
    alpha = float(rng.uniform(0.02, 0.3))
    max_len = int(max(1, ls.max()) * rng.uniform(0.5, 2.0)) + 1
    path = ["default", "pstore", "runs", "targets"][int(rng.integers(0, 4))]
    tr = None
    if path == "targets":
        tr = np.array([int(rng.integers(0, L)) if L > 0 else 0 for L in ls], np.int32)
    return ls, H, f, alpha, max_len, path, tr


SWEEP_CASES = int(os.environ.get("HSTU_SWEEP_CASES", "12"))


@pytest.mark.parametrize("seed", range(SWEEP_CASES))
def test_random_sweep(hj, seed):
    """Random configurations against the oracle (HSTU_SWEEP_CASES sets how
    many); the stored-P runs path must also reproduce the whole-buffer one
    bitwise."""
    ls, H, f, alpha, max_len, path, tr = random_case(seed)
    print(f"seed {seed}: lengths {ls.tolist()} H {H} nfunc {f.shape[0]} path {path}", flush=True)
    run_case(hj, ls, H, 128, "bf16", f, alpha, max_len, seed=3000 + seed, targets=tr,
             pstore=path in ("pstore", "runs"))
    if path == "runs":
        off = wl.offsets_from_lengths(ls)
        off_t = torch.from_numpy(off).to(DEV)
        inp = make_inputs(ls, H, 128, "bf16", 3000 + seed)
        args = (inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t,
                torch.from_numpy(np.ascontiguousarray(f)).to(DEV), alpha, max_len)
        ref = hj.attn_bwd(*args, pstore=pstore_for(hj, off_t, H))
        per_seq = max(-(-int(L) // 128) * -(-int(L) // 32) * 8192 * H for L in ls)
        buf = torch.empty(max(per_seq, 256), dtype=torch.uint8, device=DEV)
        got = hj.attn_bwd(*args, pstore=buf, host_offsets=torch.from_numpy(off))
        torch.cuda.synchronize()
        for a, b, nm in zip(ref, got, ("dq", "dk", "dv")):
            assert torch.equal(a, b), f"runs path {nm} differs"


@pytest.mark.parametrize("seed", range(max(4, SWEEP_CASES // 2)))
def test_random_sweep_atomic(hj, seed):
    """The atomic-dQ backward on the sweep's full-length configurations: dq
    against the oracle, dk and dv bitwise those of attn_bwd."""
    ls, H, f, alpha, max_len, path, _ = random_case(seed)
    print(f"seed {seed}: lengths {ls.tolist()} H {H} nfunc {f.shape[0]}", flush=True)
    off = wl.offsets_from_lengths(ls)
    off_t = torch.from_numpy(off).to(DEV)
    inp = make_inputs(ls, H, 128, "bf16", 5000 + seed)
    (q, qn), (k, kn), (v, vn), (do, don) = inp["q"], inp["k"], inp["v"], inp["do"]
    args = (q, k, v, do, off_t, torch.from_numpy(np.ascontiguousarray(f)).to(DEV), alpha, max_len)
    dq, dk, dv = hj.attn_bwd_atomic(*args)
    _, rk, rv = hj.attn_bwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(dk, rk) and torch.equal(dv, rv)
    wq, _, _ = oracle.bwd(qn, kn, vn, don, off, f, alpha, max_len, None)
    assert_parity("dq", dq, wq, "bf16")


@pytest.mark.parametrize("seed", range(max(4, SWEEP_CASES // 2)))
def test_random_sweep_generic(hj, seed):
    """The plain-FMA kernels (fp32 at D = 32, 64, 128; bf16 at D = 32, 64) on
    random configurations against the oracle, full-length and targets-only."""
    ls, H, f, alpha, max_len, path, tr = random_case(10000 + seed)
    rng = np.random.Generator(np.random.PCG64(20000 + seed))
    dtype, D = [("fp32", 32), ("fp32", 64), ("fp32", 128), ("bf16", 32), ("bf16", 64)][
        int(rng.integers(0, 5))]
    ls = np.minimum(ls, 300)  # the plain kernels are slow; keep the case small
    f = random_case_func(ls, f.shape[0], seed)
    tr = None if path != "targets" else np.array(
        [int(rng.integers(0, L)) if L > 0 else 0 for L in ls], np.int32)
    print(f"seed {seed}: {dtype} D {D} lengths {ls.tolist()} H {H} targets {tr is not None}",
          flush=True)
    run_case(hj, ls, H, D, dtype, f, alpha, max_len, seed=4000 + seed, targets=tr)


def random_case_func(ls, nfunc, seed):
    return wl.func_random(ls, nfunc, 5000 + seed, spread=12)


def test_graph_capture_replays(hj):
    """fwd + stored-P bwd captured once in a HIP graph (the entry points only
    enqueue kernels: no memset, copy, allocation or synchronization inside),
    replayed with new inputs and eager work between the replays: every
    replay equals the eager result bitwise."""
    ls = np.array([300, 1, 0, 129])
    H = 2
    off = wl.offsets_from_lengths(ls)
    off_t = torch.from_numpy(off).to(DEV)
    f = torch.from_numpy(wl.func_sla(ls, 96, 8, 5)).to(DEV)
    static = [make_inputs(ls, H, 128, "bf16", 60)[n][0].clone() for n in ("q", "k", "v", "do")]
    ps = pstore_for(hj, off_t, H)

    def step(q, k, v, do):
        o = hj.attn_fwd(q, k, v, off_t, f, 0.1, 300)
        return (o,) + tuple(hj.attn_bwd(q, k, v, do, off_t, f, 0.1, 300, pstore=ps))

    step(*static)  # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(*static)
    for rep in range(4):
        fresh = [make_inputs(ls, H, 128, "bf16", 61 + rep)[n][0] for n in ("q", "k", "v", "do")]
        for dst, src in zip(static, fresh):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        want = step(*fresh)  # eager, between the replays
        torch.cuda.synchronize()
        for nm, a, b in zip(("o", "dq", "dk", "dv"), got, want):
            assert torch.equal(a, b), f"replay {rep}: {nm} differs from eager"


def test_check_inputs(hj):
    off = torch.tensor([0, 3, 7], dtype=torch.int64, device=DEV)
    hj.check_inputs(off, 7)
    hj.check_inputs(off, 7, torch.tensor([2, 3], dtype=torch.int32, device=DEV))
    with pytest.raises(hj.HstuError, match="seq_offsets\\[B\\] != total"):
        hj.check_inputs(off, 8)
    with pytest.raises(hj.HstuError, match="decreasing"):
        hj.check_inputs(torch.tensor([0, 5, 3, 7], dtype=torch.int64, device=DEV), 7)
    with pytest.raises(hj.HstuError, match="target row"):
        hj.check_inputs(off, 7, torch.tensor([3, 0], dtype=torch.int32, device=DEV))


def test_malformed_offsets_stay_in_bounds(hj):
    """Garbage offsets give garbage but no fault: kernels clamp them."""
    ls = np.array([100, 50])
    inp = make_inputs(ls, 2, 128, "bf16", 23)
    bad = torch.tensor([5, 400, -7], dtype=torch.int64, device=DEV)
    ft = torch.from_numpy(wl.func_causal(ls, 5)).to(DEV)
    o = hj.attn_fwd(inp["q"][0], inp["k"][0], inp["v"][0], bad, ft, 0.1, 100)
    g = hj.attn_bwd(inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], bad, ft, 0.1, 100)
    torch.cuda.synchronize()
    assert o.shape == inp["q"][0].shape and g[0].shape == o.shape


# --- the stored-P backward (bf16, D = 128) ------------------------------------

PSTORE_CASES = {
    "causal_ragged": (RAGGED, lambda ls: wl.func_causal(ls, 5), 1 / np.sqrt(128), 300),
    "sla": ([600, 333, 1000], lambda ls: wl.func_sla(ls, 256, 32, 5), 1 / np.sqrt(128), 1000),
    "three_interval": ([300, 520, 270, 100], lambda ls: wl.func_three_interval(ls, 32, 8, 5),
                       1 / np.sqrt(128), 520),
    "random_nfunc9": ([5, 0, 77, 200, 64, 65], lambda ls: wl.func_random(ls, 9, 109, spread=20),
                      0.1, 200),
    "long_windows": ([4700, 130, 4160], lambda ls: wl.func_sla(ls, 1200, 32, 5),
                     1 / np.sqrt(128), 4700),
    "single_rows": ([1, 0, 3, 0], lambda ls: wl.func_causal(ls, 5), 0.5, 3),
    "onerank": (list(wl.onerank_lengths([100, 2, 1968, 300], [8, 4, 60, 30], 3)),
                lambda ls: wl.func_onerank(ls, [8, 4, 60, 30], 3, 5), 1 / np.sqrt(128), 2208),
}


@pytest.mark.parametrize("name", sorted(PSTORE_CASES))
def test_bf16_pstore_backward(hj, name):
    lengths, fn, alpha, max_len = PSTORE_CASES[name]
    ls = np.array(lengths)
    H = 1 if name == "long_windows" else 2
    run_case(hj, ls, H, 128, "bf16", fn(ls), alpha, max_len, seed=31, pstore=True)


def test_bf16_pstore_dk_dv_bitwise_equal_recompute_path(hj):
    """The stored-P key-owner pass computes dK and dV exactly as the default
    one (it only adds the stores); dQ comes from another kernel."""
    ls = np.array([700, 128, 900, 1, 0])
    off = wl.offsets_from_lengths(ls)
    off_t = torch.from_numpy(off).to(DEV)
    inp = make_inputs(ls, 4, 128, "bf16", 33)
    f = torch.from_numpy(wl.func_sla(ls, 256, 32, 5)).to(DEV)
    args = (inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t, f, 0.09, 900)
    dq0, dk0, dv0 = hj.attn_bwd(*args)
    dq1, dk1, dv1 = hj.attn_bwd(*args, pstore=pstore_for(hj, off_t, 4))
    dq2, dk2, dv2 = hj.attn_bwd(*args, pstore=pstore_for(hj, off_t, 4))
    assert torch.equal(dk0, dk1) and torch.equal(dv0, dv1)
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    err = (dq0.float() - dq1.float()).abs().max().item()
    assert err <= 2e-2 * dq0.float().abs().max().item()


@pytest.mark.parametrize("name", ["causal_ragged", "random_nfunc9", "onerank", "sla",
                                  "single_rows"])
def test_bf16_pstore_chunked_bitwise(hj, name):
    """The stored-P backward cut into runs of sequences that share one smaller
    buffer gives bitwise the outputs of one run over a buffer for the whole
    batch, at budgets from the largest sequence's need (most runs) up to the
    whole batch; every P access stays inside the budget (a guard region after
    it keeps its bytes)."""
    lengths, fn, alpha, max_len = PSTORE_CASES[name]
    # empty sequences at the ends (not for OneRank, whose mask follows its layout)
    ls = np.array(list(lengths) if name == "onerank" else [0] + list(lengths) + [0, 0])
    H = 2
    off = wl.offsets_from_lengths(ls)
    off_t = torch.from_numpy(off).to(DEV)
    inp = make_inputs(ls, H, 128, "bf16", 35)
    f = torch.from_numpy(fn(ls)).to(DEV)
    args = (inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t, f, alpha, max_len)
    need = hj.pstore_bytes(off_t, H)
    ref = hj.attn_bwd(*args, pstore=pstore_for(hj, off_t, H))
    per_seq = [-(-int(L) // 128) * -(-int(L) // 32) * 8192 * H for L in ls]
    for budget in sorted({max(per_seq), max(max(per_seq), need // 2), need}):
        budget = max(budget, 256)
        buf = torch.full((budget + (64 << 10),), 0x5A, dtype=torch.uint8, device=DEV)
        got = hj.attn_bwd(*args, pstore=buf[:budget], host_offsets=torch.from_numpy(off))
        torch.cuda.synchronize()
        for r, g, nm in zip(ref, got, ("dq", "dk", "dv")):
            assert torch.equal(r, g), f"{name} budget {budget}: {nm} differs"
        assert bool((buf[budget:] == 0x5A).all()), f"{name} budget {budget}: guard overwritten"


def test_bf16_pstore_buffer_too_small(hj):
    """A stored-P buffer smaller than the device offsets need: the call does
    not synchronize to find out; every P access stays inside the buffer (a
    guard region after it keeps its bytes), dk and dv are still exact and dq
    comes back as NaN."""
    ls = np.array([300, 200])
    off_t = torch.from_numpy(wl.offsets_from_lengths(ls)).to(DEV)
    inp = make_inputs(ls, 2, 128, "bf16", 34)
    f = torch.from_numpy(wl.func_causal(ls, 5)).to(DEV)
    need = hj.pstore_bytes(off_t, 2)
    assert need == (3 * 10 + 2 * 7) * 2 * 8192
    short = need - 8192
    buf = torch.full((need + (64 << 10),), 0x5A, dtype=torch.uint8, device=DEV)
    args = (inp["q"][0], inp["k"][0], inp["v"][0], inp["do"][0], off_t, f, 0.1, 300)
    dq, dk, dv = hj.attn_bwd(*args, pstore=buf[:short])
    torch.cuda.synchronize()
    assert bool((buf[short:] == 0x5A).all()), "a P access left the buffer"
    assert bool(torch.isnan(dq.float()).all())
    dq0, dk0, dv0 = hj.attn_bwd(*args)
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
