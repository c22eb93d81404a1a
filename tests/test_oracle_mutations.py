"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The mistakes are planted in the oracle's C source on the CPU (a copy, built into
a temporary directory); the pins run in a child process so that a mutant that
crashes cannot take the test runner with it.  A crash counts as detected.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("drop_last_interval", "j <= (nfunc - 1) / 2", "j < (nfunc - 1) / 2"),
    ("interval_end_inclusive", "for (int64_t c = lo; c < hi; ++c)", "for (int64_t c = lo; c <= hi && c < L; ++c)"),
    ("clip_end_off_by_one", "if (hi > L) hi = L;", "if (hi > L) hi = L - 1;"),
    ("reversed_pair_swapped", "if (hi <= lo) return; /* empty pair: skipped */",
     "if (hi < lo) { int64_t t = lo; lo = hi; hi = t; }"),
    ("start_not_clipped_to_zero", "if (lo < 0) lo = 0;", "if (lo < 0) lo = -lo;"),
    ("pairs_shifted", "(int64_t)(2 * j - 1) * total", "(int64_t)(2 * j - 2) * total"),
    ("alpha_after_silu", "silu(alpha * dot) / max_len", "alpha * silu(dot) / max_len"),
    ("sigmoid_not_silu", "static double silu(double x) { return x * logistic(x); }",
     "static double silu(double x) { return logistic(x); }"),
    ("no_max_len_fwd", "double s = silu(alpha * dot) / max_len;\n          for (int d = 0; d < D; ++d) oi",
     "double s = silu(alpha * dot);\n          for (int d = 0; d < D; ++d) oi"),
    ("silu_grad_sign", "x * (1.0 - s)", "x * (1.0 + s)"),
    ("silu_grad_no_one", "s * (1.0 + x * (1.0 - s))", "s * (x * (1.0 - s))"),
    ("dp_no_max_len", "double dp = ds * silu_grad(p) / max_len;", "double dp = ds * silu_grad(p);"),
    ("dk_uses_k", "dk[kr + d] += alpha * dp * qi[d];", "dk[kr + d] += alpha * dp * kc[d];"),
    ("dq_uses_q", "dqi[d] += alpha * dp * kc[d];", "dqi[d] += alpha * dp * qi[d];"),
    ("dq_no_alpha", "dqi[d] += alpha * dp * kc[d];", "dqi[d] += dp * kc[d];"),
    ("dv_uses_dp", "dv[kr + d] += s * doi[d];", "dv[kr + d] += dp * doi[d];"),
    ("ds_uses_k", "ds += doi[d] * vc[d];", "ds += doi[d] * kc[d];"),
    ("bwd_recompute_uses_v", "for (int d = 0; d < D; ++d) dot += qi[d] * kc[d];\n          for (int d = 0; d < D; ++d) ds",
     "for (int d = 0; d < D; ++d) dot += qi[d] * vc[d];\n          for (int d = 0; d < D; ++d) ds"),
    ("targets_func_column_local", "decode_row(func, nfunc, total, off[b] + i, L, mark);\n        for (int64_t c = 0; c < L; ++c) {\n          if (!mark[c]) continue;\n          const double* kc",
     "decode_row(func, nfunc, total, target_rows ? i : off[b] + i, L, mark);\n        for (int64_t c = 0; c < L; ++c) {\n          if (!mark[c]) continue;\n          const double* kc"),
    ("column_offset_missing", "const double* kc = k + ((off[b] + c) * H + h) * D;", "const double* kc = k + (c * H + h) * D;"),
    ("head_ignored_fwd", "const double* qi = q + (qrow * H + h) * D;\n        double* oi", "const double* qi = q + (qrow * H) * D;\n        double* oi"),
]


def test_mutations_apply_once():
    src = open(oracle.SOURCE).read()
    for name, old, _ in MUTATIONS:
        assert src.count(old) == 1, f"{name}: pattern found {src.count(old)} times"


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, mutation):
    name, old, new = mutation
    src = open(oracle.SOURCE).read().replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = str(tmp_path / "libmutant.so")
    oracle.compile_library(str(path), lib, werror=False)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                          capture_output=True, text=True, timeout=600)
    detected = proc.returncode != 0 or proc.stdout.strip() != ""
    assert detected, f"mutation {name} passed every pin"


def test_unmutated_oracle_passes_in_child(tmp_path):
    lib = str(tmp_path / "libclean.so")
    oracle.compile_library(oracle.SOURCE, lib)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                          capture_output=True, text=True, timeout=600)
    assert proc.returncode == 0 and proc.stdout.strip() == "", proc.stdout + proc.stderr
