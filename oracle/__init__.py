"""fp64 CPU oracle for HSTU jagged masked attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
package imports nothing from the product path.

The arithmetic lives in ``hstu_oracle.c`` (plain loops over rows and columns in
double precision); this module compiles it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "hstu_oracle.c")
LIBRARY = os.path.join(_HERE, "libhstu_oracle.so")

_ERRORS = {-1: "bad arguments", -2: "bad seq_offsets", -3: "target row out of range",
           -4: "out of memory"}


def compile_library(source: str = SOURCE, output: str = LIBRARY, werror: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           *(["-Werror"] if werror else []), source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(output + ".tmp", output)
    return output


def _stale(lib: str, src: str) -> bool:
    return not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src)


class Oracle:
    """ctypes front end over one build of the oracle library."""

    def __init__(self, library: str = LIBRARY):
        if library == LIBRARY and _stale(LIBRARY, SOURCE):
            compile_library()
        self.path = library
        self._lib = ctypes.CDLL(library)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        self._lib.oracle_visible_counts.argtypes = [P, i64, i64, P, i32, P, P, P]
        self._lib.oracle_fwd.argtypes = [P, P, P, P, P, i64, i64, i32, i32, P, i32, f64, f64, P]
        self._lib.oracle_bwd.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i32, i32, P, i32,
                                         f64, f64, P]
        for f in (self._lib.oracle_visible_counts, self._lib.oracle_fwd, self._lib.oracle_bwd):
            f.restype = ctypes.c_int

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _arr(x, dtype):
        return np.ascontiguousarray(np.asarray(x), dtype=dtype)

    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    @staticmethod
    def _check(status):
        if status != 0:
            raise ValueError(f"oracle: {_ERRORS.get(status, status)}")

    def _common(self, offsets, func, target_rows):
        off = self._arr(offsets, np.int64)
        fn = self._arr(func, np.int32)
        if fn.ndim != 2:
            raise ValueError("func must be [nfunc, total]")
        tr = None if target_rows is None else self._arr(target_rows, np.int32)
        return off, fn, tr

    # -- entry points ----------------------------------------------------
    def visible_counts(self, offsets, func, target_rows=None):
        off, fn, tr = self._common(offsets, func, target_rows)
        B = off.size - 1
        total = fn.shape[1]
        counts = np.zeros(B if tr is not None else total, dtype=np.int32)
        tot = ctypes.c_int64(0)
        self._check(self._lib.oracle_visible_counts(
            self._ptr(off), B, total, self._ptr(fn), fn.shape[0], self._ptr(tr),
            self._ptr(counts), ctypes.byref(tot)))
        return counts, int(tot.value)

    def fwd(self, q, k, v, offsets, func, alpha, max_len, target_rows=None):
        off, fn, tr = self._common(offsets, func, target_rows)
        q, k, v = (self._arr(x, np.float64) for x in (q, k, v))
        total, H, D = k.shape
        o = np.empty_like(q)
        self._check(self._lib.oracle_fwd(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(o), self._ptr(off),
            off.size - 1, total, H, D, self._ptr(fn), fn.shape[0], float(alpha),
            float(max_len), self._ptr(tr)))
        return o

    def bwd(self, q, k, v, dout, offsets, func, alpha, max_len, target_rows=None):
        off, fn, tr = self._common(offsets, func, target_rows)
        q, k, v, dout = (self._arr(x, np.float64) for x in (q, k, v, dout))
        total, H, D = k.shape
        dq = np.empty_like(q)
        dk = np.empty_like(k)
        dv = np.empty_like(v)
        self._check(self._lib.oracle_bwd(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dout), self._ptr(dq),
            self._ptr(dk), self._ptr(dv), self._ptr(off), off.size - 1, total, H, D,
            self._ptr(fn), fn.shape[0], float(alpha), float(max_len), self._ptr(tr)))
        return dq, dk, dv


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def visible_counts(offsets, func, target_rows=None):
    return default().visible_counts(offsets, func, target_rows)


def fwd(q, k, v, offsets, func, alpha, max_len, target_rows=None):
    return default().fwd(q, k, v, offsets, func, alpha, max_len, target_rows)


def bwd(q, k, v, dout, offsets, func, alpha, max_len, target_rows=None):
    return default().bwd(q, k, v, dout, offsets, func, alpha, max_len, target_rows)


def subset(offsets, seqs):
    """Row indices and rebased offsets of the sequences ``seqs`` (in order).

    Every output of a sequence depends only on that sequence's rows, so the
    oracle run on a subset gives the exact expected values of those sequences.
    """
    off = np.asarray(offsets, dtype=np.int64)
    rows = np.concatenate([np.arange(off[b], off[b + 1]) for b in seqs]) if len(seqs) else \
        np.zeros(0, dtype=np.int64)
    lengths = np.array([off[b + 1] - off[b] for b in seqs], dtype=np.int64)
    sub = np.zeros(len(seqs) + 1, dtype=np.int64)
    np.cumsum(lengths, out=sub[1:])
    return rows, sub
