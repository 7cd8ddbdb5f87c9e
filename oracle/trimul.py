"""FP64 CPU oracle of the triangle multiplicative update's contraction — TEST
INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU baseline).

The arithmetic is in ``tri_mul_oracle.c`` (plain C, double precision, OpenMP); this
module converts inputs exactly to fp64 and binds the two entry points.  See that file
for the definitions (outgoing and incoming contractions over the third node of every
triangle, per channel, and their gradients).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "tri_mul_oracle.c"
_LIB = _HERE / "libtrimul_oracle.so"
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (plain -O2, IEEE double, OpenMP)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-o", str(tmp), str(_SRC), "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def bind(path) -> ctypes.CDLL:
    lib = ctypes.CDLL(str(path))
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_trimul_rows.argtypes = [i64, i64, i64, i32, _dp, _dp, i64, _i64p, _i64p, _dp]
    lib.oracle_trimul_rows.restype = None
    lib.oracle_trimul_grad_rows.argtypes = [i64, i64, i64, i32, i32, _dp, _dp, _dp, i64, _i64p, _i64p, _dp]
    lib.oracle_trimul_grad_rows.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        _lib = bind(_LIB)
    return _lib


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a, t=_dp):
    return a.ctypes.data_as(t)


class TriMul:
    """One contraction problem held in fp64: a, b (and optionally g = dL/dz), all
    [B, N, N, C]."""

    def __init__(self, a, b, g=None, incoming=False):
        self.a, self.b = _f64(a), _f64(b)
        self.g = None if g is None else _f64(g)
        self.incoming = bool(incoming)
        self.B, self.N, n2, self.C = self.a.shape
        assert n2 == self.N and self.b.shape == self.a.shape
        assert self.g is None or self.g.shape == self.a.shape

    def _sel(self, rows):
        if rows is None:
            rows = [(b, x) for b in range(self.B) for x in range(self.N)]
        rb = np.ascontiguousarray([r[0] for r in rows], dtype=np.int64)
        rx = np.ascontiguousarray([r[1] for r in rows], dtype=np.int64)
        return rows, rb, rx

    def z_rows(self, rows=None) -> np.ndarray:
        """z[b, x, :, :] of the selected rows [(b, x), ...] -> [R, N, C]."""
        rows, rb, rx = self._sel(rows)
        out = np.zeros((len(rows), self.N, self.C))
        _load().oracle_trimul_rows(self.B, self.N, self.C, int(self.incoming), _p(self.a), _p(self.b),
                                   len(rows), _p(rb, _i64p), _p(rx, _i64p), _p(out))
        return out

    def grad_rows(self, which: str, rows=None) -> np.ndarray:
        """da (which="a") or db (which="b") rows [(b, x), ...] -> [R, N, C]."""
        assert self.g is not None and which in ("a", "b")
        rows, rb, rx = self._sel(rows)
        out = np.zeros((len(rows), self.N, self.C))
        _load().oracle_trimul_grad_rows(self.B, self.N, self.C, int(self.incoming), 0 if which == "a" else 1,
                                        _p(self.a), _p(self.b), _p(self.g), len(rows),
                                        _p(rb, _i64p), _p(rx, _i64p), _p(out))
        return out


def forward(a, b, incoming=False) -> np.ndarray:
    """z [B, N, N, C] in fp64."""
    p = TriMul(a, b, incoming=incoming)
    return p.z_rows().reshape(p.B, p.N, p.N, p.C)


def backward(a, b, g, incoming=False):
    """(da, db), each [B, N, N, C] in fp64."""
    p = TriMul(a, b, g, incoming=incoming)
    shp = (p.B, p.N, p.N, p.C)
    return p.grad_rows("a").reshape(shp), p.grad_rows("b").reshape(shp)
