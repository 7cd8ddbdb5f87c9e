"""FP64 CPU oracle for triangle attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``triangle_attention_amd``) never calls
it, and the two share no code: the arithmetic lives in ``tri_attn_oracle.c``
(plain C, double precision, OpenMP) and in the NumPy transposes below.

Definitions followed (TurboPairFormer pages, Lambda post "Как работает
TurboPairFormer" and biocloudservice page "它优化了什么"): softmax attention of
every row's queries over that row's keys, with a per-head pair bias shared by
all rows and a key mask; the backward returns the query, key, value and
pair-bias gradients, the last one a sum over all rows.

Ending-node orientation (the pages are silent; plainest reading): the pair
tensor is transposed, the starting-node operation is applied with the bias as
given and the mask transposed, and the outputs are transposed back:
    o_end[b, i, j] = TA(q^T, k^T, v^T, bias, mask^T)[b, j, i]
with x^T swapping the two pair axes.  The saved log-sum-exp is indexed
[b, r, h, q] by attention row r and query q of the attended frame.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "tri_attn_oracle.c"
_LIB = _HERE / "liboracle.so"
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (plain -O2, IEEE double, OpenMP)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-o", str(tmp), str(_SRC), "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def bind(path) -> ctypes.CDLL:
    """Open a compiled oracle library and declare its entry points."""
    lib = ctypes.CDLL(str(path))
    i64 = ctypes.c_int64
    lib.oracle_rows.argtypes = [i64, i64, i64, i64, ctypes.c_double,
                                _dp, _dp, _dp, _dp, _u8p, _dp,
                                i64, _i64p, _i64p,
                                _dp, _dp, _dp, _dp, _dp, _dp]
    lib.oracle_rows.restype = None
    lib.oracle_dbias.argtypes = [i64, i64, i64, i64, ctypes.c_double,
                                 _dp, _dp, _dp, _dp, _u8p, _dp,
                                 i64, _i64p, _i64p, _i64p, _dp]
    lib.oracle_dbias.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        _lib = bind(_LIB)
    return _lib


def _f64(x) -> np.ndarray:
    """Exact conversion to a C-contiguous float64 array (bf16 -> fp64 is exact)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _u8(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.uint8))


def _ptr(a, t=_dp):
    return None if a is None else a.ctypes.data_as(t)


class Problem:
    """One triangle-attention problem held in fp64 (and the mask as u8), already
    in the attended frame (transposed for the ending node)."""

    def __init__(self, q, k, v, bias, mask=None, do=None, scale=None, ending=False):
        self.ending = bool(ending)
        q, k, v = _f64(q), _f64(k), _f64(v)
        do = None if do is None else _f64(do)
        mask = _u8(mask)
        if self.ending:
            q, k, v = (np.ascontiguousarray(x.swapaxes(1, 2)) for x in (q, k, v))
            if do is not None:
                do = np.ascontiguousarray(do.swapaxes(1, 2))
            if mask is not None:
                mask = np.ascontiguousarray(mask.swapaxes(1, 2))
        self.q, self.k, self.v, self.do, self.mask = q, k, v, do, mask
        self.bias = _f64(bias)
        self.B, self.N, _, self.H, self.D = q.shape
        assert self.bias.shape == (self.B, self.H, self.N, self.N)
        self.alpha = float(scale) if scale else 1.0 / np.sqrt(self.D)

    def _dims(self):
        return (self.B, self.N, self.H, self.D, self.alpha)

    def rows(self, rows=None, grads=True):
        """Outputs of the selected attention rows [(b, r), ...] (default: all).

        Returns a dict of compact arrays: o, dq, dk, dv [R, N, H, D]; lse, delta
        [R, H, N] (delta = sum_k P dP).  Arrays are in the attended frame.
        """
        lib = _load()
        if rows is None:
            rows = [(b, i) for b in range(self.B) for i in range(self.N)]
        rb = np.ascontiguousarray([r[0] for r in rows], dtype=np.int64)
        ri = np.ascontiguousarray([r[1] for r in rows], dtype=np.int64)
        R, N, H, D = len(rows), self.N, self.H, self.D
        out = {"o": np.zeros((R, N, H, D)), "lse": np.zeros((R, H, N))}
        want = grads and self.do is not None
        if want:
            for name in ("dq", "dk", "dv"):
                out[name] = np.zeros((R, N, H, D))
            out["delta"] = np.zeros((R, H, N))
        lib.oracle_rows(*self._dims(), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                        _ptr(self.bias), _ptr(self.mask, _u8p),
                        _ptr(self.do) if want else None,
                        R, _ptr(rb, _i64p), _ptr(ri, _i64p),
                        _ptr(out["o"]), _ptr(out["lse"]),
                        _ptr(out.get("dq")), _ptr(out.get("dk")), _ptr(out.get("dv")),
                        _ptr(out.get("delta")))
        return out

    def dbias(self, sel=None):
        """dbias rows for the selected [(b, h, j), ...] (default: all) -> [S, N]."""
        lib = _load()
        assert self.do is not None
        if sel is None:
            sel = [(b, h, j) for b in range(self.B) for h in range(self.H)
                   for j in range(self.N)]
        sb = np.ascontiguousarray([s[0] for s in sel], dtype=np.int64)
        sh = np.ascontiguousarray([s[1] for s in sel], dtype=np.int64)
        sj = np.ascontiguousarray([s[2] for s in sel], dtype=np.int64)
        out = np.zeros((len(sel), self.N))
        lib.oracle_dbias(*self._dims(), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                         _ptr(self.bias), _ptr(self.mask, _u8p), _ptr(self.do),
                         len(sel), _ptr(sb, _i64p), _ptr(sh, _i64p), _ptr(sj, _i64p),
                         _ptr(out))
        return out


def _back(x, ending):
    """Full [B, N, N, H, D] array from the attended frame to the caller's frame."""
    return np.ascontiguousarray(x.swapaxes(1, 2)) if ending else x


def forward(q, k, v, bias, mask=None, scale=None, ending=False):
    """Full forward: (o [B,N,N,H,D], lse [B,N,H,N]) in fp64."""
    p = Problem(q, k, v, bias, mask, None, scale, ending)
    r = p.rows(grads=False)
    B, N, H, D = p.B, p.N, p.H, p.D
    o = r["o"].reshape(B, N, N, H, D)
    lse = r["lse"].reshape(B, N, H, N)
    return _back(o, p.ending), lse


def forward_backward(q, k, v, bias, mask, do, scale=None, ending=False):
    """Full forward and backward in fp64.

    Returns dict: o, dq, dk, dv ([B,N,N,H,D], caller's frame), lse, delta
    ([B,N,H,N], attended frame), dbias ([B,H,N,N]).
    """
    p = Problem(q, k, v, bias, mask, do, scale, ending)
    r = p.rows(grads=True)
    B, N, H, D = p.B, p.N, p.H, p.D
    res = {name: _back(r[name].reshape(B, N, N, H, D), p.ending)
           for name in ("o", "dq", "dk", "dv")}
    res["lse"] = r["lse"].reshape(B, N, H, N)
    res["delta"] = r["delta"].reshape(B, N, H, N)
    res["dbias"] = p.dbias().reshape(B, H, N, N)
    return res
