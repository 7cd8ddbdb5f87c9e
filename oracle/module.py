"""FP64 oracle of the triangle-attention module around the core — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark may use it; the product path
never does.  The pages present the kernel only as triangle attention in the style of
AlphaFold3 (biocloudservice page, opening paragraph) and describe nothing around the
attention core, so this follows the plainest reading, the AlphaFold3 triangle-attention block
around the starting node, on a pair tensor z [B, N, N, C] with C = H * D channels:

    zn        = LayerNorm(z) over the C channels (learned scale w and offset b, eps)
    q, k, v   = zn Wq, zn Wk, zn Wv                      (no bias; [B, N, N, H, D])
    bias      = zn Wb, transposed to [B, H, N, N]:       bias[b, h, j, k] = (zn Wb)[b, j, k, h]
    g         = sigmoid(zn Wg)                            (no bias; [B, N, N, H * D])
    o         = core(q, k, v, bias, mask)                 (the triangle attention of this library)
    y         = (g * o) Wo                                (no bias; [B, N, N, C])

with Wq | Wk | Wv | Wg stored side by side as w_qkvg [C, 4 C] (column h * D + d of each
block is channel d of head h), Wb as w_bias [C, H] and Wo as w_out [C, C].  The
ending-node module is the same block applied to the pair tensor with its two pair
axes swapped (z and the mask transposed, y transposed back).

Everything here is fp64: the products are numpy matrix products, the core is the
attention oracle of this package (its C code), and the backward is the chain rule of
the lines above written out by hand.  `Module.rows` evaluates y and dz at the positions
of selected pair rows only (the same lines, for sizes where the whole problem is too
slow for a test).
"""
from __future__ import annotations

import numpy as np

from . import Problem as _CoreProblem
from . import forward_backward as _core_fwd_bwd
from . import forward as _core_fwd


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _u8(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.uint8)


def layer_norm(z, w, b, eps):
    """LayerNorm over the last axis: returns (zn, mean, rstd, xhat), xhat = (z - mean) * rstd."""
    mean = z.mean(axis=-1, keepdims=True)
    var = ((z - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (z - mean) * rstd
    return xhat * w + b, mean[..., 0], rstd[..., 0], xhat


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def bias_from_positions(x):
    """[B, N, N, H] per-position head values -> the pair bias [B, H, N, N]."""
    return np.ascontiguousarray(x.transpose(0, 3, 1, 2))


def positions_from_bias(x):
    """[B, H, N, N] pair-bias gradient -> [B, N, N, H] per position."""
    return x.transpose(0, 2, 3, 1)


def layer_norm_backward(dzn, xhat, rstd, w):
    """Input gradient of zn = xhat * w + b, xhat = (z - mean) * rstd, over the last axis."""
    dxhat = dzn * w
    return rstd[..., None] * (dxhat - dxhat.mean(axis=-1, keepdims=True)
                              - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))


class Module:
    """One module problem in fp64: parameters and inputs converted exactly."""

    def __init__(self, z, mask, ln_w, ln_b, w_qkvg, w_bias, w_out, H, ending=False, eps=1e-5):
        self.ending = bool(ending)
        z = _f64(z)
        mask = _u8(mask)
        if self.ending:  # the starting-node block on the transposed pair tensor
            z = z.swapaxes(1, 2)
            mask = None if mask is None else mask.swapaxes(1, 2)
        self.z = np.ascontiguousarray(z)
        self.mask = None if mask is None else np.ascontiguousarray(mask)
        self.ln_w, self.ln_b = _f64(ln_w), _f64(ln_b)
        self.w_qkvg, self.w_bias, self.w_out = _f64(w_qkvg), _f64(w_bias), _f64(w_out)
        self.B, self.N, _, self.C = self.z.shape
        self.H = int(H)
        self.D = self.C // self.H
        self.eps = float(eps)
        assert self.w_qkvg.shape == (self.C, 4 * self.C) and self.w_bias.shape == (self.C, self.H)
        assert self.w_out.shape == (self.C, self.C)

    def _heads(self, x):
        return x.reshape(self.B, self.N, self.N, self.H, self.D)

    def _project(self):
        zn, mean, rstd, xhat = layer_norm(self.z, self.ln_w, self.ln_b, self.eps)
        proj = zn @ self.w_qkvg
        C = self.C
        q, k, v = (self._heads(proj[..., i * C:(i + 1) * C]) for i in range(3))
        gpre = proj[..., 3 * C:]
        bias = bias_from_positions(zn @ self.w_bias)  # [B, H, N, N]
        return zn, mean, rstd, xhat, q, k, v, gpre, bias

    def _out(self, x):
        """Starting-node frame -> the caller's frame."""
        return np.ascontiguousarray(x.swapaxes(1, 2)) if self.ending else x

    def forward(self):
        """y [B, N, N, C] and the intermediates (caller's frame for position tensors)."""
        zn, mean, rstd, xhat, q, k, v, gpre, bias = self._project()
        o, lse = _core_fwd(q, k, v, bias, self.mask)
        g = sigmoid(gpre)
        go = g * o.reshape(self.B, self.N, self.N, self.C)
        y = go @ self.w_out
        return {"y": self._out(y), "zn": self._out(zn), "q": self._out(q), "k": self._out(k),
                "v": self._out(v), "g": self._out(g), "o": self._out(o), "bias": bias,
                "mean": self._out(mean), "rstd": self._out(rstd)}

    def backward(self, dy):
        """Gradients of <dy, y>: dz [B, N, N, C] (caller's frame) and the parameter gradients."""
        dy = _f64(dy)
        if self.ending:
            dy = dy.swapaxes(1, 2)
        B, N, C, H = self.B, self.N, self.C, self.H
        zn, mean, rstd, xhat, q, k, v, gpre, bias = self._project()
        g = sigmoid(gpre)
        # y = go Wo, go = g * o
        o_fwd, _ = _core_fwd(q, k, v, bias, self.mask)
        o = o_fwd.reshape(B, N, N, C)
        go = g * o
        dgo = dy @ self.w_out.T
        dw_out = go.reshape(-1, C).T @ dy.reshape(-1, C)
        do = dgo * g
        dgpre = dgo * o * g * (1.0 - g)
        # the core's backward with dO = do
        r = _core_fwd_bwd(q, k, v, bias, self.mask, self._heads(do))
        dq, dk, dv = (r[n].reshape(B, N, N, C) for n in ("dq", "dk", "dv"))
        dbias_pos = positions_from_bias(r["dbias"])  # [B, N, N, H]: position (j, k), head h
        dproj = np.concatenate([dq, dk, dv, dgpre], axis=-1)
        dzn = dproj @ self.w_qkvg.T + dbias_pos @ self.w_bias.T
        dw_qkvg = zn.reshape(-1, C).T @ dproj.reshape(-1, 4 * C)
        dw_bias = zn.reshape(-1, C).T @ dbias_pos.reshape(-1, H)
        # LayerNorm: zn = xhat * w + b
        d_ln_w = (dzn * xhat).reshape(-1, C).sum(axis=0)
        d_ln_b = dzn.reshape(-1, C).sum(axis=0)
        dz = layer_norm_backward(dzn, xhat, rstd, self.ln_w)
        return {"dz": self._out(dz), "d_ln_w": d_ln_w, "d_ln_b": d_ln_b, "dw_qkvg": dw_qkvg,
                "dw_bias": dw_bias, "dw_out": dw_out}

    def rows(self, rows, dy):
        """y and dz at the positions of selected pair rows, in the starting-node frame.

        rows: [(b, j), ...]; every position (b, j, k) of those rows is returned (for the
        ending block, row j of the transposed pair tensor, i.e. column j of the caller's
        tensors).  The same lines as forward() and backward(), evaluated at those
        positions only: the projections of every position (the pair bias and dO need
        them), the core oracle on the selected attention rows, and the pair-bias
        gradient entries dbias[b, h, j, :] that reach those positions (sums over every
        attention row).  Returns {"y": [R, N, C], "dz": [R, N, C]}.
        """
        dy = _f64(dy)
        if self.ending:
            dy = dy.swapaxes(1, 2)
        B, N, C, H = self.B, self.N, self.C, self.H
        zn, mean, rstd, xhat, q, k, v, gpre, bias = self._project()
        g = sigmoid(gpre)
        dgo = dy @ self.w_out.T                  # [B, N, N, C], every position
        do = self._heads(dgo * g)                # dO of every attention row
        core = _CoreProblem(q, k, v, bias, self.mask, do=do)
        r = core.rows(rows, grads=True)
        R = len(rows)
        o = r["o"].reshape(R, N, C)
        bi = [b for b, _ in rows]
        ji = [j for _, j in rows]
        g_r, dgo_r, dy_r = g[bi, ji], dgo[bi, ji], dy[bi, ji]          # [R, N, C]
        y = (g_r * o) @ self.w_out
        dgpre = dgo_r * o * g_r * (1.0 - g_r)
        dproj = np.concatenate([r["dq"].reshape(R, N, C), r["dk"].reshape(R, N, C),
                                r["dv"].reshape(R, N, C), dgpre], axis=-1)
        db = core.dbias([(b, h, j) for b, j in rows for h in range(H)]).reshape(R, H, N)
        dzn = dproj @ self.w_qkvg.T + db.transpose(0, 2, 1) @ self.w_bias.T
        dz = layer_norm_backward(dzn, xhat[bi, ji], rstd[bi, ji], self.ln_w)
        return {"y": y, "dz": dz}
