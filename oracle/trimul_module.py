"""FP64 oracle of the triangle multiplicative update block — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark may use it; the product path
never does.  The pages name the triangle multiplicative update as the method's second
kernel family (biocloudservice page, opening paragraph; Lambda post, opening section)
and describe nothing of it, so this follows the plainest reading, the AlphaFold3
triangle multiplicative update, on a pair tensor z [B, N, N, C] (C = 128 channels, the
hidden width equal to C) with a pair mask m [B, N, N] in {0, 1}:

    zn = LayerNorm_in(z)                                  (learned scale and offset, eps)
    a  = sigmoid(zn Wag) * (zn Wap) * m                   (no bias terms)
    b  = sigmoid(zn Wbg) * (zn Wbp) * m
    g  = sigmoid(zn Wg)
    x[b, i, j, c] = sum_k a[b, i, k, c] b[b, j, k, c]     (outgoing edges)
    x[b, i, j, c] = sum_k a[b, k, i, c] b[b, k, j, c]     (incoming edges)
    y  = g * (LayerNorm_out(x) Wo)

with Wag | Wap | Wbg | Wbp | Wg side by side as w_in [C, 5 C] and Wo as w_out [C, C].
Everything is fp64 NumPy (the contraction is an einsum over the third node); the
backward is the chain rule of these lines written out by hand.  `TriMulModule.rows`
evaluates y and dz at the positions of selected pair rows only (outgoing edges), for
sizes where the whole problem is too slow for a test.
"""
from __future__ import annotations

import numpy as np

from .module import _f64, _u8, layer_norm, layer_norm_backward, sigmoid


def contract(a, b, incoming):
    """The triangle contraction over the third node, channel by channel."""
    if incoming:
        return np.einsum("bkic,bkjc->bijc", a, b)
    return np.einsum("bikc,bjkc->bijc", a, b)


def contract_grads(a, b, dx, incoming):
    """(da, db) of x = contract(a, b) for dL/dx = dx."""
    if incoming:
        return np.einsum("bijc,bkjc->bkic", dx, b), np.einsum("bijc,bkic->bkjc", dx, a)
    return np.einsum("bijc,bjkc->bikc", dx, b), np.einsum("bijc,bikc->bjkc", dx, a)


class TriMulModule:
    """One triangle-multiplication block problem in fp64 (inputs converted exactly)."""

    def __init__(self, z, mask, ln_in_w, ln_in_b, w_in, ln_out_w, ln_out_b, w_out, incoming=False, eps=1e-5):
        self.z = _f64(z)
        self.B, self.N, _, self.C = self.z.shape
        m = _u8(mask)
        self.m = np.ones((self.B, self.N, self.N)) if m is None else (m != 0).astype(np.float64)
        self.ln_in_w, self.ln_in_b = _f64(ln_in_w), _f64(ln_in_b)
        self.ln_out_w, self.ln_out_b = _f64(ln_out_w), _f64(ln_out_b)
        self.w_in, self.w_out = _f64(w_in), _f64(w_out)
        self.incoming = bool(incoming)
        self.eps = float(eps)
        assert self.w_in.shape == (self.C, 5 * self.C) and self.w_out.shape == (self.C, self.C)

    def _forward(self):
        C = self.C
        zn, mean, rstd, xhat = layer_norm(self.z, self.ln_in_w, self.ln_in_b, self.eps)
        p = zn @ self.w_in
        ag, ap, bg, bp, gp = (p[..., i * C:(i + 1) * C] for i in range(5))
        m = self.m[..., None]
        a = sigmoid(ag) * ap * m
        b = sigmoid(bg) * bp * m
        g = sigmoid(gp)
        x = contract(a, b, self.incoming)
        xn, xmean, xrstd, xxhat = layer_norm(x, self.ln_out_w, self.ln_out_b, self.eps)
        yp = xn @ self.w_out
        return dict(zn=zn, mean=mean, rstd=rstd, xhat=xhat, ag=ag, ap=ap, bg=bg, bp=bp, a=a, b=b, g=g, x=x,
                    xn=xn, xmean=xmean, xrstd=xrstd, xxhat=xxhat, yp=yp, y=g * yp)

    def forward(self):
        f = self._forward()
        return {n: f[n] for n in ("y", "zn", "a", "b", "g", "x", "xn", "mean", "rstd", "xmean", "xrstd")}

    def backward(self, dy):
        """Gradients of <dy, y>: dz and the parameter gradients."""
        dy = _f64(dy)
        f = self._forward()
        C = self.C
        m = self.m[..., None]
        # y = g * yp, yp = xn Wo, xn = LayerNorm_out(x)
        dyp = dy * f["g"]
        dgp = dy * f["yp"] * f["g"] * (1.0 - f["g"])
        dw_out = f["xn"].reshape(-1, C).T @ dyp.reshape(-1, C)
        dxn = dyp @ self.w_out.T
        d_ln_out_w = (dxn * f["xxhat"]).reshape(-1, C).sum(axis=0)
        d_ln_out_b = dxn.reshape(-1, C).sum(axis=0)
        dx = layer_norm_backward(dxn, f["xxhat"], f["xrstd"], self.ln_out_w)
        # the contraction
        da, db = contract_grads(f["a"], f["b"], dx, self.incoming)
        # a = sigmoid(ag) ap m, b = sigmoid(bg) bp m
        sa, sb = sigmoid(f["ag"]), sigmoid(f["bg"])
        dap = da * sa * m
        dag = da * f["ap"] * m * sa * (1.0 - sa)
        dbp = db * sb * m
        dbg = db * f["bp"] * m * sb * (1.0 - sb)
        dproj = np.concatenate([dag, dap, dbg, dbp, dgp], axis=-1)
        dzn = dproj @ self.w_in.T
        dw_in = f["zn"].reshape(-1, C).T @ dproj.reshape(-1, 5 * C)
        d_ln_in_w = (dzn * f["xhat"]).reshape(-1, C).sum(axis=0)
        d_ln_in_b = dzn.reshape(-1, C).sum(axis=0)
        dz = layer_norm_backward(dzn, f["xhat"], f["rstd"], self.ln_in_w)
        return {"dz": dz, "d_ln_in_w": d_ln_in_w, "d_ln_in_b": d_ln_in_b, "dw_in": dw_in,
                "d_ln_out_w": d_ln_out_w, "d_ln_out_b": d_ln_out_b, "dw_out": dw_out}

    def rows(self, rows, dy):
        """y and dz at the positions (b, p, k) of selected pair rows [(b, p), ...], outgoing
        edges.  The same lines as forward() and backward(), evaluated where they reach
        those positions: a, b and g at every position; x, and from it the output side's
        gradient dx, along row p (x[p, j] for every j: y at the row, and da[p, k] = sum_j
        dx[p, j] b[j, k]) and along column p (x[i, p] for every i: db[p, k] = sum_i dx[i, p]
        a[i, k]).  Returns {"y": [R, N, C], "dz": [R, N, C]}."""
        assert not self.incoming, "row sampling needs outgoing edges (da of a row needs all of dx otherwise)"
        dy = _f64(dy)
        C = self.C
        zn, mean, rstd, xhat = layer_norm(self.z, self.ln_in_w, self.ln_in_b, self.eps)
        p = zn @ self.w_in
        ag, ap, bg, bp, gp = (p[..., i * C:(i + 1) * C] for i in range(5))
        m = self.m[..., None]
        sa, sb = sigmoid(ag), sigmoid(bg)
        a = sa * ap * m
        b = sb * bp * m
        g = sigmoid(gp)

        def out_side(x, gg, dd):
            """y and dx at positions with contraction output x, gate g, upstream dy."""
            xn, _, xrstd, xxhat = layer_norm(x, self.ln_out_w, self.ln_out_b, self.eps)
            yp = xn @ self.w_out
            dxn = (dd * gg) @ self.w_out.T
            return gg * yp, layer_norm_backward(dxn, xxhat, xrstd, self.ln_out_w), dd * yp * gg * (1.0 - gg)

        ys, dzs = [], []
        for bb, pr in rows:
            ab, bbb = a[bb], b[bb]
            x_row = np.einsum("kc,jkc->jc", ab[pr], bbb)        # x[p, j]
            x_col = np.einsum("ikc,kc->ic", ab, bbb[pr])        # x[i, p]
            y_row, dx_row, dgp_row = out_side(x_row, g[bb, pr], dy[bb, pr])
            _, dx_col, _ = out_side(x_col, g[bb, :, pr], dy[bb, :, pr])
            da = np.einsum("jc,jkc->kc", dx_row, bbb)           # da[p, k]
            db = np.einsum("ic,ikc->kc", dx_col, ab)            # db[p, k]
            mr = m[bb, pr]
            dap = da * sa[bb, pr] * mr
            dag = da * ap[bb, pr] * mr * sa[bb, pr] * (1.0 - sa[bb, pr])
            dbp = db * sb[bb, pr] * mr
            dbg = db * bp[bb, pr] * mr * sb[bb, pr] * (1.0 - sb[bb, pr])
            dzn = np.concatenate([dag, dap, dbg, dbp, dgp_row], axis=-1) @ self.w_in.T
            dzs.append(layer_norm_backward(dzn, xhat[bb, pr], rstd[bb, pr], self.ln_in_w))
            ys.append(y_row)
        return {"y": np.stack(ys), "dz": np.stack(dzs)}
