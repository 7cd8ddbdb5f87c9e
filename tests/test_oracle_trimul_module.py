"""Pins of the triangle-multiplication block oracle (oracle/trimul_module.py) against
definitions it does not share.

- An independent torch fp64 formulation (torch's layer_norm, matrix products, sigmoid
  and a loop over the third node for the contraction), differentiated by autograd:
  forward and all seven gradients, both edge directions, masks, B = 2.
- Central finite differences of the oracle's own forward.
- Closed forms: an all-zero mask makes a = b = 0, x = 0 and y = g * (offset_out Wo); the
  oracle's contraction equals the plain-C contraction oracle (oracle/trimul.py, channel-
  major) in both directions.
- Planted mistakes must each be caught by the autograd pin.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import trimul_module as otm
from oracle import module as om

GRADS = {"dz": "z", "d_ln_in_w": "ln_in_w", "d_ln_in_b": "ln_in_b", "dw_in": "w_in",
         "d_ln_out_w": "ln_out_w", "d_ln_out_b": "ln_out_b", "dw_out": "w_out"}


def small(B=1, N=6, C=8, seed=3, mask="random"):
    return si.make_trimul_module(B, N, C, seed, mask)


def torch_block(t, mask, incoming):
    z = t["z"]
    C = z.shape[-1]
    m = mask.to(torch.float64)[..., None]
    zn = torch.nn.functional.layer_norm(z, (C,), t["ln_in_w"], t["ln_in_b"], eps=1e-5)
    ag, ap, bg, bp, gp = (zn @ t["w_in"]).split(C, dim=-1)
    a = torch.sigmoid(ag) * ap * m
    b = torch.sigmoid(bg) * bp * m
    N = z.shape[1]
    x = torch.zeros_like(a)
    for k in range(N):  # the third node, one at a time
        if incoming:
            x = x + a[:, k, :, None, :] * b[:, k, None, :, :]
        else:
            x = x + a[:, :, k, None, :] * b[:, None, :, k, :]
    xn = torch.nn.functional.layer_norm(x, (C,), t["ln_out_w"], t["ln_out_b"], eps=1e-5)
    return torch.sigmoid(gp) * (xn @ t["w_out"])


def autograd_ref(inp, incoming):
    t = {n: inp[n].double().clone().requires_grad_(True) for n in GRADS.values()}
    y = torch_block(t, inp["mask"], incoming)
    (y * inp["dy"].double()).sum().backward()
    return y.detach().numpy(), {n: t[n].grad.numpy() for n in t}


def oracle_of(inp, incoming):
    return otm.TriMulModule(inp["z"], inp["mask"], inp["ln_in_w"], inp["ln_in_b"], inp["w_in"], inp["ln_out_w"],
                            inp["ln_out_b"], inp["w_out"], incoming=incoming)


def rel(x, r):
    return float(np.linalg.norm(np.asarray(x) - r) / np.linalg.norm(r))


@pytest.mark.parametrize("B,N,C,mask,incoming", [(1, 6, 8, "random", False), (1, 6, 8, "random", True),
                                                  (2, 5, 4, "pad32", False), (2, 7, 4, "none", True)])
def test_block_oracle_matches_torch_autograd(B, N, C, mask, incoming):
    if mask == "pad32":
        inp = small(B, N, C, 7 + N, "none")
        inp["mask"][:, :, N - 2:] = 0
    else:
        inp = small(B, N, C, 7 + N, mask)
    y_ref, g_ref = autograd_ref(inp, incoming)
    m = oracle_of(inp, incoming)
    assert rel(m.forward()["y"], y_ref) < 1e-12
    grads = m.backward(inp["dy"])
    for name, src in GRADS.items():
        assert rel(grads[name], g_ref[src]) < 1e-10, name


def test_block_oracle_finite_differences():
    inp = small(1, 5, 4, 13, "random")
    for k in inp:
        if inp[k].is_floating_point():
            inp[k] = inp[k].double()
    grads = oracle_of(inp, False).backward(inp["dy"])
    dy = inp["dy"].numpy()

    def loss(x):
        return float((oracle_of(x, False).forward()["y"] * dy).sum())
    h = 1e-6
    for name, src, idx in (("dz", "z", (0, 1, 2, 3)), ("d_ln_in_w", "ln_in_w", (1,)), ("d_ln_in_b", "ln_in_b", (2,)),
                           ("dw_in", "w_in", (0, 1)), ("dw_in", "w_in", (1, 5)), ("dw_in", "w_in", (2, 10)),
                           ("dw_in", "w_in", (3, 13)), ("dw_in", "w_in", (1, 17)), ("d_ln_out_w", "ln_out_w", (3,)),
                           ("d_ln_out_b", "ln_out_b", (0,)), ("dw_out", "w_out", (2, 1))):
        up, dn = dict(inp), dict(inp)
        up[src], dn[src] = inp[src].clone(), inp[src].clone()
        up[src][idx] += h
        dn[src][idx] -= h
        fd = (loss(up) - loss(dn)) / (2 * h)
        assert abs(fd - grads[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grads[name][idx])


def test_all_masked_block_is_the_gated_offset():
    inp = small(1, 6, 8, 23, "none")
    inp["mask"][:] = 0
    f = oracle_of(inp, False).forward()
    assert np.abs(f["x"]).max() == 0
    want = f["g"] * (inp["ln_out_b"].double().numpy() @ inp["w_out"].double().numpy())
    assert rel(f["y"], want) < 1e-14


@pytest.mark.parametrize("incoming", [False, True])
def test_contraction_matches_the_c_oracle(incoming):
    from oracle import trimul
    g = torch.Generator().manual_seed(5)
    a = torch.randn((1, 6, 6, 3), generator=g, dtype=torch.float64)
    b = torch.randn((1, 6, 6, 3), generator=g, dtype=torch.float64)
    x = otm.contract(a.numpy(), b.numpy(), incoming)
    p = trimul.TriMul(a, b, torch.zeros_like(a), incoming)
    rows = [(0, i) for i in range(6)]
    assert rel(x[0], p.z_rows(rows)) < 1e-14


MUTANTS = ["gate without sigmoid", "mask ignored on b", "contraction direction swapped",
           "output layer norm without offset", "layer norm backward without the xhat term"]


@pytest.mark.parametrize("name", MUTANTS)
def test_planted_mistakes_are_caught(monkeypatch, name):
    target = [None]  # the output LayerNorm's offset array, for the mutant that drops it
    if name == "gate without sigmoid":
        monkeypatch.setattr(otm, "sigmoid", lambda x: 0.5 + 0.25 * x)
    elif name == "mask ignored on b":
        real = otm.TriMulModule._forward

        def fwd(self):
            m0 = self.m
            f = real(self)
            self.m = np.ones_like(m0)
            f2 = real(self)
            self.m = m0
            f["b"] = f2["b"]
            f["x"] = otm.contract(f["a"], f["b"], self.incoming)
            xn, xm, xr, xx = otm.layer_norm(f["x"], self.ln_out_w, self.ln_out_b, self.eps)
            f.update(xn=xn, xmean=xm, xrstd=xr, xxhat=xx, yp=xn @ self.w_out)
            f["y"] = f["g"] * f["yp"]
            return f
        monkeypatch.setattr(otm.TriMulModule, "_forward", fwd)
    elif name == "contraction direction swapped":
        real_c = otm.contract
        monkeypatch.setattr(otm, "contract", lambda a, b, inc: real_c(a, b, not inc))
    elif name == "output layer norm without offset":
        real_ln = om.layer_norm

        def ln(z, w, b, eps):  # drops the offset of the output LayerNorm only
            zn, mean, rstd, xhat = real_ln(z, w, b, eps)
            return (zn - b if b is target[0] else zn), mean, rstd, xhat
        monkeypatch.setattr(otm, "layer_norm", ln)
    elif name == "layer norm backward without the xhat term":
        def lnb(dzn, xhat, rstd, w):
            dxhat = dzn * w
            return rstd[..., None] * (dxhat - dxhat.mean(axis=-1, keepdims=True))
        monkeypatch.setattr(otm, "layer_norm_backward", lnb)
    inp = small(1, 6, 8, 31, "random")
    m = oracle_of(inp, False)
    target[0] = m.ln_out_b
    y_ref, g_ref = autograd_ref(inp, False)
    bad = rel(m.forward()["y"], y_ref) > 1e-6
    grads = m.backward(inp["dy"])
    bad = bad or any(rel(grads[n], g_ref[s]) > 1e-6 for n, s in GRADS.items())
    assert bad, name



@pytest.mark.parametrize("mask", ["none", "random"])
def test_sampled_rows_match_the_whole_block(mask):
    """TriMulModule.rows (y and dz at selected pair rows, outgoing edges) against the
    whole-problem oracle."""
    inp = small(B=2, N=9, C=8, seed=11, mask=mask)
    o = oracle_of(inp, False)
    f, bwd = o.forward(), o.backward(inp["dy"])
    rows = [(0, 0), (1, 4), (0, 8), (1, 2)]
    r = o.rows(rows, inp["dy"])
    for i, (bb, p) in enumerate(rows):
        np.testing.assert_allclose(r["y"][i], f["y"][bb, p], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["dz"][i], bwd["dz"][bb, p], rtol=1e-9, atol=1e-11)
