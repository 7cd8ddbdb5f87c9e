"""Pins of the module oracle (oracle/module.py) against definitions it does not share.

- An independent torch fp64 formulation of the same block (torch's layer_norm, matrix
  products, sigmoid and an explicit masked softmax over einsum logits, not the
  attention oracle's C code), differentiated by autograd: forward and every gradient.
- Central finite differences of the oracle's own forward.
- Closed forms: zero gate weights give g = 1/2; zero query and key weights make the
  attention weights the softmax of the projected bias alone, computed here by hand;
  the LayerNorm input gradient sums to zero over the channels of every position.
- Planted mistakes (gate, bias transposition, LayerNorm offset, LayerNorm backward,
  bias-gradient transposition) must each be caught by the autograd pin.
"""
import math

import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import module as om

pytestmark = pytest.mark.filterwarnings("ignore")


def small(B=1, N=8, H=2, D=4, seed=5, mask="pad32"):
    inp = si.make_module(B, N, H, D, seed, "none")
    if mask == "pad32":  # the last two keys of every row masked (N is small here)
        m = torch.ones((B, N, N), dtype=torch.uint8)
        m[:, :, N - 2:] = 0
        inp["mask"] = m
    elif mask == "random":
        g = torch.Generator().manual_seed(seed)
        m = (torch.rand((B, N, N), generator=g) < 0.7).to(torch.uint8)
        m[:, :, 0] = 1  # every row keeps a key, in both orientations
        m[:, 0, :] = 1
        inp["mask"] = m
    return inp


def torch_block(z, mask, ln_w, ln_b, w_qkvg, w_bias, w_out, H, ending):
    """The block of oracle/module.py written independently in torch (fp64)."""
    if ending:
        z, mask = z.transpose(1, 2), mask.transpose(1, 2)
    C = z.shape[-1]
    D = C // H
    zn = torch.nn.functional.layer_norm(z, (C,), ln_w, ln_b, eps=1e-5)
    q, k, v, gp = (zn @ w_qkvg).split(C, dim=-1)
    q, k, v = (x.unflatten(-1, (H, D)) for x in (q, k, v))
    bias = (zn @ w_bias).permute(0, 3, 1, 2)                              # [B, H, j, k]
    logits = torch.einsum("bijhd,bikhd->bihjk", q, k) / math.sqrt(D) + bias[:, None]
    logits = logits.masked_fill(mask[:, :, None, None, :] == 0, float("-inf"))
    o = torch.einsum("bihjk,bikhd->bijhd", torch.softmax(logits, dim=-1), v).flatten(-2)
    y = (torch.sigmoid(gp) * o) @ w_out
    return y.transpose(1, 2) if ending else y


def autograd_ref(inp, H, ending):
    t = {n: inp[n].double().clone().requires_grad_(True)
         for n in ("z", "ln_w", "ln_b", "w_qkvg", "w_bias", "w_out")}
    y = torch_block(t["z"], inp["mask"], t["ln_w"], t["ln_b"], t["w_qkvg"], t["w_bias"], t["w_out"],
                    H, ending)
    (y * inp["dy"].double()).sum().backward()
    return y.detach().numpy(), {n: t[n].grad.numpy() for n in t}


def oracle_of(inp, H, ending):
    return om.Module(inp["z"], inp["mask"], inp["ln_w"], inp["ln_b"], inp["w_qkvg"], inp["w_bias"],
                     inp["w_out"], H, ending=ending)


GRAD_NAMES = {"dz": "z", "d_ln_w": "ln_w", "d_ln_b": "ln_b", "dw_qkvg": "w_qkvg", "dw_bias": "w_bias",
              "dw_out": "w_out"}


def rel(x, r):
    return float(np.linalg.norm(np.asarray(x) - r) / np.linalg.norm(r))


@pytest.mark.parametrize("B,N,H,D,mask,ending", [(1, 8, 2, 4, "pad32", False), (1, 8, 2, 4, "random", True),
                                                  (2, 6, 3, 2, "random", False), (2, 6, 1, 4, "random", True)])
def test_module_oracle_matches_torch_autograd(B, N, H, D, mask, ending):
    inp = small(B, N, H, D, 11 + N + H, mask)
    y_ref, g_ref = autograd_ref(inp, H, ending)
    m = oracle_of(inp, H, ending)
    assert rel(m.forward()["y"], y_ref) < 1e-12
    grads = m.backward(inp["dy"])
    for name, src in GRAD_NAMES.items():
        assert rel(grads[name], g_ref[src]) < 1e-10, name


def test_module_oracle_finite_differences():
    inp = small(1, 6, 2, 4, 3, "pad32")
    for k in inp:
        if inp[k].is_floating_point():
            inp[k] = inp[k].double()
    m = oracle_of(inp, 2, False)
    grads = m.backward(inp["dy"])
    dy = inp["dy"].numpy()

    def loss(x):
        return float((oracle_of(x, 2, False).forward()["y"] * dy).sum())
    h = 1e-6
    for name, src, idx in (("dz", "z", (0, 1, 2, 3)), ("d_ln_w", "ln_w", (5,)), ("d_ln_b", "ln_b", (2,)),
                           ("dw_qkvg", "w_qkvg", (1, 3)), ("dw_qkvg", "w_qkvg", (4, 9)),
                           ("dw_qkvg", "w_qkvg", (6, 18)), ("dw_qkvg", "w_qkvg", (7, 29)),
                           ("dw_bias", "w_bias", (3, 1)), ("dw_out", "w_out", (2, 5))):
        up, dn = dict(inp), dict(inp)
        up[src], dn[src] = inp[src].clone(), inp[src].clone()
        up[src][idx] += h
        dn[src][idx] -= h
        fd = (loss(up) - loss(dn)) / (2 * h)
        assert abs(fd - grads[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grads[name][idx])


def test_zero_gate_weights_halve_the_output():
    inp = small(1, 8, 2, 4, 21, "pad32")
    C = 8
    inp["w_qkvg"][:, 3 * C:] = 0
    m = oracle_of(inp, 2, False)
    f = m.forward()
    assert np.allclose(f["g"], 0.5, rtol=0, atol=0)
    o = f["o"].reshape(1, 8, 8, C)
    assert rel(f["y"], 0.5 * o @ inp["w_out"].double().numpy()) < 1e-14


@pytest.mark.parametrize("ending", [False, True])
def test_zero_query_and_key_weights_leave_the_bias_softmax(ending):
    """q = k = 0: row i's weights over keys k are softmax_k(bias[h, j, k]) with
    bias[h, j, k] = (zn Wb)[j, k, h] taken from the (transposed, for the ending node)
    pair tensor, so a transposed bias would fail here."""
    inp = small(1, 6, 2, 4, 31, "none")
    C, H, D, N = 8, 2, 4, 6
    inp["w_qkvg"][:, :2 * C] = 0
    f = oracle_of(inp, H, ending).forward()
    z = inp["z"].double().numpy()[0]
    if ending:
        z = z.swapaxes(0, 1)
    zn, _, _, _ = om.layer_norm(z, inp["ln_w"].double().numpy(), inp["ln_b"].double().numpy(), 1e-5)
    bj = zn @ inp["w_bias"].double().numpy()            # [j, k, h]
    v = (zn @ inp["w_qkvg"].double().numpy()[:, 2 * C:3 * C]).reshape(N, N, H, D)
    want = np.zeros((N, N, H, D))
    for i in range(N):
        for h in range(H):
            for j in range(N):
                w = np.exp(bj[j, :, h] - bj[j, :, h].max())
                want[i, j, h] = (w / w.sum()) @ v[i, :, h]
    got = f["o"][0]
    if ending:
        got = got.swapaxes(0, 1)
    assert rel(got, want) < 1e-12


def test_layer_norm_gradient_sums_to_zero_per_position():
    inp = small(2, 6, 2, 4, 41, "random")
    dz = oracle_of(inp, 2, False).backward(inp["dy"])["dz"]
    scale = np.abs(dz).max()
    assert np.abs(dz.sum(axis=-1)).max() <= 1e-12 * scale * dz.shape[-1]


MUTANTS = {
    "gate without sigmoid": ("sigmoid", lambda x: 0.5 + 0.25 * x),
    "bias transposed": ("bias_from_positions", lambda x: np.ascontiguousarray(x.transpose(0, 3, 2, 1))),
    "bias gradient transposed": ("positions_from_bias", lambda x: x.transpose(0, 3, 2, 1)),
    "layer norm without offset": ("layer_norm", None),
    "layer norm backward without the xhat term": ("layer_norm_backward", None),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_are_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    if name == "layer norm without offset":
        real = om.layer_norm

        def fn(z, w, b, eps):
            zn, mean, rstd, xhat = real(z, w, b, eps)
            return zn - b, mean, rstd, xhat
    elif name == "layer norm backward without the xhat term":
        def fn(dzn, xhat, rstd, w):
            dxhat = dzn * w
            return rstd[..., None] * (dxhat - dxhat.mean(axis=-1, keepdims=True))
    monkeypatch.setattr(om, attr, fn)
    inp = small(1, 8, 2, 4, 51, "pad32")
    y_ref, g_ref = autograd_ref(inp, 2, False)
    m = oracle_of(inp, 2, False)
    bad = rel(m.forward()["y"], y_ref) > 1e-6
    grads = m.backward(inp["dy"])
    bad = bad or any(rel(grads[n], g_ref[s]) > 1e-6 for n, s in GRAD_NAMES.items())
    assert bad, name


@pytest.mark.parametrize("ending,mask", [(False, "none"), (False, "random"), (True, "pad32"), (True, "random")])
def test_sampled_rows_match_the_whole_block(ending, mask):
    """Module.rows (y and dz at selected pair rows) against the whole-problem oracle."""
    inp = small(B=2, N=12, H=2, D=4, seed=9, mask=mask)
    m = om.Module(inp["z"], inp["mask"], inp["ln_w"], inp["ln_b"], inp["w_qkvg"], inp["w_bias"], inp["w_out"],
                  2, ending=ending)
    f, b = m.forward(), m.backward(inp["dy"])
    rows = [(0, 0), (1, 5), (0, 11), (1, 7)]
    r = m.rows(rows, inp["dy"])
    for i, (bb, j) in enumerate(rows):
        # row j of the attended frame: positions (b, j, :) of the caller's tensors, or
        # (b, :, j) for the ending block
        ref_y = f["y"][bb, :, j] if ending else f["y"][bb, j]
        ref_dz = b["dz"][bb, :, j] if ending else b["dz"][bb, j]
        np.testing.assert_allclose(r["y"][i], ref_y, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(r["dz"][i], ref_dz, rtol=1e-9, atol=1e-11)
