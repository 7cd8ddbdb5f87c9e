"""Pins of the FP64 triangle-multiplication oracle (CPU only).

The oracle (oracle/tri_mul_oracle.c, plain C loops) is checked against sources other
than itself:
  - torch.einsum in fp64 for the forward contraction in both directions;
  - torch fp64 autograd through that einsum for both gradients;
  - central finite differences of the oracle's own forward;
  - closed forms: an identity factor turns the contraction into a copy or a transpose
    of the other factor, all-ones factors give N everywhere;
  - invariants: the incoming contraction is the outgoing one of the pair-transposed
    factors; the contraction is bilinear, so <g, z> = <da, a> = <db, b>;
  - sampled rows equal the corresponding rows of the whole result.
Planted mistakes in copies of the oracle (an index transposed, a channel mixed up,
the incoming direction ignored, a gradient's operand or index swapped) must each be
caught by these checks.
"""
import subprocess

import numpy as np
import pytest
import torch

from oracle import trimul

EQ = {False: "bikc,bjkc->bijc", True: "bkic,bkjc->bijc"}


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def torch_ref(a, b, g, incoming):
    A = torch.tensor(a, requires_grad=True)
    Bt = torch.tensor(b, requires_grad=True)
    Z = torch.einsum(EQ[incoming], A, Bt)
    (Z * torch.tensor(g)).sum().backward()
    return Z.detach().numpy(), A.grad.numpy(), Bt.grad.numpy()


def rel(x, y):
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def pins_pass() -> bool:
    a, b, g = rand((2, 9, 9, 4), 1), rand((2, 9, 9, 4), 2), rand((2, 9, 9, 4), 3)
    for incoming in (False, True):
        z = trimul.forward(a, b, incoming)
        da, db = trimul.backward(a, b, g, incoming)
        zr, dar, dbr = torch_ref(a, b, g, incoming)
        if not (rel(z, zr) < 1e-12 and rel(da, dar) < 1e-12 and rel(db, dbr) < 1e-12):
            return False
    return True


@pytest.mark.parametrize("incoming", [False, True])
def test_forward_matches_einsum(incoming):
    a, b = rand((2, 12, 12, 5), 10), rand((2, 12, 12, 5), 11)
    z = trimul.forward(a, b, incoming)
    assert rel(z, np.einsum(EQ[incoming], a, b)) < 1e-13


@pytest.mark.parametrize("incoming", [False, True])
def test_gradients_match_autograd(incoming):
    a, b, g = rand((2, 12, 12, 5), 20), rand((2, 12, 12, 5), 21), rand((2, 12, 12, 5), 22)
    da, db = trimul.backward(a, b, g, incoming)
    _, dar, dbr = torch_ref(a, b, g, incoming)
    assert rel(da, dar) < 1e-13 and rel(db, dbr) < 1e-13


@pytest.mark.parametrize("incoming", [False, True])
def test_gradients_match_finite_differences(incoming):
    a, b, g = rand((1, 7, 7, 3), 30), rand((1, 7, 7, 3), 31), rand((1, 7, 7, 3), 32)
    da, db = trimul.backward(a, b, g, incoming)
    eps = 1e-6
    for which, x, grad in (("a", a, da), ("b", b, db)):
        for idx in [(0, 0, 0, 0), (0, 3, 5, 1), (0, 6, 2, 2), (0, 4, 4, 0)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            if which == "a":
                fp, fm = trimul.forward(xp, b, incoming), trimul.forward(xm, b, incoming)
            else:
                fp, fm = trimul.forward(a, xp, incoming), trimul.forward(a, xm, incoming)
            fd = float(np.sum(g * (fp - fm)) / (2 * eps))
            assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(grad[idx])), (which, idx)


def test_closed_forms():
    N, C = 10, 3
    b = rand((1, N, N, C), 40)
    eye = np.broadcast_to(np.eye(N)[None, :, :, None], (1, N, N, C)).copy()
    # outgoing with a[i, k] = delta(i, k): z[i, j] = b[j, i] (a transpose of b)
    assert np.array_equal(trimul.forward(eye, b, False), b.transpose(0, 2, 1, 3))
    # incoming with a[k, i] = delta(k, i): z[i, j] = b[i, j] (a copy of b)
    assert np.array_equal(trimul.forward(eye, b, True), b)
    ones = np.ones((1, N, N, C))
    for incoming in (False, True):
        assert np.array_equal(trimul.forward(ones, ones, incoming), np.full((1, N, N, C), float(N)))


def test_incoming_is_outgoing_of_transposed_factors():
    a, b = rand((2, 11, 11, 4), 50), rand((2, 11, 11, 4), 51)
    t = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))  # noqa: E731
    assert rel(trimul.forward(a, b, True), trimul.forward(t(a), t(b), False)) < 1e-14


@pytest.mark.parametrize("incoming", [False, True])
def test_bilinearity_adjoint_identity(incoming):
    a, b, g = rand((1, 13, 13, 6), 60), rand((1, 13, 13, 6), 61), rand((1, 13, 13, 6), 62)
    z = trimul.forward(a, b, incoming)
    da, db = trimul.backward(a, b, g, incoming)
    s = float(np.sum(g * z))
    assert abs(float(np.sum(da * a)) - s) < 1e-10 * abs(s)
    assert abs(float(np.sum(db * b)) - s) < 1e-10 * abs(s)


@pytest.mark.parametrize("incoming", [False, True])
def test_sampled_rows_equal_whole_result(incoming):
    a, b, g = rand((2, 8, 8, 3), 70), rand((2, 8, 8, 3), 71), rand((2, 8, 8, 3), 72)
    p = trimul.TriMul(a, b, g, incoming)
    rows = [(1, 5), (0, 0), (1, 7)]
    z = trimul.forward(a, b, incoming)
    da, db = trimul.backward(a, b, g, incoming)
    assert np.array_equal(p.z_rows(rows), np.stack([z[r] for r in rows]))
    assert np.array_equal(p.grad_rows("a", rows), np.stack([da[r] for r in rows]))
    assert np.array_equal(p.grad_rows("b", rows), np.stack([db[r] for r in rows]))


MUTANTS = {
    "a index transposed (outgoing)": [("acc += a[at4(N, C, b, i, k) + c] * bb[at4(N, C, b, j, k) + c];",
                                      "acc += a[at4(N, C, b, k, i) + c] * bb[at4(N, C, b, j, k) + c];")],
    "b index transposed (outgoing)": [("acc += a[at4(N, C, b, i, k) + c] * bb[at4(N, C, b, j, k) + c];",
                                      "acc += a[at4(N, C, b, i, k) + c] * bb[at4(N, C, b, k, j) + c];")],
    "channel mixed up": [("acc += a[at4(N, C, b, i, k) + c] * bb[at4(N, C, b, j, k) + c];",
                          "acc += a[at4(N, C, b, i, k) + c] * bb[at4(N, C, b, j, k)];")],
    "incoming ignored": [("                    if (incoming)\n", "                    if (0)\n")],
    "da wrong operand (outgoing)": [("acc += g[at4(N, C, b, x, t) + c] * bb[at4(N, C, b, t, y) + c];",
                                    "acc += g[at4(N, C, b, x, t) + c] * a[at4(N, C, b, t, y) + c];")],
    "db g transposed (outgoing)": [("acc += g[at4(N, C, b, t, x) + c] * a[at4(N, C, b, t, y) + c];",
                                   "acc += g[at4(N, C, b, x, t) + c] * a[at4(N, C, b, t, y) + c];")],
    "da g index (incoming)": [("acc += g[at4(N, C, b, y, t) + c] * bb[at4(N, C, b, x, t) + c];",
                              "acc += g[at4(N, C, b, t, y) + c] * bb[at4(N, C, b, x, t) + c];")],
    "db a index (incoming)": [("acc += g[at4(N, C, b, t, y) + c] * a[at4(N, C, b, x, t) + c];",
                              "acc += g[at4(N, C, b, t, y) + c] * a[at4(N, C, b, t, x) + c];")],
}


def test_unmutated_oracle_passes_the_pins():
    assert pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    src = trimul._SRC.read_text()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    c_path, so_path = tmp_path / "mutant.c", tmp_path / "libmutant.so"
    c_path.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-o", str(so_path), str(c_path), "-lm"], check=True)
    monkeypatch.setattr(trimul, "_lib", trimul.bind(so_path))
    assert not pins_pass(), f"planted mistake '{name}' went unnoticed"
