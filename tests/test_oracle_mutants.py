"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle/tri_attn_oracle.c, plants one plausible mistake (a
dropped term, a wrong sign, a wrong index, a transposed operand), compiles the
copy into a temporary library and runs the pin checks against it.  The checks
are the same independent sources used in test_oracle_pins: torch SDPA for the
forward, torch autograd for the gradients, and the derivative of the
log-sum-exp with respect to the bias, which must equal the softmax probability.
"""
import math
import subprocess

import numpy as np
import pytest
import torch

import oracle
from test_oracle_pins import rand_problem, rel_err, sdpa_reference, torch_grads

MUTANTS = {
    "bias dropped": [("+ bias_row[k];", ";")],
    "bias transposed": [
        ("const double *bias_row = p->bias + ((b * p->H + h) * N + j) * N;",
         "const double *bias_row = p->bias + ((b * p->H + h) * N) * N + j;"),
        ("+ bias_row[k];", "+ bias_row[k * N];")],
    "key index transposed": [("dot(qj, p->k + at5(p, b, i, k, h), p->D)",
                              "dot(qj, p->k + at5(p, b, k, i, h), p->D)")],
    "mask ignored": [("return p->mask == NULL || p->mask[(b * p->N + i) * p->N + k] != 0;",
                      "return 1;")],
    "lse without log": [("return m + log(l);", "return m + l;")],
    "dS sign (q/k path)": [("const double ds = prob[kk] * (dprob[kk] - Dj);",
                            "const double ds = prob[kk] * (dprob[kk] + Dj);")],
    "dS sign (bias path)": [("out[kk] += prob[kk] * (dprob[kk] - Dj);",
                             "out[kk] += prob[kk] * (dprob[kk] + Dj);")],
    "D without P": [("Dj += prob[k] * dprob[k];", "Dj += dprob[k];")],
    "dq without scale": [("dqj[c] += alpha * ds * kv[c];", "dqj[c] += ds * kv[c];")],
    "dk wrong operand": [("dkk[c] += alpha * ds * qj[c];", "dkk[c] += alpha * ds * gj[c];")],
    "dv wrong operand": [("dvk[c] += prob[kk] * gj[c];", "dvk[c] += prob[kk] * qj[c];")],
}


def pins_pass() -> bool:
    """True when the currently bound oracle library passes every pin check."""
    q, k, v, bias, mask, do = rand_problem(1, 8, 2, 4, 3, "random", 1.5)
    scale = 1 / math.sqrt(4)
    for ending in (False, True):
        res = oracle.forward_backward(q, k, v, bias, mask, do, ending=ending)
        ref = torch_grads(q, k, v, bias, mask, do, scale, ending)
        for got, want in zip((res["o"], res["dq"], res["dk"], res["dv"], res["dbias"]), ref):
            if not rel_err(got, want) < 1e-10:
                return False
    # d lse / d bias = P, with P from SDPA over identity values
    N = 8
    eye = np.broadcast_to(np.eye(N)[None, None, :, None, :], (1, N, N, 2, N)).copy()
    with torch.no_grad():
        P = sdpa_reference(torch.tensor(q), torch.tensor(k), torch.tensor(eye),
                           torch.tensor(bias), torch.tensor(mask), scale).numpy()
    eps = 1e-6
    h, j, kk = 1, 2, 0
    bp, bm = bias.copy(), bias.copy()
    bp[0, h, j, kk] += eps
    bm[0, h, j, kk] -= eps
    lp = oracle.forward(q, k, v, bp, mask)[1]
    lm = oracle.forward(q, k, v, bm, mask)[1]
    fd = (lp[0, :, h, j] - lm[0, :, h, j]) / (2 * eps)
    return bool(np.max(np.abs(fd - P[0, :, j, h, kk])) < 1e-8)


def test_unmutated_oracle_passes():
    oracle._load()
    assert pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    src = (oracle._SRC).read_text()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-o", str(so_path), str(c_path), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.bind(so_path))
    with np.errstate(all="ignore"):
        assert not pins_pass(), f"planted mistake '{name}' went unnoticed"
