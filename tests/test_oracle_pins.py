"""Pins of the FP64 oracle against things other than itself (CPU only).

The oracle (oracle/tri_attn_oracle.c) writes the plain definition of triangle
attention out in double precision.  Each test below checks it against an
independent source of truth:
  * a library routine: torch's scaled_dot_product_attention (math backend, fp64)
    for the forward, and torch autograd through it for all four gradients;
  * central finite differences of the oracle's own forward;
  * closed forms and special cases (single attended key, uniform logits, fully
    masked rows, bias shifts);
  * invariants of the exact gradients (sum_k dbias = 0, sum_k dk = 0, zero
    gradients on masked keys, D = sum_k P dP = <dO, o>, dbias = sum_i dS_i with
    P read out of the oracle through one-hot values).
A dropped term, wrong sign, wrong index or transposed operand in the oracle makes
at least the autograd and finite-difference checks fail.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention import SDPBackend, sdpa_kernel

import oracle


def rand_problem(B, N, H, D, seed, mask_kind="none", bias_std=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, N, H, D))
    k = rng.standard_normal((B, N, N, H, D))
    v = rng.standard_normal((B, N, N, H, D))
    do = rng.standard_normal((B, N, N, H, D))
    bias = bias_std * rng.standard_normal((B, H, N, N))
    mask = np.ones((B, N, N), dtype=np.uint8)
    if mask_kind == "random":
        mask = (rng.random((B, N, N)) < 0.7).astype(np.uint8)
        mask[:, :, 0] = 1  # keep every row attending at least one key
    elif mask_kind == "tail":
        mask[:, :, N - max(1, N // 4):] = 0
    return q, k, v, bias, mask, do


def sdpa_reference(q, k, v, bias, mask, scale, ending=False):
    """Triangle attention through torch SDPA (math backend), fp64 torch tensors.

    The pair axes are permuted with torch (not NumPy) for the ending node, and the
    bias is broadcast over rows so autograd sums its gradient over rows.
    """
    if ending:
        q, k, v = (x.transpose(1, 2) for x in (q, k, v))
        mask = mask.transpose(1, 2)
    B, N, _, H, D = q.shape
    Q = q.permute(0, 1, 3, 2, 4).reshape(B * N, H, N, D)
    K = k.permute(0, 1, 3, 2, 4).reshape(B * N, H, N, D)
    V = v.permute(0, 1, 3, 2, 4).reshape(B * N, H, N, v.shape[-1])
    mu = torch.zeros(mask.shape, dtype=torch.float64).masked_fill(mask == 0, -math.inf)
    am = bias[:, None, :, :, :] + mu[:, :, None, None, :]
    am = am.reshape(B * N, H, N, N)
    with sdpa_kernel(SDPBackend.MATH):
        O = F.scaled_dot_product_attention(Q, K, V, attn_mask=am, scale=scale)
    o = O.reshape(B, N, H, N, v.shape[-1]).permute(0, 1, 3, 2, 4)
    if ending:
        o = o.transpose(1, 2)
    return o


def torch_grads(q, k, v, bias, mask, do, scale, ending=False):
    t = {name: torch.tensor(x, dtype=torch.float64, requires_grad=True)
         for name, x in (("q", q), ("k", k), ("v", v), ("bias", bias))}
    o = sdpa_reference(t["q"], t["k"], t["v"], t["bias"], torch.tensor(mask), scale, ending)
    (o * torch.tensor(do)).sum().backward()
    return (o.detach().numpy(), t["q"].grad.numpy(), t["k"].grad.numpy(),
            t["v"].grad.numpy(), t["bias"].grad.numpy())


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


@pytest.mark.parametrize("mask_kind", ["none", "random", "tail"])
@pytest.mark.parametrize("ending", [False, True])
def test_forward_matches_sdpa(mask_kind, ending):
    q, k, v, bias, mask, do = rand_problem(2, 12, 3, 8, 11, mask_kind, 2.0)
    scale = 1 / math.sqrt(8)
    o, lse = oracle.forward(q, k, v, bias, mask, ending=ending)
    with torch.no_grad():
        ref = sdpa_reference(*(torch.tensor(x) for x in (q, k, v, bias, mask)), scale, ending)
    assert rel_err(o, ref.numpy()) < 1e-12


def test_custom_scale_matches_sdpa():
    q, k, v, bias, mask, do = rand_problem(1, 10, 2, 4, 5, "random")
    o, _ = oracle.forward(q, k, v, bias, mask, scale=0.37)
    with torch.no_grad():
        ref = sdpa_reference(*(torch.tensor(x) for x in (q, k, v, bias, mask)), 0.37)
    assert rel_err(o, ref.numpy()) < 1e-12


@pytest.mark.parametrize("mask_kind", ["none", "random"])
@pytest.mark.parametrize("ending", [False, True])
def test_gradients_match_torch_autograd(mask_kind, ending):
    q, k, v, bias, mask, do = rand_problem(2, 10, 2, 8, 21, mask_kind, 1.5)
    res = oracle.forward_backward(q, k, v, bias, mask, do, ending=ending)
    o_t, dq_t, dk_t, dv_t, db_t = torch_grads(q, k, v, bias, mask, do, 1 / math.sqrt(8), ending)
    assert rel_err(res["o"], o_t) < 1e-12
    assert rel_err(res["dq"], dq_t) < 1e-11
    assert rel_err(res["dk"], dk_t) < 1e-11
    assert rel_err(res["dv"], dv_t) < 1e-11
    assert rel_err(res["dbias"], db_t) < 1e-11


def test_full_size_config_shape_matches_autograd():
    """The tiny workload's shape (N=64, H=4, d=32) with an fp64 draw."""
    q, k, v, bias, mask, do = rand_problem(1, 64, 4, 32, 3, "tail")
    res = oracle.forward_backward(q, k, v, bias, mask, do)
    o_t, dq_t, dk_t, dv_t, db_t = torch_grads(q, k, v, bias, mask, do, 1 / math.sqrt(32))
    for name, ref in (("o", o_t), ("dq", dq_t), ("dk", dk_t), ("dv", dv_t), ("dbias", db_t)):
        assert rel_err(res[name], ref) < 1e-11, name


@pytest.mark.parametrize("ending", [False, True])
def test_gradients_match_finite_differences(ending):
    B, N, H, D = 1, 6, 2, 4
    q, k, v, bias, mask, do = rand_problem(B, N, H, D, 7, "random", 1.0)
    res = oracle.forward_backward(q, k, v, bias, mask, do, ending=ending)
    rng = np.random.default_rng(0)
    eps = 1e-6

    def loss(**over):
        args = dict(q=q, k=k, v=v, bias=bias)
        args.update(over)
        o, _ = oracle.forward(args["q"], args["k"], args["v"], args["bias"], mask,
                              ending=ending)
        return float(np.sum(o * do))

    for name, grad in (("q", res["dq"]), ("k", res["dk"]), ("v", res["dv"]),
                       ("bias", res["dbias"])):
        base = dict(q=q, k=k, v=v, bias=bias)[name]
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in base.shape)
            xp, xm = base.copy(), base.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * (1 + abs(grad[idx])), (name, idx)


def test_lse_derivative_is_softmax_probability():
    """d lse[b,i,h,j] / d bias[b,h,j,k] = P_i[j,k]; P taken from SDPA with V = I."""
    B, N, H, D = 1, 8, 2, 4
    q, k, v, bias, mask, do = rand_problem(B, N, H, D, 9, "random", 1.0)
    scale = 1 / math.sqrt(D)
    eye = np.broadcast_to(np.eye(N)[None, None, :, None, :], (B, N, N, H, N)).copy()
    with torch.no_grad():
        P = sdpa_reference(torch.tensor(q), torch.tensor(k), torch.tensor(eye),
                           torch.tensor(bias), torch.tensor(mask), scale).numpy()
    # P[b, i, j, h, k]
    eps = 1e-6
    for (h, j, kk) in [(0, 0, 0), (1, 3, 5), (0, 7, 2), (1, 6, 7)]:
        bp, bm = bias.copy(), bias.copy()
        bp[0, h, j, kk] += eps
        bm[0, h, j, kk] -= eps
        _, lp = oracle.forward(q, k, v, bp, mask)
        _, lm = oracle.forward(q, k, v, bm, mask)
        fd = (lp[0, :, h, j] - lm[0, :, h, j]) / (2 * eps)  # over rows i
        assert np.max(np.abs(fd - P[0, :, j, h, kk])) < 1e-8


def _softmax_probs(q, k, bias, mask):
    """P[b,i,j,h,k] read out of the oracle by attending over one-hot values (D = N)."""
    B, N, _, H, _ = q.shape
    eye = np.broadcast_to(np.eye(N)[None, None, :, None, :], (B, N, N, H, N)).copy()
    o, _ = oracle.forward(q, k, eye, bias, mask)
    return o


def test_softmax_rows_sum_to_one_and_masked_keys_get_zero_weight():
    B, N, H = 2, 8, 2
    q, k, _, bias, mask, _ = rand_problem(B, N, H, N, 13, "random", 3.0)
    P = _softmax_probs(q, k, bias, mask)
    assert np.max(np.abs(P.sum(-1) - 1.0)) < 1e-13
    masked = np.broadcast_to((mask == 0)[:, :, None, None, :], P.shape)
    assert np.all(P[masked] == 0.0)
    assert np.all(P[~masked] > 0.0)


def test_dbias_is_sum_over_rows_of_score_gradients():
    """dS_i = P_i (dP_i - D_i) with P read out of the oracle, dP = dO v^T with
    v one-hot so dP[j,k] = dO[j,k]; dbias must equal the explicit sum over i."""
    B, N, H = 2, 8, 2
    q, k, _, bias, mask, _ = rand_problem(B, N, H, N, 17, "random", 1.0)
    rng = np.random.default_rng(5)
    do = rng.standard_normal((B, N, N, H, N))
    eye = np.broadcast_to(np.eye(N)[None, None, :, None, :], (B, N, N, H, N)).copy()
    res = oracle.forward_backward(q, k, eye, bias, mask, do)
    P = res["o"]                                   # [b,i,j,h,k]
    Dj = np.sum(P * do, axis=-1, keepdims=True)
    dS = P * (do - Dj)
    dbias_explicit = dS.sum(axis=1).transpose(0, 2, 1, 3)  # [b,h,j,k]
    assert rel_err(res["dbias"], dbias_explicit) < 1e-12


def test_gradient_invariants():
    B, N, H, D = 2, 16, 3, 8
    q, k, v, bias, mask, do = rand_problem(B, N, H, D, 23, "random", 1.0)
    res = oracle.forward_backward(q, k, v, bias, mask, do)
    scale_ref = np.max(np.abs(res["dbias"]))
    # sum_k dS = 0 row by row, hence sum_k dbias = 0 and sum_k dk = 0
    assert np.max(np.abs(res["dbias"].sum(-1))) < 1e-12 * max(1, scale_ref) * N
    assert np.max(np.abs(res["dk"].sum(2))) < 1e-12 * N * max(1, np.max(np.abs(res["dk"])))
    # masked keys: no key or value gradient
    masked = np.broadcast_to((mask == 0)[:, :, :, None, None], res["dk"].shape)
    assert np.all(res["dk"][masked] == 0.0) and np.all(res["dv"][masked] == 0.0)
    # D = sum_k P dP equals <dO, o>
    do_o = np.einsum("bijhc,bijhc->bihj", do, res["o"])
    assert rel_err(res["delta"], do_o) < 1e-12


def test_single_attended_key_closed_form():
    B, N, H, D = 1, 6, 2, 4
    q, k, v, bias, _, do = rand_problem(B, N, H, D, 29)
    mask = np.zeros((B, N, N), dtype=np.uint8)
    key = np.array([3, 0, 5, 2, 2, 1])
    for i in range(N):
        mask[0, i, key[i]] = 1
    res = oracle.forward_backward(q, k, v, bias, mask, do)
    for i in range(N):
        for j in range(N):
            assert np.allclose(res["o"][0, i, j], v[0, i, key[i]], rtol=0, atol=1e-15)
        # lse equals the single logit
        for h in range(H):
            s = (q[0, i, :, h] @ k[0, i, key[i], h]) / math.sqrt(D) + bias[0, h, :, key[i]]
            assert np.allclose(res["lse"][0, i, h], s, rtol=0, atol=1e-13)
        # dv at the key is the sum of dO over queries, zero elsewhere
        assert np.allclose(res["dv"][0, i, key[i]], do[0, i].sum(0), atol=1e-13)
    assert np.max(np.abs(res["dq"])) < 1e-13
    assert np.max(np.abs(res["dk"])) < 1e-13
    assert np.max(np.abs(res["dbias"])) < 1e-13


def test_zero_query_zero_bias_gives_masked_mean():
    B, N, H, D = 1, 8, 2, 4
    _, k, v, _, mask, _ = rand_problem(B, N, H, D, 31, "random")
    q = np.zeros((B, N, N, H, D))
    bias = np.zeros((B, H, N, N))
    o, lse = oracle.forward(q, k, v, bias, mask)
    for i in range(N):
        valid = mask[0, i] != 0
        mean = v[0, i, valid].mean(axis=0)  # [H, D]
        for j in range(N):
            assert np.allclose(o[0, i, j], mean, atol=1e-14)
        assert np.allclose(lse[0, i], math.log(valid.sum()), atol=1e-14)


def test_bias_shift_leaves_output_and_shifts_lse():
    B, N, H, D = 1, 8, 2, 4
    q, k, v, bias, mask, _ = rand_problem(B, N, H, D, 37, "random")
    c = np.random.default_rng(1).standard_normal((B, H, N, 1))
    o1, l1 = oracle.forward(q, k, v, bias, mask)
    o2, l2 = oracle.forward(q, k, v, bias + c, mask)
    assert rel_err(o2, o1) < 1e-13
    shift = np.broadcast_to(c[:, None, :, :, 0], l1.shape)  # [b, i, h, j]
    assert np.max(np.abs(l2 - l1 - shift)) < 1e-12


def test_fully_masked_row_convention():
    B, N, H, D = 1, 6, 2, 4
    q, k, v, bias, mask, do = rand_problem(B, N, H, D, 41)
    mask[0, 2, :] = 0
    res = oracle.forward_backward(q, k, v, bias, mask, do)
    assert np.all(res["o"][0, 2] == 0.0)
    assert np.all(np.isinf(res["lse"][0, 2])) and np.all(res["lse"][0, 2] > 0)
    for name in ("dq", "dk", "dv"):
        assert np.all(res[name][0, 2] == 0.0)
    # the other rows are unaffected by the dead row
    mask2 = mask.copy()
    res_other = oracle.forward_backward(q, k, v, bias, mask2, do)
    assert np.all(np.isfinite(res_other["dbias"]))


def test_sampled_rows_match_full_run():
    """The sampled entry points (used at full size) agree with the full run."""
    B, N, H, D = 2, 10, 2, 4
    q, k, v, bias, mask, do = rand_problem(B, N, H, D, 43, "random")
    for ending in (False, True):
        full = oracle.forward_backward(q, k, v, bias, mask, do, ending=ending)
        p = oracle.Problem(q, k, v, bias, mask, do, ending=ending)
        rows = [(1, 3), (0, 9)]
        part = p.rows(rows)
        for r, (b, i) in enumerate(rows):
            for name in ("o", "dq", "dk", "dv"):
                ref = full[name][b, :, i] if ending else full[name][b, i]
                assert np.array_equal(part[name][r], ref), name
            assert np.array_equal(part["lse"][r], full["lse"][b, i])
        sel = [(1, 1, 4), (0, 0, 0)]
        db = p.dbias(sel)
        for s, (b, h, j) in enumerate(sel):
            assert np.array_equal(db[s], full["dbias"][b, h, j])
