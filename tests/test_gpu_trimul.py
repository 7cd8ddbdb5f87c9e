"""Parity of the triangle-multiplication contraction kernels with the FP64 oracle (needs
an MI355X).

The library's tensors are channel-major [B, C, N, N]; the oracle's are [B, N, N, C]
(the tests permute on the host).  Criteria, as for triangle attention: z rel-RMSE <=
1e-2 and max-abs <= 2e-2 of its RMS, da and db rel-RMSE <= 2e-2, each also on every
(row, 32 positions) tile over all channels; outputs filled with NaN beforehand;
bitwise-identical reruns.  The oracle runs on the whole problem up to N = 160 and on
sampled rows at the crop sizes (every sampled value is checked one by one).
"""
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import trimul
from parity_checks import rel_rmse, row_tile_errors, worst

pytestmark = pytest.mark.gpu
Z_REL, GRAD_REL = 1e-2, 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ta():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import triangle_attention_amd as mod
    mod.load_library()
    return mod


def nan_like(t):
    x = torch.empty_like(t)
    x.view(torch.uint8).fill_(0xFF)
    return x


def to_oracle(x):  # [B, C, N, N] -> [B, N, N, C]
    return x.permute(0, 2, 3, 1).contiguous()


def run(ta, inp, incoming):
    dev = torch.device("cuda:0")
    a, b, g = (inp[n].to(dev) for n in ("a", "b", "g"))
    z = ta.tri_mul_fwd(a, b, incoming=incoming, out=nan_like(a))
    da, db = ta.tri_mul_bwd(a, b, g, incoming=incoming, out=(nan_like(a), nan_like(a)))
    torch.cuda.synchronize()
    return {"z": z, "da": da, "db": db}


def rows_of(t, rows):
    """[R, N, C] rows x of a channel-major [B, C, N, N] GPU tensor (row = first pair index)."""
    return np.stack([t[b, :, x, :].float().cpu().double().numpy().T for (b, x) in rows])


def check(name, got, ref, bound, tag):
    e = rel_rmse(got, ref)
    R, N, C = ref.shape
    te = row_tile_errors(got.reshape(R, N, 1, C), ref.reshape(R, N, 1, C))
    w, idx = worst(te)
    say(f"[trimul] {tag} {name}: rel-RMSE {e:.2e}, worst (row, 32-position) tile {w:.2e} at {idx}")
    assert e <= bound, (tag, name, e)
    assert w <= bound, (tag, name, "tile", idx, w)


@pytest.mark.parametrize("B,N,C", [(1, 64, 16), (2, 96, 8), (1, 160, 4), (1, 32, 3)])
@pytest.mark.parametrize("incoming", [False, True])
def test_trimul_full(ta, B, N, C, incoming):
    """Whole-problem parity, including sizes that leave a ragged last 128-wide tile."""
    inp = si.make_trimul(B, N, C, 3000 + N + C)
    out = run(ta, inp, incoming)
    p = trimul.TriMul(to_oracle(inp["a"]), to_oracle(inp["b"]), to_oracle(inp["g"]), incoming)
    rows = [(b, x) for b in range(B) for x in range(N)]
    tag = f"B{B}N{N}C{C}{'in' if incoming else 'out'}"
    zr = p.z_rows(rows)
    zg = rows_of(out["z"], rows)
    assert np.max(np.abs(zg - zr)) <= 2e-2 * float(np.sqrt(np.mean(zr * zr))), tag
    check("z", zg, zr, Z_REL, tag)
    check("da", rows_of(out["da"], rows), p.grad_rows("a", rows), GRAD_REL, tag)
    check("db", rows_of(out["db"], rows), p.grad_rows("b", rows), GRAD_REL, tag)


@pytest.mark.parametrize("name", ["trimul_crop384", "trimul_crop768"])
@pytest.mark.parametrize("incoming", [False, True])
def test_trimul_crop_sampled(ta, name, incoming):
    w = si.TRIMUL_WORKLOADS[name]
    inp = si.make_trimul_workload(name)
    out = run(ta, inp, incoming)
    p = trimul.TriMul(to_oracle(inp["a"]), to_oracle(inp["b"]), to_oracle(inp["g"]), incoming)
    rows = [(0, x) for x in sorted({0, 1, 127, 128, w.N // 2, w.N - 129, w.N - 1, 37})]
    tag = f"{name}-{'in' if incoming else 'out'}"
    check("z", rows_of(out["z"], rows), p.z_rows(rows), Z_REL, tag)
    check("da", rows_of(out["da"], rows), p.grad_rows("a", rows), GRAD_REL, tag)
    check("db", rows_of(out["db"], rows), p.grad_rows("b", rows), GRAD_REL, tag)


@pytest.mark.parametrize("incoming", [False, True])
def test_trimul_bitwise_reruns(ta, incoming):
    inp = si.make_trimul_workload("trimul_crop384")
    first = run(ta, inp, incoming)
    for _ in range(2):
        again = run(ta, inp, incoming)
        for n in ("z", "da", "db"):
            assert torch.equal(first[n].view(torch.int16), again[n].view(torch.int16)), n


def test_trimul_rejects_unsupported_on_device(ta):
    a = torch.zeros((1, 2, 48, 48), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ta.TriAttnError) as e:
        ta.tri_mul_fwd(a, a.clone())
    assert e.value.status == 2
