"""Parity of the triangle multiplicative update block (include/tri_mul_module.h) with its
FP64 oracle (oracle/trimul_module.py); needs an MI355X.

Every intermediate is rounded as in a bf16 training step (zn, a, b, g, the contraction,
xn, the gradients), so the criteria are those of the attention module: rel-RMSE <= 1e-2
for y and the saved activations, <= 2e-2 for dz and every parameter gradient, per
(position, 32 channels) tile checks of y and dz, and bitwise-identical reruns.
"""
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import trimul_module as otm
from parity_checks import rel_rmse, worst

pytestmark = pytest.mark.gpu
FWD_REL, GRAD_REL = 1e-2, 2e-2
TILE_REL = 5e-2   # as for the attention module: several bf16 steps per 32-channel tile


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


def to_np(t):
    return t.float().cpu().double().numpy()


PARAMS = ("ln_in_w", "ln_in_b", "w_in", "ln_out_w", "ln_out_b", "w_out")


def run(ta, inp, incoming):
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in inp.items()}
    params = {n: g[n] for n in PARAMS}
    y, saved = ta.tri_mul_module_fwd(g["z"], g["mask"], params, incoming=incoming)
    dz, grads = ta.tri_mul_module_bwd(g["z"], g["mask"], params, saved, g["dy"], incoming=incoming)
    torch.cuda.synchronize()
    return y, saved, dz, grads


def tile_errors(x, ref, floor=0.1):
    C = ref.shape[-1]
    x, r = x.reshape(-1, C // 32, 32), ref.reshape(-1, C // 32, 32)
    num = np.sqrt(((x - r) ** 2).sum(-1))
    den = np.maximum(np.sqrt((r ** 2).sum(-1)), floor * np.sqrt((r ** 2).sum(-1).mean()))
    return num / den


def check(name, got, ref, bound, tag, tiles=False):
    e = rel_rmse(got, ref)
    msg = f"[trimul-block] {tag} {name}: rel-RMSE {e:.2e}"
    w = idx = None
    if tiles:
        te = tile_errors(got, ref)
        w, idx = worst(te)
        msg += f", worst tile {w:.2e} at {idx}"
    say(msg)
    assert e <= bound, (tag, name, e)
    if tiles:
        assert w <= TILE_REL, (tag, name, "tile", idx, w)


def compare(ta, inp, incoming, tag):
    y, saved, dz, grads = run(ta, inp, incoming)
    m = otm.TriMulModule(inp["z"], inp["mask"], *(inp[n] for n in PARAMS), incoming=incoming)
    f = m.forward()
    check("y", to_np(y), f["y"], FWD_REL, tag, tiles=True)
    for n in ("zn", "g", "xn"):
        check(n, to_np(saved[n]), f[n], FWD_REL, tag)
    for n in ("a", "b", "x"):  # channel-major on the GPU
        check(n, to_np(saved[n]).transpose(0, 2, 3, 1), f[n], FWD_REL, tag)
    b = m.backward(inp["dy"])
    check("dz", to_np(dz), b["dz"], GRAD_REL, tag, tiles=True)
    for n in PARAMS:
        ref = b[("d_" if n.startswith("ln") else "d") + n]
        check("d" + n, to_np(grads[n]), ref, GRAD_REL, tag)


@pytest.mark.parametrize("incoming", [False, True])
def test_trimul_block_tiny64(ta, incoming):
    compare(ta, si.make_trimul_module_workload("trimul_block_tiny64"), incoming, f"tiny64-in{int(incoming)}")


@pytest.mark.parametrize("B,N,mask,incoming", [(2, 96, "random", False), (1, 128, "none", True),
                                                (1, 256, "pad32", False)])
def test_trimul_block_shapes(ta, B, N, mask, incoming):
    compare(ta, si.make_trimul_module(B, N, 128, 4100 + N, mask), incoming, f"B{B}N{N}{mask}-in{int(incoming)}")


def test_trimul_block_crop768_sampled(ta):
    """The benchmarked size (trimul_block_crop768: B=1, N=768, C=128, outgoing edges): y
    and dz at the positions of six pair rows spread over the tiles, against the oracle
    evaluated at those rows (oracle TriMulModule.rows)."""
    inp = si.make_trimul_module_workload("trimul_block_crop768")
    y, saved, dz, grads = run(ta, inp, False)
    rows = [(0, 0), (0, 127), (0, 128), (0, 383), (0, 640), (0, 767)]
    say(f"[trimul-block] crop768 sampled rows {[p for _, p in rows]}")
    m = otm.TriMulModule(inp["z"], inp["mask"], *(inp[n] for n in PARAMS))
    ref = m.rows(rows, inp["dy"])
    idx = torch.tensor([p for _, p in rows])
    check("y", to_np(y[0].index_select(0, idx.to(y.device))), ref["y"], FWD_REL, "crop768-sampled", tiles=True)
    check("dz", to_np(dz[0].index_select(0, idx.to(dz.device))), ref["dz"], GRAD_REL, "crop768-sampled", tiles=True)


def test_trimul_block_bitwise_reruns(ta):
    inp = si.make_trimul_module(1, 128, 128, 4201, "pad32")
    first = run(ta, inp, False)
    for _ in range(2):
        again = run(ta, inp, False)
        assert torch.equal(first[0].view(torch.int16), again[0].view(torch.int16))
        assert torch.equal(first[2].view(torch.int16), again[2].view(torch.int16))
        for n in first[3]:
            assert torch.equal(first[3][n].view(torch.int32), again[3][n].view(torch.int32)), n


def test_trimul_block_rejects_other_channel_counts(ta):
    dev = torch.device("cuda:0")
    C = 64
    z = torch.zeros((1, 64, 64, C), dtype=torch.bfloat16, device=dev)
    params = {"ln_in_w": torch.ones(C, device=dev), "ln_in_b": torch.zeros(C, device=dev),
              "w_in": torch.zeros((C, 5 * C), dtype=torch.bfloat16, device=dev),
              "ln_out_w": torch.ones(C, device=dev), "ln_out_b": torch.zeros(C, device=dev),
              "w_out": torch.zeros((C, C), dtype=torch.bfloat16, device=dev)}
    with pytest.raises(ta.TriAttnError) as e:
        ta.tri_mul_module_fwd(z, None, params)
    assert e.value.status == 2
