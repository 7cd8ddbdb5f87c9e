"""Parity of the triangle-attention module around the core (include/tri_module.h) with
its FP64 oracle (oracle/module.py); needs an MI355X.

The GPU module rounds every intermediate the way a bf16 training step does (zn, the
projections, the gated output, the gradients), so the criteria are those of the core:
rel-RMSE <= 1e-2 for y and the saved projections, <= 2e-2 for dz and every parameter
gradient, each also per (position row, 32 channels) tile for the position tensors;
bitwise-identical reruns.
"""
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import module as om
from parity_checks import rel_rmse, worst

pytestmark = pytest.mark.gpu
FWD_REL, GRAD_REL = 1e-2, 2e-2
# Per-tile bound: a 32-channel tile of one position carries the rounding of about five
# bf16 steps (zn, the projections, o, the gated product, the output), whose spread over
# the ~10^4 - 10^5 tiles of a problem reaches a few times the whole-tensor error; a
# structural mistake (a tile dropped, misplaced or transposed) gives errors near 1.
TILE_REL = 5e-2


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


def run(ta, inp, H, ending, fill=0xFF):
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in inp.items()}
    params = {n: g[n] for n in ("ln_w", "ln_b", "w_qkvg", "w_bias", "w_out")}
    y, saved = ta.tri_attn_module_fwd(g["z"], g["mask"], params, H, ending=ending)
    for t in saved.values():  # the backward must read only what the forward wrote
        assert not bool(torch.isnan(t.float()).any())
    dz, grads = ta.tri_attn_module_bwd(g["z"], g["mask"], params, saved, g["dy"], H, ending=ending)
    torch.cuda.synchronize()
    return y, saved, dz, grads


def tile_errors(x, ref, floor):
    """Per (position, 32 channels) tile rel-RMSE of [..., C] position arrays; a tile whose
    norm is below `floor` times the RMS tile norm is compared against that floor instead."""
    C = ref.shape[-1]
    x = x.reshape(-1, C // 32, 32)
    r = ref.reshape(-1, C // 32, 32)
    num = np.sqrt(((x - r) ** 2).sum(-1))
    den = np.maximum(np.sqrt((r ** 2).sum(-1)), floor * np.sqrt((r ** 2).sum(-1).mean()))
    return num / den


# Tile floors.  y: 0.1 of the RMS tile norm.  dz: 0.5, because at positions whose
# attention row has no attended key (rows fully masked, e.g. by a padding mask in the
# ending orientation) the core's o and its dq, dk, dv and gate gradients are zero, and dz
# reaches z only through the pair-bias gradient of that position: four values each of
# which is a sum of bf16-rounded dS over all rows, with the per-element cancellation
# noise of that sum (up to ~7e-2 relative on single stretches of a bias row).  Those
# tiles are small, so they are compared against half the typical tile norm.
TILE_FLOOR = {"y": 0.1, "dz": 0.5}


def check(name, got, ref, bound, tag, tiles=False):
    e = rel_rmse(got, ref)
    msg = f"[module] {tag} {name}: rel-RMSE {e:.2e}"
    w = idx = None
    if tiles:
        te = tile_errors(got, ref, TILE_FLOOR[name])
        w, idx = worst(te)
        msg += f", worst tile {w:.2e} at {idx}, 99.9th percentile {np.quantile(te, 0.999):.2e}"
    say(msg)
    assert e <= bound, (tag, name, e)
    if tiles:
        assert w <= TILE_REL, (tag, name, "tile", idx, w)


def compare(ta, inp, H, ending, tag):
    y, saved, dz, grads = run(ta, inp, H, ending)
    m = om.Module(inp["z"], inp["mask"], inp["ln_w"], inp["ln_b"], inp["w_qkvg"], inp["w_bias"], inp["w_out"],
                  H, ending=ending)
    f = m.forward()
    B, N, _, C = inp["z"].shape
    check("y", to_np(y), f["y"], FWD_REL, tag, tiles=True)
    for n in ("zn", "q", "k", "v", "g"):
        check(n, to_np(saved[n]).reshape(B, N, N, C), f[n].reshape(B, N, N, C), FWD_REL, tag)
    check("bias", to_np(saved["bias"]), f["bias"], FWD_REL, tag)
    st = to_np(saved["ln_stats"])
    assert np.max(np.abs(st[..., 0] - f["mean"])) <= 1e-5 * max(1.0, np.abs(f["mean"]).max()), tag
    assert rel_rmse(st[..., 1], f["rstd"]) <= 1e-5, tag
    b = m.backward(inp["dy"])
    check("dz", to_np(dz), b["dz"], GRAD_REL, tag, tiles=True)
    names = {"ln_w": "d_ln_w", "ln_b": "d_ln_b", "w_qkvg": "dw_qkvg", "w_bias": "dw_bias", "w_out": "dw_out"}
    for n, ref_name in names.items():
        check(ref_name, to_np(grads[n]), b[ref_name], GRAD_REL, tag)
    return y, saved, dz, grads


@pytest.mark.parametrize("ending", [False, True])
def test_module_tiny64(ta, ending):
    inp = si.make_module_workload("module_tiny64")
    compare(ta, inp, 4, ending, f"tiny64-end{int(ending)}")


@pytest.mark.parametrize("B,N,H,D,mask,ending", [
    (2, 96, 4, 32, "random", False),   # B > 1, 72 position tiles, a per-element mask
    (1, 128, 2, 64, "pad32", True),    # head dimension 64
    (1, 64, 8, 16, "none", False),     # head dimension 16, no mask
    (1, 256, 4, 32, "pad32", True),
])
def test_module_shapes(ta, B, N, H, D, mask, ending):
    inp = si.make_module(B, N, H, D, 3100 + N + H, mask)
    compare(ta, inp, H, ending, f"B{B}N{N}H{H}D{D}{mask}-end{int(ending)}")


def test_module_crop768_sampled(ta):
    """The benchmarked size (module_crop768: B=1, N=768, H=4, D=32, starting node): y and
    dz at the positions of one pair row in each of the core backward's five row chunks
    and the last row, against the oracle evaluated at those rows (oracle Module.rows)."""
    inp = si.make_module_workload("module_crop768")
    y, saved, dz, grads = run(ta, inp, 4, False)
    rows = [(0, 0), (0, 154), (0, 383), (0, 500), (0, 616), (0, 767)]
    say(f"[module] crop768 sampled rows {[j for _, j in rows]}")
    m = om.Module(inp["z"], inp["mask"], inp["ln_w"], inp["ln_b"], inp["w_qkvg"], inp["w_bias"], inp["w_out"], 4)
    ref = m.rows(rows, inp["dy"])
    idx = torch.tensor([j for _, j in rows])
    got_y = to_np(y[0].index_select(0, idx.to(y.device)))[None]      # [1, R, N, C]
    got_dz = to_np(dz[0].index_select(0, idx.to(dz.device)))[None]
    check("y", got_y, ref["y"][None], FWD_REL, "crop768-sampled", tiles=True)
    check("dz", got_dz, ref["dz"][None], GRAD_REL, "crop768-sampled", tiles=True)


def test_module_bitwise_reruns(ta):
    inp = si.make_module(1, 128, 4, 32, 3201, "pad32")
    first = run(ta, inp, 4, False)
    for _ in range(2):
        again = run(ta, inp, 4, False)
        assert torch.equal(first[0].view(torch.int16), again[0].view(torch.int16))
        assert torch.equal(first[2].view(torch.int16), again[2].view(torch.int16))
        for n in first[3]:
            assert torch.equal(first[3][n].view(torch.int32), again[3][n].view(torch.int32)), n


def test_module_rejects_unsupported_channel_counts(ta):
    dev = torch.device("cuda:0")
    z = torch.zeros((1, 64, 64, 96), dtype=torch.bfloat16, device=dev)
    C, H = 96, 3
    params = {"ln_w": torch.ones(C, device=dev), "ln_b": torch.zeros(C, device=dev),
              "w_qkvg": torch.zeros((C, 4 * C), dtype=torch.bfloat16, device=dev),
              "w_bias": torch.zeros((C, H), dtype=torch.bfloat16, device=dev),
              "w_out": torch.zeros((C, C), dtype=torch.bfloat16, device=dev)}
    with pytest.raises(ta.TriAttnError) as e:
        ta.tri_attn_module_fwd(z, None, params, H)
    assert e.value.status == 2
