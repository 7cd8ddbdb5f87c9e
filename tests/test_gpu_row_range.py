"""Attention-row ranges (needs an MI355X): one GPU's share of a row-sharded problem.

A call on rows [i0, i1) computes o, the residual, lse, dq, dk and dv of those rows only
and returns dbias as the range's unreduced partial sum over its rows.  Splitting the
rows into ranges must give, for every row, the same bits as the call on all rows (each
row is computed by one wave whatever the chunking), leave the other rows of the
output buffers untouched, and give dbias partials whose sum in range order is the
whole problem's dbias up to fp32 summation order, within the parity bounds of the
FP64 oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from parity_checks import dbias_tile_errors, rel_rmse, worst

pytestmark = pytest.mark.gpu


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


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def filled(shape, dtype, dev, byte):
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def run_rows(ta, g, mask, shp, ending, ranges, fill=0xFF):
    """Forward and backward per range into shared outputs filled with `fill`; one fp32
    dbias partial per range."""
    B, N, _, H, D = shp
    dev = g["q"].device
    o = filled(shp, torch.bfloat16, dev, fill)
    res = filled(shp, torch.float32, dev, fill)
    lse = filled((B, N, H, N), torch.float32, dev, fill)
    dq, dk, dv = (filled(shp, torch.bfloat16, dev, fill) for _ in range(3))
    parts = []
    for rows in ranges:
        ta.tri_attn_fwd(g["q"], g["k"], g["v"], g["bias"], mask, ending=ending, out=(o, res, lse), rows=rows)
    for rows in ranges:
        db = filled((B, H, N, N), torch.float32, dev, fill)
        ta.tri_attn_bwd(g["q"], g["k"], g["v"], g["bias"], mask, o, res, lse, g["do"], ending=ending,
                        dbias_fp32=True, out=(dq, dk, dv, db), rows=rows)
        parts.append(db)
    torch.cuda.synchronize()
    return {"o": o, "res": res, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, parts


@pytest.mark.parametrize("name,ending,ranges", [
    ("pad256", False, [(0, 96), (96, 160), (160, 256)]),
    ("pad256", True, [(0, 37), (37, 200), (200, 256)]),
    ("crop384", False, [(0, 192), (192, 384)]),
    ("crop768", True, [(0, 100), (100, 768)]),
])
def test_row_ranges_reproduce_the_whole_problem(ta, name, ending, ranges):
    say(f"[rows] {name} ending={ending} ranges={ranges}")
    inp = si.make_workload(name)
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in inp.items()}
    w = si.WORKLOADS[name]
    mask = g["mask"] if w.mask != "none" else None
    shp = tuple(inp["q"].shape)
    full, (db_full,) = run_rows(ta, g, mask, shp, ending, [None])
    part, dbs = run_rows(ta, g, mask, shp, ending, ranges, fill=0x00)
    for n in ("o", "res", "lse", "dq", "dk", "dv"):
        assert torch.equal(bits(full[n]), bits(part[n])), (name, n)
    total = dbs[0].clone()
    for d in dbs[1:]:
        total += d
    e = float((total - db_full).norm() / db_full.norm())
    say(f"[rows] {name} sum of range dbias partials vs whole-problem dbias: rel {e:.2e}")
    assert e <= 1e-5
    if w.N <= 384:
        p = oracle.Problem(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"], ending=ending)
        ref = p.dbias().reshape(w.B, w.H, w.N, w.N)
        x = total.double().cpu().numpy()
        assert rel_rmse(x, ref) <= 2e-2
        assert worst(dbias_tile_errors(x, ref))[0] <= 2e-2
        say(f"[rows] {name} whole dbias from partials rel-RMSE {rel_rmse(x, ref):.2e}")
        # each range's own partial: the oracle's dbias with dO zeroed outside the range
        # (a row with dO = 0 has dS = 0, so the sum runs over the range's rows only)
        for rows, d in zip(ranges, dbs):
            do = inp["do"].clone()
            keep = torch.zeros(w.N, dtype=torch.bool)
            keep[rows[0]:rows[1]] = True
            if ending:
                do[:, :, ~keep] = 0
            else:
                do[:, ~keep] = 0
            pr = oracle.Problem(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], do, ending=ending)
            refp = pr.dbias().reshape(w.B, w.H, w.N, w.N)
            xp = d.double().cpu().numpy()
            say(f"[rows] {name} range {rows} partial rel-RMSE {rel_rmse(xp, refp):.2e}")
            assert rel_rmse(xp, refp) <= 2e-2
            assert worst(dbias_tile_errors(xp, refp))[0] <= 2e-2


@pytest.mark.parametrize("ending", [False, True])
def test_a_range_leaves_other_rows_untouched(ta, ending):
    inp = si.make_workload("pad256")
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in inp.items()}
    shp = tuple(inp["q"].shape)
    out, (db,) = run_rows(ta, g, g["mask"], shp, ending, [(96, 160)])

    def rows_of(t):  # [B, rows, ...] view in the attended frame
        return t.transpose(1, 2) if (ending and t.dim() == 5) else t
    for n in ("o", "res", "dq", "dk", "dv", "lse"):
        t = rows_of(out[n])
        inside, before, after = t[:, 96:160], t[:, :96], t[:, 160:]
        assert bool(torch.isfinite(inside.float()).all()), n
        assert bool((bits(before) == -1).all()) and bool((bits(after) == -1).all()), n
    assert bool(torch.isfinite(db).all())
