"""Parity of the HIP path with the FP64 oracle (needs an MI355X).

Every GPU call goes through the C ABI (via the thin binding).  Criteria:
  forward o       : max |o - o_ref| <= 2e-2 and rel-RMSE <= 1e-2
  lse             : max |lse - lse_ref| <= 1e-4 (fp32 log-sum-exp)
  dq, dk, dv, dbias: rel-RMSE <= 2e-2 each
with rel-RMSE(x) = ||x - x_ref||_2 / ||x_ref||_2 over all compared elements, and
the same 2e-2 (1e-2 for o) on every tile of the kernels' tiling on its own: each
(attention row, head, 32 positions) of o, dq, dk, dv and each (head, 32 queries)
block of dbias over all keys, or each sampled dbias row (tests/parity_checks.py).
The oracle runs on the whole problem at N = 64 and N = 256; at N = 384, 640 and
768 it runs on sampled attention rows (o, lse, dq, dk, dv of those rows) and
sampled pair-bias-gradient rows dbias[b, h, j, :], each an exact sum over all
rows, so every sampled value is checked one by one at full size.  The sampled
rows include the first, second and last row of every row chunk of the launch
plan.  Outputs and the backward workspace are filled with NaN before each call,
so a value the kernels never write fails the comparison.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import bench
import oracle
import seeded_inputs as si
from parity_checks import (dbias_row_tile_errors, dbias_tile_errors, full_tile_errors, rel_rmse,
                           row_tile_errors, worst)

pytestmark = pytest.mark.gpu

FWD_MAX_ABS, FWD_REL_RMSE, GRAD_REL_RMSE, LSE_ABS = 2e-2, 1e-2, 2e-2, 1e-4
NAN_FILL = 0xFF  # every byte 0xff: NaN in bf16 and fp32


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
    return t.detach().float().cpu().double().numpy()


def filled(shape, dtype, dev, byte):
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def mask_arg(g, inp, use_mask):
    """The mask passed to the library: None (the unmasked kernels) for an all-ones
    mask unless use_mask is True; the given mask otherwise."""
    m = inp.get("mask")
    if m is None:
        return None
    if use_mask is None:
        use_mask = not bool(torch.all(m != 0))
    return g["mask"] if use_mask else None


def run_gpu(ta, inp, ending=False, compensated=True, scale=None, dbias_fp32=False, residual="fp32",
            use_mask=None, fill=NAN_FILL):
    """One forward and backward through the C ABI into outputs and a workspace
    whose every byte is `fill` beforehand."""
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in inp.items()}
    mask = mask_arg(g, inp, use_mask)
    B, N, _, H, D = inp["q"].shape
    shp = tuple(inp["q"].shape)
    fo = (filled(shp, torch.bfloat16, dev, fill), filled(shp, ta.RESIDUAL_DTYPES[residual], dev, fill),
          filled((B, N, H, N), torch.float32, dev, fill))
    o, res, lse = ta.tri_attn_fwd(g["q"], g["k"], g["v"], g["bias"], mask, ending=ending,
                                  scale=scale, residual=residual, out=fo)
    ws = filled((ta.bwd_workspace_bytes(B, N, H, D, ending=ending, dbias_fp32=dbias_fp32, scale=scale),),
                torch.uint8, dev, fill)
    bo = tuple(filled(shp, torch.bfloat16, dev, fill) for _ in range(3)) + (
        filled((B, H, N, N), torch.float32 if dbias_fp32 else torch.bfloat16, dev, fill),)
    dq, dk, dv, db = ta.tri_attn_bwd(g["q"], g["k"], g["v"], g["bias"], mask, o,
                                     res if compensated else None, lse, g["do"],
                                     ending=ending, scale=scale, dbias_fp32=dbias_fp32,
                                     workspace=ws, out=bo)
    torch.cuda.synchronize()
    return {"o": o, "res": res, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dbias": db}


def assert_tiles(errs, bound, tag, name):
    e, idx = worst(errs)
    assert e <= bound, (tag, name, "worst tile", idx, e)
    return e


def check_full(ta, inp, ending=False, scale=None, tag="", use_mask=None, lse_ok=None):
    """Whole-problem comparison with the oracle.  lse_ok, if given, is a boolean
    [B, N, H, N] array of the lse entries to compare (the others are skipped)."""
    say(f"[parity] {tag} ending={ending} full oracle")
    out = run_gpu(ta, inp, ending=ending, scale=scale, use_mask=use_mask)
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"],
                                  inp["do"], scale=scale, ending=ending)
    o = to_np(out["o"])
    assert np.max(np.abs(o - ref["o"])) <= FWD_MAX_ABS, tag
    assert rel_rmse(o, ref["o"]) <= FWD_REL_RMSE, tag
    assert_tiles(full_tile_errors(o, ref["o"], ending), FWD_REL_RMSE, tag, "o")
    lse, lref = to_np(out["lse"]), ref["lse"]
    sel = np.ones(lref.shape, bool) if lse_ok is None else lse_ok
    fin = np.isfinite(lref)
    assert np.array_equal(np.isfinite(lse)[sel], fin[sel]), tag
    if (fin & sel).any():
        assert np.max(np.abs(lse[fin & sel] - lref[fin & sel])) <= LSE_ABS, tag
    errs, tiles = {}, {}
    for n in ("dq", "dk", "dv", "dbias"):
        x = to_np(out[n])
        errs[n] = rel_rmse(x, ref[n])
        te = dbias_tile_errors(x, ref[n]) if n == "dbias" else full_tile_errors(x, ref[n], ending)
        tiles[n] = assert_tiles(te, GRAD_REL_RMSE, tag, n)
    say(f"[parity] {tag} o_rmse={rel_rmse(o, ref['o']):.2e} grads={errs} worst tiles={tiles}")
    for n, e in errs.items():
        assert e <= GRAD_REL_RMSE, (tag, n, e)
    return out, ref


def check_sampled(ta, inp, ending, rows, sel, tag, use_mask=None, **kw):
    say(f"[parity] {tag} ending={ending} sampled rows={rows} dbias rows={sel}")
    out = run_gpu(ta, inp, ending=ending, use_mask=use_mask, **kw)
    p = oracle.Problem(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"],
                       ending=ending)
    ref = p.rows(rows)
    refb = p.dbias(sel)

    # the sampled rows are cut out on the device, so that only they are copied back
    def row_of(t, b, r):
        return t[b, :, r] if ending else t[b, r]   # attended-frame row r of a caller-frame tensor

    cat = {n: (np.stack([to_np(row_of(out[n], b, r)) for (b, r) in rows]), ref[n])
           for n in ("o", "dq", "dk", "dv")}
    o_g, o_r = cat["o"]
    assert np.max(np.abs(o_g - o_r)) <= FWD_MAX_ABS, tag
    assert rel_rmse(o_g, o_r) <= FWD_REL_RMSE, tag
    assert_tiles(row_tile_errors(o_g, o_r), FWD_REL_RMSE, tag, "o")
    lse_g = np.stack([to_np(out["lse"][b, r]) for (b, r) in rows])
    fin = np.isfinite(ref["lse"])  # a row without attended keys has lse = +inf on both sides
    assert np.array_equal(np.isfinite(lse_g), fin), tag
    if fin.any():
        assert np.max(np.abs(lse_g[fin] - ref["lse"][fin])) <= LSE_ABS, tag
    db_g = np.stack([to_np(out["dbias"][b, h, j]) for (b, h, j) in sel])
    errs = {n: rel_rmse(*cat[n]) for n in ("dq", "dk", "dv")}
    errs["dbias"] = rel_rmse(db_g, refb)
    tiles = {n: assert_tiles(row_tile_errors(*cat[n]), GRAD_REL_RMSE, tag, n) for n in ("dq", "dk", "dv")}
    tiles["dbias"] = assert_tiles(dbias_row_tile_errors(db_g, refb), GRAD_REL_RMSE, tag, "dbias")
    say(f"[parity] {tag} o_rmse={rel_rmse(o_g, o_r):.2e} grads={errs} worst tiles={tiles}")
    for n, e in errs.items():
        assert e <= GRAD_REL_RMSE, (tag, n, e)
    return out


@pytest.mark.parametrize("ending", [False, True])
def test_tiny64_full(ta, ending):
    check_full(ta, si.make_workload("tiny64"), ending=ending, tag="tiny64")


@pytest.mark.parametrize("ending", [False, True])
def test_pad256_full(ta, ending):
    check_full(ta, si.make_workload("pad256"), ending=ending, tag="pad256")


def chunk_rows(B, N, H, D=32):
    """First, second and last row of every row chunk of the launch plan (one round of
    workgroups of 64 queries or keys, 32 at D = 64; the same chunking in both
    passes)."""
    C = bench.row_chunks(B * H * -(-N // bench.block_size(D)), N)
    per = -(-N // C)
    rows = set()
    for c in range(C):
        r0, r1 = c * per, min(N, (c + 1) * per)
        rows.update({r0, min(r0 + 1, r1 - 1), r1 - 1})
    return rows


def sample_rows(N, H=4, B=1, D=32):
    rows = {0, 1, N // 2, N - 1, 37 % N, (N * 5) // 7} | chunk_rows(B, N, H, D)
    return [(0, r) for r in sorted(rows)]


def sample_dbias(N, H):
    sel = [(0, 0, 0), (0, 1 % H, N // 3), (0, 2 % H, N - 1), (0, 3 % H, 17), (0, 0, N // 2),
           (0, H - 1, (N * 3) // 4)]
    # one query of every 32-query tile, heads in turn
    sel += [(0, t % H, 32 * t + (7 * t) % 32) for t in range(N // 32)]
    return sorted(set(sel))


@pytest.mark.parametrize("name", ["crop384", "crop640"])
def test_crop_sampled(ta, name):
    w = si.WORKLOADS[name]
    check_sampled(ta, si.make_workload(name), False, sample_rows(w.N), sample_dbias(w.N, w.H), name)


@pytest.mark.parametrize("ending", [False, True])
def test_crop768_sampled(ta, ending):
    """The timed workload: no mask (the unmasked kernel variants), rows from every row
    chunk of both passes."""
    w = si.WORKLOADS["crop768"]
    rows = sample_rows(w.N, w.H)
    assert len({r * 5 // w.N for _, r in rows}) == 5   # every fifth of the rows is sampled
    check_sampled(ta, si.make_workload("crop768"), ending, rows, sample_dbias(w.N, w.H), "crop768",
                  use_mask=False)


@pytest.mark.parametrize("name,ending", [("tiny64", False), ("tiny64", True), ("crop384", False),
                                         ("crop768", True)])
def test_absent_mask_equals_all_ones_mask(ta, name, ending):
    """mask = NULL selects compile-time unmasked kernels; an all-ones mask the masked
    ones.  Both must give the same bits."""
    inp = si.make_workload(name)
    a = run_gpu(ta, inp, ending=ending, use_mask=False)
    b = run_gpu(ta, inp, ending=ending, use_mask=True, fill=0x00)
    for n in ("o", "res", "lse", "dq", "dk", "dv", "dbias"):
        assert torch.equal(bits(a[n]), bits(b[n])), (name, n)


@pytest.mark.parametrize("ending", [False, True])
def test_tiny64_full_with_explicit_ones_mask(ta, ending):
    check_full(ta, si.make_workload("tiny64"), ending=ending, tag="tiny64-ones-mask", use_mask=True)


def test_residual_is_the_rounding_remainder(ta):
    inp = si.make_workload("pad256")
    out = run_gpu(ta, inp)
    o = out["o"].float()
    r = out["res"]
    assert r.dtype == torch.float32
    # r is O - float(o) for the round-to-nearest-even o, so |r| is at most half an ulp of o
    ulp_half = torch.where(o == 0, torch.zeros_like(o),
                           torch.ldexp(torch.ones_like(o), torch.frexp(o.abs()).exponent - 9))
    assert bool((r.abs() <= ulp_half + 1e-30).all())
    full = o + r  # the kernel's fp32 output, exactly
    ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"])[0]
    e_bf = rel_rmse(to_np(out["o"]), ref)
    e_fp = rel_rmse(to_np(full), ref)
    say(f"[residual] o rel-RMSE bf16={e_bf:.3e} with residual={e_fp:.3e}")
    # what remains of the error of o + r comes from the bf16 probabilities fed to the
    # PV product, so the gain is bounded (about 2x)
    assert e_fp < 0.75 * e_bf


@pytest.mark.parametrize("ending", [False, True])
def test_bf16_residual(ta, ending):
    """With the bf16-residual flag the forward saves the bf16 rounding of the fp32
    residual O - float(o), bitwise; o and lse do not change, and the backward (flag
    on) meets the gradient criteria, next to the fp32-residual and uncompensated
    corrections."""
    inp = si.make_workload("pad256")
    out32 = run_gpu(ta, inp, ending=ending)
    out16 = run_gpu(ta, inp, ending=ending, residual="bf16")
    unc = run_gpu(ta, inp, ending=ending, compensated=False)
    r32 = out32["res"]
    assert r32.dtype == torch.float32 and out16["res"].dtype == torch.bfloat16
    assert torch.equal(out32["o"], out16["o"]) and torch.equal(out32["lse"], out16["lse"])
    assert torch.equal(r32.to(torch.bfloat16).view(torch.int16), out16["res"].view(torch.int16))
    o = out32["o"].float()
    ulp_half = torch.where(o == 0, torch.zeros_like(o),
                           torch.ldexp(torch.ones_like(o), torch.frexp(o.abs()).exponent - 9))
    bad = r32.abs() > ulp_half + 1e-30
    if bool(bad.any()):
        idx = bad.nonzero()[:5]
        for ix in idx:
            t = tuple(int(x) for x in ix)
            say(f"[fp32 residual] at {t}: o={o[t]!r} r={r32[t]!r} half ulp={ulp_half[t]!r} "
                f"r16={out16['res'][t]!r}")
    assert not bool(bad.any())
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"],
                                  ending=ending)
    assert rel_rmse(to_np(o + r32), ref["o"]) <= rel_rmse(to_np(o + out16["res"].float()), ref["o"]) * 1.01
    for n in ("dq", "dk", "dv", "dbias"):
        e32 = rel_rmse(to_np(out32[n]), ref[n])
        e16 = rel_rmse(to_np(out16[n]), ref[n])
        eu = rel_rmse(to_np(unc[n]), ref[n])
        say(f"[residual] ending={ending} {n}: fp32 residual {e32:.3e}, bf16 residual {e16:.3e}, "
            f"uncompensated {eu:.3e}")
        assert e32 <= GRAD_REL_RMSE and e16 <= GRAD_REL_RMSE
    assert torch.equal(out32["dv"].view(torch.int16), out16["dv"].view(torch.int16))


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# byte patterns the outputs and the workspace are filled with before each rerun: NaN
# first, then patterns that differ from each other, so that any value the kernels read
# without writing it first (or never write) differs between reruns
RERUN_FILLS = (0xFF, 0x00, 0x7F, 0xA5, 0x5A)


@pytest.mark.parametrize("name,reps,ending", [("tiny64", 3, False), ("pad256", 3, False),
                                              ("crop640", 3, False), ("crop768_h8d16", 3, False),
                                              ("crop768", 5, False), ("crop768", 5, True),
                                              ("crop768_h2d64", 5, False), ("crop768_h2d64", 5, True)])
def test_bitwise_determinism(ta, name, reps, ending):
    inp = si.make_workload(name)
    say(f"[determinism] {name} ending={ending} x{reps}")
    first = run_gpu(ta, inp, ending=ending, fill=RERUN_FILLS[0])
    for n in ("o", "res", "lse", "dq", "dk", "dv", "dbias"):
        assert not bool(torch.isnan(first[n].float()).any()), (name, n)
    for rep in range(1, reps):
        again = run_gpu(ta, inp, ending=ending, fill=RERUN_FILLS[rep])
        for n in ("o", "res", "lse", "dq", "dk", "dv", "dbias"):
            assert torch.equal(bits(first[n]), bits(again[n])), (name, rep, n)
        del again


@pytest.mark.parametrize("name", ["pad256", "crop640"])
def test_compensation(ta, name):
    """dV never reads D, so it is bitwise equal in both modes; the compensated
    query, key and bias gradients are reported next to the uncompensated ones."""
    inp = si.make_workload(name)
    comp = run_gpu(ta, inp, compensated=True)
    unc = run_gpu(ta, inp, compensated=False)
    assert torch.equal(comp["dv"].view(torch.int16), unc["dv"].view(torch.int16))
    w = si.WORKLOADS[name]
    if w.N <= 256:
        ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"],
                                      inp["do"])
        pick = lambda x, n: x  # noqa: E731
        refs = {n: ref[n] for n in ("dq", "dk", "dbias")}
    else:
        rows, sel = sample_rows(w.N), sample_dbias(w.N, w.H)
        p = oracle.Problem(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"])
        rr = p.rows(rows)
        refs = {"dq": rr["dq"], "dk": rr["dk"], "dbias": p.dbias(sel)}

        def pick(x, n):
            if n == "dbias":
                return np.stack([x[b, h, j] for (b, h, j) in sel])
            return np.stack([x[b, r] for (b, r) in rows])
    for n in ("dq", "dk", "dbias"):
        ec = rel_rmse(pick(to_np(comp[n]), n), refs[n])
        eu = rel_rmse(pick(to_np(unc[n]), n), refs[n])
        say(f"[compensation] {name} {n}: compensated {ec:.3e} uncompensated {eu:.3e}")
        assert ec <= GRAD_REL_RMSE and eu <= GRAD_REL_RMSE


def custom(B, N, H, seed, mask_kind="none", bias_std=1.0, D=32):
    return si.make_problem(B, N, H, D, seed, bias_std=bias_std, mask=mask_kind)


@pytest.mark.parametrize("B,N,H,mask_kind,ending", [
    (1, 32, 1, "none", False),          # smallest size, one key tile, one head
    (2, 96, 3, "random", False),        # odd number of 32-key tiles, per-element mask, B > 1
    (2, 96, 3, "random", True),
    (1, 160, 2, "pad32", True),
    (1, 128, 5, "random", False),
    (1, 64, 8, "random", False),        # more heads: 8 and 16 (head pairs across workgroups)
    (1, 64, 16, "none", True),
])
def test_shapes_and_masks(ta, B, N, H, mask_kind, ending):
    inp = custom(B, N, H, 7 + N + H, mask_kind)
    check_full(ta, inp, ending=ending, tag=f"B{B}N{N}H{H}{mask_kind}")


@pytest.mark.parametrize("B,N,H,mask_kind,ending", [
    (1, 736, 2, "pad32", False),   # largest row tiling (6 query tiles per wave), last key block one 32-key tile
    (1, 736, 2, "random", True),
    (2, 352, 3, "random", False),  # B > 1 with a ragged key block at a mid size
])
def test_large_ragged_sampled(ta, B, N, H, mask_kind, ending):
    inp = custom(B, N, H, 101 + N + H, mask_kind)
    rows = sorted(set((b, r) for b in range(B) for (_, r) in sample_rows(N)))
    sel = sorted(set((b, h, j) for b in range(B) for (_, h, j) in sample_dbias(N, H)))
    check_sampled(ta, inp, ending, rows, sel, f"B{B}N{N}H{H}{mask_kind}")


@pytest.mark.parametrize("B,N,H,mask_kind,ending", [
    (3, 128, 64, "random", False),  # 384 workgroups in both passes: more than one round, one row chunk
    (2, 256, 33, "pad32", True),    # an odd head count above 32 (no head pairs), 264 workgroups
])
def test_multi_round_grids_sampled(ta, B, N, H, mask_kind, ending):
    inp = custom(B, N, H, 211 + N + H, mask_kind)
    rows = sorted(set((b, r) for b in range(B) for (_, r) in sample_rows(N)))
    sel = sorted(set((b, h, j) for b in range(B) for (_, h, j) in sample_dbias(N, H)))
    check_sampled(ta, inp, ending, rows, sel, f"B{B}N{N}H{H}{mask_kind}")


@pytest.mark.parametrize("ending", [False, True])
def test_maximum_size_sampled(ta, ending):
    """N = 768 with H = 64, the largest problem the library accepts (1.2e9 elements per
    tensor): element offsets of the dQ partials and of the outputs pass 2^32, the
    backward runs three rounds of workgroups, and in the ending orientation one
    attention row spans 2.4e9 bytes (its key tiles lie more than 2^31 bytes apart)."""
    say(f"[parity] maximum size ending={ending}: generating inputs")
    inp = custom(1, 768, 64, 97, "ragged512")
    check_sampled(ta, inp, ending, [(0, 0), (0, 383), (0, 767)],
                  [(0, 0, 5), (0, 31, 400), (0, 63, 767)], f"B1N768H64ragged512-end{int(ending)}")


@pytest.mark.parametrize("B,N,H,mask_kind,ending", [
    (1, 64, 4, "none", False),
    (2, 96, 3, "random", True),
    (1, 256, 8, "pad32", False),
    (1, 160, 2, "pad32", True),
])
def test_head_dim16_full(ta, B, N, H, mask_kind, ending):
    """Head dimension 16: the kernels run the 32-channel tiles with channels 16..31 at
    zero and store only the caller's 16."""
    inp = custom(B, N, H, 301 + N + H, mask_kind, D=16)
    out, ref = check_full(ta, inp, ending=ending, tag=f"D16 B{B}N{N}H{H}{mask_kind}")
    assert out["res"].shape[-1] == 16


@pytest.mark.parametrize("ending", [False, True])
def test_head_dim16_crop768_sampled(ta, ending):
    w = si.WORKLOADS["crop768_h8d16"]
    check_sampled(ta, si.make_workload("crop768_h8d16"), ending, sample_rows(w.N),
                  sample_dbias(w.N, w.H), "crop768_h8d16")


@pytest.mark.parametrize("B,N,H,mask_kind,ending", [
    (1, 64, 2, "none", False),
    (1, 64, 2, "random", True),
    (1, 256, 2, "pad32", False),       # the workload sizes of pad256 at H = 2, d = 64
    (1, 256, 2, "pad32", True),
    (2, 96, 3, "random", False),       # three 32-key blocks, B > 1, an odd head count
    (1, 160, 1, "pad32", True),
])
def test_head_dim64_full(ta, B, N, H, mask_kind, ending):
    """Head dimension 64: 128-byte tile rows, four contraction slices, 32-query
    forward blocks and 32-key backward blocks (whole-problem oracle)."""
    inp = custom(B, N, H, 401 + N + H, mask_kind, D=64)
    out, ref = check_full(ta, inp, ending=ending, tag=f"D64 B{B}N{N}H{H}{mask_kind}")
    assert out["res"].shape[-1] == 64


@pytest.mark.parametrize("ending", [False, True])
def test_head_dim64_crop768_sampled(ta, ending):
    """N = 768, H = 2, d = 64 (the 128 pair channels of the d = 32 workload) with a row
    of every backward row chunk."""
    w = si.WORKLOADS["crop768_h2d64"]
    check_sampled(ta, si.make_workload("crop768_h2d64"), ending, sample_rows(w.N, w.H, D=64),
                  sample_dbias(w.N, w.H), "crop768_h2d64")


@pytest.mark.parametrize("B,N,H,mask_kind,ending", [
    (1, 736, 3, "ragged512", False),  # 23 key blocks, ragged valid lengths, odd heads
    (2, 352, 2, "random", True),
])
def test_head_dim64_large_sampled(ta, B, N, H, mask_kind, ending):
    inp = custom(B, N, H, 503 + N + H, mask_kind, D=64)
    rows = sorted(set((b, r) for b in range(B) for (_, r) in sample_rows(N, H, B, D=64)))
    sel = sorted(set((b, h, j) for b in range(B) for (_, h, j) in sample_dbias(N, H)))
    check_sampled(ta, inp, ending, rows, sel, f"D64 B{B}N{N}H{H}{mask_kind}")


def test_fully_masked_rows_and_keys(ta):
    inp = custom(1, 64, 2, 11, "random")
    m = inp["mask"]
    m[0, 5, :] = 0           # a row with no attended key
    m[0, :, 40:] = 0         # keys 40..63 masked in every row
    m[0, 9, :] = 0
    m[0, 9, 63] = 1          # a row whose only key is in an otherwise masked tile
    out, ref = check_full(ta, inp, tag="masked-rows")
    assert torch.all(out["o"][0, 5] == 0) and torch.all(out["res"][0, 5] == 0)
    assert torch.isinf(out["lse"][0, 5]).all()
    assert torch.all(out["dk"][0, :, 40:63] == 0) and torch.all(out["dv"][0, :, 40:63] == 0)


@pytest.mark.parametrize("shift", [30.0, 60.0, 150.0])
def test_forward_probability_overflow(ta, shift):
    """A key tile whose logits exceed the first attended tile's maximum: by 30 the
    row's probability sum stays below 2^64 and the pass stands (its reciprocal taken
    at about 2^48); by 60 the sum is finite but above 2^64, and by 150 it leaves the
    fp32 range: in both the forward's per-row check must catch the row and recompute
    it against the true maximum."""
    inp = custom(1, 96, 2, 17, "none")
    inp["bias"][:, :, :, 64:] += shift   # keys 64..95: logits about `shift` above the rest
    out, ref = check_full(ta, inp, tag=f"overflow{shift:g}")
    assert torch.isfinite(out["o"].float()).all() and torch.isfinite(out["lse"]).all()


def test_bias_beyond_the_fp16_range(ta):
    """The kernels hold the bias as fp16 and saturate finite values beyond +-65504.
    That keeps the exact softmax where such values mask keys or shift every key of
    a query alike: -1e9 on every key of one query row, +7e4 on one key of a query
    (which then takes all the weight), -7e4 on some keys of a query (zero weight).
    The lse of the queries whose bias saturates is that of the saturated logits and
    is not compared; everything else is."""
    inp = custom(1, 64, 2, 29, "none")
    big = inp["bias"].float()
    big[0, 0, 5, :] = -1e9          # every key of query 5, head 0
    big[0, 1, 9, 30] = 7.0e4        # one key of query 9, head 1
    big[0, 1, 12, 3:40] = -7.0e4    # keys 3..39 of query 12, head 1
    big[0, 0, 20, 50] = -3.0e5      # one key of query 20, head 0
    inp["bias"] = big.to(torch.bfloat16)
    lse_ok = np.ones((1, 64, 2, 64), bool)
    lse_ok[0, :, 0, 5] = False
    lse_ok[0, :, 1, 9] = False
    for ending in (False, True):
        out, ref = check_full(ta, inp, ending=ending, tag=f"large-bias-end{int(ending)}", lse_ok=lse_ok)
        assert torch.isfinite(out["o"].float()).all()


def test_custom_scale_and_fp32_dbias(ta):
    inp = custom(1, 64, 4, 13, "pad32", bias_std=2.0)
    check_full(ta, inp, scale=0.3, tag="scale0.3")
    out = run_gpu(ta, inp, dbias_fp32=True)
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"])
    assert out["dbias"].dtype == torch.float32
    e32 = rel_rmse(to_np(out["dbias"]), ref["dbias"])
    out16 = run_gpu(ta, inp)
    e16 = rel_rmse(to_np(out16["dbias"]), ref["dbias"])
    say(f"[dbias] fp32 output rel-RMSE {e32:.3e}, bf16 output {e16:.3e}")
    assert e32 <= e16


@pytest.mark.parametrize("D,ending", [(32, False), (16, True), (64, True)])
def test_autograd_wrapper(ta, D, ending):
    inp = custom(1, 64, 2, 17, "pad32", D=D)
    dev = torch.device("cuda:0")
    q, k, v, bias = (inp[n].to(dev).requires_grad_(True) for n in ("q", "k", "v", "bias"))
    o = ta.tri_attn(q, k, v, bias, inp["mask"].to(dev), ending=ending)
    o.backward(inp["do"].to(dev))
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"],
                                  ending=ending)
    for t, n in ((q, "dq"), (k, "dk"), (v, "dv"), (bias, "dbias")):
        assert rel_rmse(to_np(t.grad), ref[n]) <= GRAD_REL_RMSE, n


def test_timed_backward_matches_and_times_each_kernel(ta):
    """tri_attn_bwd_timed gives the same bits as tri_attn_bwd and brackets each of
    the four backward kernels with an event."""
    import bench
    inp = custom(1, 128, 4, 23, "pad32")
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in inp.items()}
    o, res, lse = ta.tri_attn_fwd(g["q"], g["k"], g["v"], g["bias"], g["mask"])
    plain = ta.tri_attn_bwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], o, res, lse, g["do"])
    hip = bench.HipEvents()
    ev = [hip.create() for _ in range(5)]
    timed = ta.tri_attn_bwd(g["q"], g["k"], g["v"], g["bias"], g["mask"], o, res, lse, g["do"],
                            kernel_events=ev)
    torch.cuda.synchronize()
    for a, b in zip(plain, timed):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
    ms = [hip.elapsed_ms(ev[i], ev[i + 1]) for i in range(4)]
    for e in ev:
        hip.destroy(e)
    say(f"[timed] statistics, main, dQ reduction, dbias reduction: {ms} ms")
    assert all(t > 0 for t in ms)


def test_rejects_unsupported_on_device(ta):
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 48, 48, 1, 32), dtype=torch.bfloat16, device=dev)
    bias = torch.zeros((1, 1, 48, 48), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ta.TriAttnError) as e:
        ta.tri_attn_fwd(q, q.clone(), q.clone(), bias)
    assert e.value.status == 2
