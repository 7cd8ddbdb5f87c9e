"""CPU self-test of the tile-local error measures the GPU parity tests apply.

A stand-in for a correct kernel result is the FP64 oracle's output rounded to
bf16 (the outputs' own precision).  Every tile of it must pass the 2e-2 bound;
a result with one tile wrong must fail the tile check even where the
whole-tensor rel-RMSE still passes.  The mistakes are planted in copies of the
oracle's output, on the CPU.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from parity_checks import (dbias_row_tile_errors, dbias_tile_errors, full_tile_errors, rel_rmse,
                           row_tile_errors, worst)

BOUND = 2e-2


def bf16(x):
    return torch.from_numpy(np.asarray(x)).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def ref128():
    inp = si.make_problem(1, 128, 2, 32, 4242, mask="pad32")
    return oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"])


@pytest.mark.parametrize("name", ["o", "dq", "dk", "dv"])
def test_rounded_oracle_passes_every_tile(ref128, name):
    errs = full_tile_errors(bf16(ref128[name]), ref128[name], ending=False)
    assert errs.shape == (128, 4, 2)
    assert worst(errs)[0] < BOUND


def test_rounded_oracle_passes_every_dbias_tile(ref128):
    errs = dbias_tile_errors(bf16(ref128["dbias"]), ref128["dbias"])
    assert errs.shape == (1, 2, 4)
    assert worst(errs)[0] < BOUND


@pytest.mark.parametrize("name", ["dq", "dk", "dv"])
@pytest.mark.parametrize("ending", [False, True])
def test_one_zeroed_tile_is_rejected(ref128, name, ending):
    ref = ref128[name]
    x = bf16(ref)
    # row 77, positions 64..95, head 1 of the attended frame
    if ending:
        x[0, 64:96, 77, 1, :] = 0.0
    else:
        x[0, 77, 64:96, 1, :] = 0.0
    errs = full_tile_errors(x, ref, ending)
    e, idx = worst(errs)
    assert e > 0.5 and idx == (77, 2, 1)


@pytest.mark.parametrize("name", ["dq", "dk", "dv"])
def test_one_damaged_tile_passes_the_whole_tensor_criterion_but_not_the_tile_one(ref128, name):
    """A tile off by 30 % (as from one lost partial of a sum over key blocks) hides
    in the whole-tensor norm of 1M values but not in its own tile."""
    ref = ref128[name]
    x = bf16(ref)
    x[0, 5, 32:64, 0, :] *= 0.7
    assert rel_rmse(x, ref) < BOUND
    e, idx = worst(full_tile_errors(x, ref, False))
    assert e > 0.2 and idx == (5, 1, 0)


def test_transposed_tile_is_rejected(ref128):
    ref = ref128["dq"]
    x = bf16(ref)
    t = x[0, 9, 0:32, 1, :].copy()          # 32 positions x 32 channels
    x[0, 9, 0:32, 1, :] = t.T
    assert worst(full_tile_errors(x, ref, False))[0] > 0.5


def test_zeroed_dbias_block_is_rejected(ref128):
    ref = ref128["dbias"]
    x = bf16(ref)
    x[0, 1, 32:64, 64:96] = 0.0     # (keys 96..127 are masked: their dbias is 0 anyway)
    e, idx = worst(dbias_tile_errors(x, ref))
    assert e > 0.3 and idx == (0, 1, 1)
    assert rel_rmse(x, ref) < 0.3


def test_lost_row_chunk_partial_of_one_key_block_is_rejected(ref128):
    """One of five row-chunk partials of one 64-key block lost: a fifth of those
    values gone (keys 0..63 of every query of head 0)."""
    ref = ref128["dbias"]
    x = bf16(ref)
    x[0, 0, :, 0:64] *= 0.8
    e, idx = worst(dbias_tile_errors(x, ref))
    assert e > 0.05 and idx[:2] == (0, 0)


def test_sampled_row_and_dbias_row_tiles(ref128):
    rows = ref128["dq"][0, [3, 50, 127]]             # [3, N, H, D]
    x = bf16(rows)
    assert worst(row_tile_errors(x, rows))[0] < BOUND
    x[1, 96:128, 0, :] = 0.0
    e, idx = worst(row_tile_errors(x, rows))
    assert e > 0.5 and idx == (1, 3, 0)
    db = ref128["dbias"][0, :, 7, :]                 # two bias rows [2, N]
    y = bf16(db)
    assert worst(dbias_row_tile_errors(y, db))[0] < BOUND
    y[1, 32:64] = 0.0
    e, idx = worst(dbias_row_tile_errors(y, db))
    assert e > 0.3 and idx == (1,)


def test_zero_reference_tiles_use_the_floor(ref128):
    """Masked keys (96..127 in every row here) have exactly zero dk and dv: a tile of
    zeros matches them, and a tiny nonzero value there stays within bounds."""
    ref = ref128["dk"]
    assert np.all(ref[0, :, 96:128] == 0.0)
    x = bf16(ref)
    x[0, 3, 96:128, 0, :] = 1e-9
    assert worst(full_tile_errors(x, ref, False))[0] < BOUND
