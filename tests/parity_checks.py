"""Error measures shared by the GPU parity tests and their CPU self-test.

rel_rmse(x, ref) = ||x - ref||_2 / ||ref||_2 over all compared elements (the
whole-tensor criterion).  A whole-tensor norm can hide a local indexing mistake:
one 32 x 32 tile of a gradient dropped out of 589,824 sampled values moves the
whole-tensor figure by only ~1e-2.  tile_errors() therefore measures every tile
of the kernels' tiling on its own:

  dq, dk, dv, o : per (attention row, head, 32 positions along the attended axis)
                  -> 32 x D values
  dbias         : per (batch, head, 32 queries) over all keys -> 32 x N values (full
                  checks), or per sampled bias row -> N values

dbias is a sum over all rows of per-row score gradients that are rounded to bf16
before they are accumulated; where those terms cancel, a few dozen neighbouring
values carry a relative error far above the tensor's (at crop640, bias ~ N(0, 4^2),
an FP64 emulation of that rounding gives up to 7e-2 on 32 keys of one bias row,
1e-2 on 64 and 3e-3 on the whole row, with 1e-6 for fp32 terms).  Its tiles are
therefore whole query rows; a lost or misplaced block of 64 keys (the kernels'
key block) or of one row chunk's partial still moves such a tile by more than 5e-2.

Each tile's error is ||x - ref||_tile / max(||ref||_tile, floor) with
floor = TILE_FLOOR * RMS(ref over the whole tensor) * sqrt(tile size): a tile whose
reference values are all (nearly) zero, such as the gradient of a masked key or
of a row without attended keys, is measured against a tenth of a typical tile's
norm instead of against zero.  A tile that is wrong wholesale (zeroed,
transposed, taken from another tile) has an error near or above 1 whatever its
norm.
"""
from __future__ import annotations

import numpy as np

TILE = 32
TILE_FLOOR = 0.1


def rel_rmse(x, ref) -> float:
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _tile_rel(diff2: np.ndarray, ref2: np.ndarray, n_tile: int, total_rms: float) -> np.ndarray:
    """Per-tile relative errors from per-tile sums of squared differences and of
    squared reference values."""
    floor = TILE_FLOOR * total_rms * np.sqrt(n_tile)
    den = np.maximum(np.sqrt(ref2), floor)
    den = np.where(den > 0, den, 1.0)
    return np.sqrt(diff2) / den


def row_tile_errors(x, ref) -> np.ndarray:
    """Tile errors of [R, N, H, D] row outputs (attended frame): one value per
    (row, 32-position tile, head).  N must be a multiple of 32."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    R, N, H, D = ref.shape
    assert x.shape == ref.shape and N % TILE == 0
    d = (x - ref).reshape(R, N // TILE, TILE, H, D)
    r = ref.reshape(R, N // TILE, TILE, H, D)
    diff2 = np.sum(d * d, axis=(2, 4))
    ref2 = np.sum(r * r, axis=(2, 4))
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return _tile_rel(diff2, ref2, TILE * D, rms)


def full_tile_errors(x, ref, ending: bool) -> np.ndarray:
    """Tile errors of a whole [B, N, N, H, D] tensor in the caller's frame, tiled
    as the kernels tile it: per (batch, attention row, 32 positions, head)."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ending:  # attended frame: the attention row is the second pair axis
        x, ref = x.swapaxes(1, 2), ref.swapaxes(1, 2)
    B, N, _, H, D = ref.shape
    return row_tile_errors(x.reshape(B * N, N, H, D), ref.reshape(B * N, N, H, D))


def dbias_tile_errors(x, ref) -> np.ndarray:
    """Tile errors of a whole [B, H, N, N] bias gradient: per (batch, head, 32
    queries), over all keys."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    B, H, N, _ = ref.shape
    assert x.shape == ref.shape and N % TILE == 0
    d = (x - ref).reshape(B, H, N // TILE, TILE * N)
    r = ref.reshape(B, H, N // TILE, TILE * N)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return _tile_rel(np.sum(d * d, axis=3), np.sum(r * r, axis=3), TILE * N, rms)


def dbias_row_tile_errors(x, ref) -> np.ndarray:
    """Tile errors of sampled bias-gradient rows [S, N]: one per row."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    S, N = ref.shape
    assert x.shape == ref.shape
    d, r = x - ref, ref
    rms = float(np.sqrt(np.mean(ref * ref)))
    return _tile_rel(np.sum(d * d, axis=1), np.sum(r * r, axis=1), N, rms)


def worst(errs: np.ndarray):
    """(largest tile error, its index) of a tile-error array."""
    if errs.size == 0:
        return 0.0, ()
    flat = int(np.nanargmax(errs)) if not np.isnan(errs).any() else int(np.argmax(np.isnan(errs)))
    idx = np.unravel_index(flat, errs.shape)
    return float(errs[idx]), tuple(int(i) for i in idx)
