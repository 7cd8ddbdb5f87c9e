"""C-ABI checks that run without a GPU.

The library must load, export every entry point that include/tri_attn.h
declares, and reject invalid or unsupported requests in host-side validation,
which runs before any HIP call (so these calls are safe on a machine without a
GPU).  Fake device addresses are used: validation never dereferences them.
"""
import ctypes
import re
from pathlib import Path

import pytest

import triangle_attention_amd as ta

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "tri_attn.h"

OK, INVALID, UNSUPPORTED, WORKSPACE, LAUNCH, ABI = 0, 1, 2, 3, 4, 5
ADDR = 1 << 40  # fake, 256-byte-aligned device address


@pytest.fixture(scope="module")
def lib():
    if not ta.LIB_PATH.exists():
        from triangle_attention_amd import build
        build.build()
    return ta.load_library()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tri_attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_exported_set():
    assert declared_functions() == sorted(ta.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.tri_attn_abi_version() == ta.ABI_VERSION
    for code in range(6):
        assert lib.tri_attn_status_string(code)
    assert lib.tri_attn_status_string(99) == b"unknown status"


def fake_ptrs(n, base=ADDR, stride=1 << 34):
    return [ctypes.c_void_p(base + i * stride) for i in range(n)]


def call_fwd(lib, prob, ptrs=None, mask=None):
    q, k, v, bias, o, res, lse = ptrs or fake_ptrs(7)
    return lib.tri_attn_fwd(ctypes.byref(prob) if prob is not None else None,
                            q, k, v, bias, mask, o, res, lse, None)


# bwd pointer order: q k v bias mask o o_residual lse d_o dq dk dv dbias workspace
def call_bwd(lib, prob, ptrs=None, ws_bytes=None):
    p = ptrs or fake_ptrs(14)
    if ws_bytes is None:
        ws_bytes = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob))
    return lib.tri_attn_bwd(ctypes.byref(prob), *p, ws_bytes, None)


def test_null_problem_is_invalid(lib):
    assert call_fwd(lib, None) == INVALID


@pytest.mark.parametrize("field,value,expect", [
    ("abi_version", ta.ABI_VERSION + 1, ABI), ("B", 0, INVALID), ("N", 0, INVALID), ("H", 0, INVALID),
    ("D", 64, UNSUPPORTED), ("D", 8, UNSUPPORTED), ("N", 48, UNSUPPORTED),
    ("N", 800, UNSUPPORTED), ("N", 1024, UNSUPPORTED), ("H", 65, UNSUPPORTED),
    ("flags", 8, UNSUPPORTED), ("softmax_scale", -1.0, INVALID),
    ("softmax_scale", float("inf"), INVALID), ("softmax_scale", float("nan"), INVALID),
])
def test_problem_validation(lib, field, value, expect):
    prob = ta.make_problem(1, 64, 4, 32)
    setattr(prob, field, value)
    assert call_fwd(lib, prob) == expect
    assert call_bwd(lib, prob, ws_bytes=1 << 40) == expect
    assert lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob)) == 0


@pytest.mark.parametrize("which", range(7))
def test_fwd_rejects_null_or_misaligned_pointers(lib, which):
    prob = ta.make_problem(1, 64, 4, 32)
    ptrs = fake_ptrs(7)
    if which == 5:  # the residual may be NULL; a misaligned one is rejected
        ptrs[5] = ctypes.c_void_p(ADDR + 5 * (1 << 34) + 4)
    else:
        ptrs[which] = None
    assert call_fwd(lib, prob, ptrs) == INVALID
    ptrs = fake_ptrs(7)
    ptrs[which] = ctypes.c_void_p(ptrs[which].value + 8)
    assert call_fwd(lib, prob, ptrs) == INVALID


def test_fwd_rejects_aliased_output(lib):
    prob = ta.make_problem(1, 64, 4, 32)
    ptrs = fake_ptrs(7)
    ptrs[4] = ptrs[0]  # o == q
    assert call_fwd(lib, prob, ptrs) == INVALID
    ptrs = fake_ptrs(7)
    ptrs[6] = ctypes.c_void_p(ptrs[4].value + 64)  # lse inside o
    assert call_fwd(lib, prob, ptrs) == INVALID


@pytest.mark.parametrize("which", [0, 1, 2, 3, 5, 7, 8, 9, 10, 11, 12, 13])
def test_bwd_rejects_null_pointers(lib, which):
    prob = ta.make_problem(1, 64, 4, 32)
    ptrs = fake_ptrs(14)
    ptrs[which] = None
    assert call_bwd(lib, prob, ptrs) == INVALID


def test_bwd_workspace_checks(lib):
    prob = ta.make_problem(1, 64, 4, 32)
    need = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob))
    assert need > 0
    assert call_bwd(lib, prob, ws_bytes=need - 1) == WORKSPACE
    ptrs = fake_ptrs(14)
    ptrs[13] = ctypes.c_void_p(ptrs[13].value + 16)  # not 256-byte aligned
    assert call_bwd(lib, prob, ptrs, need) == INVALID
    ptrs = fake_ptrs(14)
    ptrs[13] = ptrs[0]  # workspace overlapping q
    assert call_bwd(lib, prob, ptrs, need) == INVALID


def test_bwd_rejects_gradient_aliasing_an_input(lib):
    prob = ta.make_problem(1, 64, 4, 32)
    ptrs = fake_ptrs(14)
    ptrs[9] = ptrs[8]  # dq == d_o
    assert call_bwd(lib, prob, ptrs) == INVALID


def test_workspace_grows_with_problem(lib):
    sizes = [lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(1, n, 4, 32)))
             for n in (64, 256, 768)]
    assert sizes[0] < sizes[1] < sizes[2]


def test_bwd_timed_validates_before_any_hip_call(lib):
    """tri_attn_bwd_timed needs its event array, and otherwise validates exactly as
    tri_attn_bwd (five NULL events: nothing is recorded)."""
    prob = ta.make_problem(1, 64, 4, 32)
    need = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob))
    nulls = (ctypes.c_void_p * 5)()
    assert lib.tri_attn_bwd_timed(ctypes.byref(prob), *fake_ptrs(14), need, None, None) == INVALID
    ptrs = fake_ptrs(14)
    ptrs[0] = None
    assert lib.tri_attn_bwd_timed(ctypes.byref(prob), *ptrs, need, nulls, None) == INVALID
    assert lib.tri_attn_bwd_timed(ctypes.byref(prob), *fake_ptrs(14), need - 1, nulls, None) == WORKSPACE


def test_mfma_probe_library_validates_arguments():
    """The matrix-core probe bench.py reports is built with the library; invalid
    arguments are rejected before any HIP call."""
    from triangle_attention_amd import build
    if not build.PROBE_LIB.exists():
        build.build()
    probe = ctypes.CDLL(str(build.PROBE_LIB))
    probe.mfma_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    probe.mfma_probe_launch.restype = ctypes.c_int
    assert probe.mfma_probe_launch(None, 4, 10, None) == 1
    assert probe.mfma_probe_launch(ctypes.c_void_p(ADDR), 0, 10, None) == 1
    assert probe.mfma_probe_launch(ctypes.c_void_p(ADDR), 4, 0, None) == 1


def test_head_dim16_is_accepted_with_a_smaller_workspace(lib):
    """D = 16 passes host validation; its dQ partials hold 16 channels, so the
    workspace is smaller than at D = 32 (same N, H)."""
    w32 = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(1, 256, 4, 32)))
    w16 = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(1, 256, 4, 16)))
    assert 0 < w16 < w32
    prob = ta.make_problem(1, 64, 4, 16)
    ptrs = fake_ptrs(7)
    ptrs[0] = None  # validation reaches the pointer checks: the size itself is accepted
    assert call_fwd(lib, prob, ptrs) == INVALID
