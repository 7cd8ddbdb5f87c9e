"""MI355X-native triangle attention (forward and backward) — Python binding.

This module only marshals arguments: every step of the computation runs in the
HIP kernels of ``libtri_attn.so`` (built from ``csrc/tri_attn.hip``), reached
through the C ABI declared in ``include/tri_attn.h``.  PyTorch provides device
memory and the current stream.  There is no CPU or eager fallback: if the
library is missing or a call is rejected, an exception is raised.

Operation (TurboPairFormer pages: Lambda post, "Как работает TurboPairFormer"):
starting-node triangle attention with a pair bias shared by every row and a key
mask; ``ending=True`` attends along the other pair axis.  Tensor layouts:
q, k, v, dO: bf16 [B, N, N, H, D]; bias: bf16 [B, H, N, N]; mask: uint8 [B, N, N].
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "libtri_attn.so"

ABI_VERSION = 3
FLAG_ENDING_NODE = 1
FLAG_DBIAS_FP32 = 2
FLAG_RESIDUAL_BF16 = 4
RESIDUAL_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}

STATUS_NAMES = {
    0: "TRI_ATTN_SUCCESS",
    1: "TRI_ATTN_ERROR_INVALID_VALUE",
    2: "TRI_ATTN_ERROR_NOT_SUPPORTED",
    3: "TRI_ATTN_ERROR_INSUFFICIENT_WORKSPACE",
    4: "TRI_ATTN_ERROR_LAUNCH_FAILED",
    5: "TRI_ATTN_ERROR_ABI_MISMATCH",
}

EXPORTED_SYMBOLS = ("tri_attn_abi_version", "tri_attn_status_string", "tri_attn_fwd",
                    "tri_attn_bwd_workspace_bytes", "tri_attn_bwd", "tri_attn_bwd_profiled",
                    "tri_attn_bwd_timed")


class Problem(ctypes.Structure):
    """Mirror of ``tri_attn_problem``."""
    _fields_ = [("abi_version", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("B", ctypes.c_int64), ("N", ctypes.c_int64), ("H", ctypes.c_int64),
                ("D", ctypes.c_int64), ("softmax_scale", ctypes.c_float)]


class TriAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}")


_lib = None


def load_library(path: Path | str | None = None) -> ctypes.CDLL:
    """Load libtri_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is missing: build it with `python -m triangle_attention_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(str(p))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    pp = ctypes.POINTER(Problem)
    lib.tri_attn_abi_version.argtypes = []
    lib.tri_attn_abi_version.restype = i32
    lib.tri_attn_status_string.argtypes = [i32]
    lib.tri_attn_status_string.restype = ctypes.c_char_p
    lib.tri_attn_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.tri_attn_fwd.restype = i32
    lib.tri_attn_bwd_workspace_bytes.argtypes = [pp]
    lib.tri_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tri_attn_bwd.argtypes = [pp] + [vp] * 14 + [ctypes.c_size_t, vp]
    lib.tri_attn_bwd.restype = i32
    lib.tri_attn_bwd_profiled.argtypes = [pp] + [vp] * 14 + [ctypes.c_size_t, vp, vp, vp]
    lib.tri_attn_bwd_profiled.restype = i32
    lib.tri_attn_bwd_timed.argtypes = [pp] + [vp] * 14 + [ctypes.c_size_t, ctypes.POINTER(vp), vp]
    lib.tri_attn_bwd_timed.restype = i32
    if lib.tri_attn_abi_version() != ABI_VERSION:
        raise RuntimeError("libtri_attn.so ABI version mismatch")
    if path is None:
        _lib = lib
    return lib


def make_problem(B, N, H, D, *, ending=False, dbias_fp32=False, scale=None, residual="fp32",
                 abi_version=ABI_VERSION) -> Problem:
    if residual not in RESIDUAL_DTYPES:
        raise ValueError("residual must be 'fp32' or 'bf16'")
    flags = ((FLAG_ENDING_NODE if ending else 0) | (FLAG_DBIAS_FP32 if dbias_fp32 else 0)
             | (FLAG_RESIDUAL_BF16 if residual == "bf16" else 0))
    return Problem(abi_version, flags, B, N, H, D, float(scale or 0.0))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_inputs(q, k, v, bias, mask):
    for name, t in (("q", q), ("k", k), ("v", v), ("bias", bias)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
    if q.dim() != 5 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share the shape [B, N, N, H, D]")
    B, N, N2, H, D = q.shape
    if N2 != N or tuple(bias.shape) != (B, H, N, N):
        raise ValueError("bias must be [B, H, N, N] with q of shape [B, N, N, H, D]")
    if mask is not None and (mask.dtype != torch.uint8 or tuple(mask.shape) != (B, N, N)
                             or not mask.is_contiguous() or not mask.is_cuda):
        raise ValueError("mask must be a contiguous uint8 CUDA tensor [B, N, N]")
    return B, N, H, D


def tri_attn_fwd(q, k, v, bias, mask=None, *, ending=False, scale=None, save_residual=True,
                 residual="fp32"):
    """Forward: returns (o bf16, o_residual or None, lse fp32 [B, N, H, N]); the residual
    O - float(o) is fp32 (exact), or its bf16 rounding with residual="bf16"."""
    B, N, H, D = _check_inputs(q, k, v, bias, mask)
    lib = load_library()
    prob = make_problem(B, N, H, D, ending=ending, scale=scale, residual=residual)
    o = torch.empty_like(q)
    res = torch.empty(q.shape, dtype=RESIDUAL_DTYPES[residual], device=q.device) if save_residual else None
    lse = torch.empty((B, N, H, N), dtype=torch.float32, device=q.device)
    st = lib.tri_attn_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask),
                          _ptr(o), _ptr(res), _ptr(lse), _stream(q.device))
    if st != 0:
        raise TriAttnError(st, "tri_attn_fwd")
    return o, res, lse


def bwd_workspace_bytes(B, N, H, D, *, ending=False, dbias_fp32=False, scale=None) -> int:
    lib = load_library()
    prob = make_problem(B, N, H, D, ending=ending, dbias_fp32=dbias_fp32, scale=scale)
    return int(lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob)))


def tri_attn_bwd(q, k, v, bias, mask, o, o_residual, lse, d_o, *, ending=False, scale=None,
                 dbias_fp32=False, workspace=None, main_events=None, kernel_events=None):
    """Backward: returns (dq, dk, dv, dbias).  o_residual=None selects the
    uncompensated softmax correction rowsum(dO * float(o)); a bf16 o_residual is
    passed with the bf16-residual flag.  main_events, a pair of raw hipEvent_t
    handles (ints), is recorded around the main kernel; kernel_events, five raw
    handles, around each of the four backward kernels (tri_attn_bwd_timed)."""
    B, N, H, D = _check_inputs(q, k, v, bias, mask)
    lib = load_library()
    if o_residual is not None and o_residual.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("o_residual must be bf16 or fp32")
    residual = "bf16" if o_residual is not None and o_residual.dtype == torch.bfloat16 else "fp32"
    prob = make_problem(B, N, H, D, ending=ending, dbias_fp32=dbias_fp32, scale=scale,
                        residual=residual)
    nbytes = int(lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob)))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dbias = torch.empty(bias.shape, dtype=torch.float32 if dbias_fp32 else torch.bfloat16,
                        device=q.device)
    args = (ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask),
            _ptr(o), _ptr(o_residual), _ptr(lse), _ptr(d_o.contiguous()),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(workspace), workspace.numel())
    if kernel_events is not None:
        if len(kernel_events) != 5:
            raise ValueError("kernel_events must hold five hipEvent_t handles")
        evs = (ctypes.c_void_p * 5)(*[ctypes.c_void_p(e) for e in kernel_events])
        st = lib.tri_attn_bwd_timed(*args, evs, _stream(q.device))
    elif main_events is None:
        st = lib.tri_attn_bwd(*args, _stream(q.device))
    else:
        ev = [ctypes.c_void_p(e) for e in main_events]
        st = lib.tri_attn_bwd_profiled(*args, ev[0], ev[1], _stream(q.device))
    if st != 0:
        raise TriAttnError(st, "tri_attn_bwd")
    return dq, dk, dv, dbias


class TriAttnFunction(torch.autograd.Function):
    """Autograd wrapper: the forward saves o, its residual and lse; the backward
    recomputes every probability tile once inside the HIP kernels."""

    @staticmethod
    def forward(ctx, q, k, v, bias, mask, ending, scale):
        o, res, lse = tri_attn_fwd(q, k, v, bias, mask, ending=ending, scale=scale)
        ctx.save_for_backward(q, k, v, bias, mask, o, res, lse)
        ctx.ending, ctx.scale = ending, scale
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, bias, mask, o, res, lse = ctx.saved_tensors
        dq, dk, dv, dbias = tri_attn_bwd(q, k, v, bias, mask, o, res, lse,
                                         d_o.to(torch.bfloat16), ending=ctx.ending,
                                         scale=ctx.scale)
        return dq, dk, dv, dbias, None, None, None


def tri_attn(q, k, v, bias, mask=None, ending=False, scale=None):
    """Differentiable triangle attention (bf16 output)."""
    return TriAttnFunction.apply(q, k, v, bias, mask, ending, scale)


__all__ = ["tri_attn", "tri_attn_fwd", "tri_attn_bwd", "bwd_workspace_bytes", "load_library",
           "make_problem", "Problem", "TriAttnError", "TriAttnFunction", "LIB_PATH",
           "EXPORTED_SYMBOLS"]
