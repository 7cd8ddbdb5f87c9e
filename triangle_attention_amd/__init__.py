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

ABI_VERSION = 4
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
                    "tri_attn_bwd_workspace_bytes", "tri_attn_bwd", "tri_attn_bwd_timed",
                    "tri_attn_bwd_noalloc", "tri_mul_abi_version", "tri_mul_fwd", "tri_mul_bwd",
                    "tri_attn_module_abi_version", "tri_attn_module_fwd", "tri_attn_module_bwd_workspace_bytes",
                    "tri_attn_module_bwd", "tri_mul_module_abi_version", "tri_mul_module_fwd",
                    "tri_mul_module_bwd_workspace_bytes", "tri_mul_module_bwd")
TRI_MUL_ABI_VERSION = 1
TRI_MUL_MODULE_ABI_VERSION = 1
MODULE_ABI_VERSION = 1
MODULE_CHANNELS = 128
TRI_MUL_FLAG_INCOMING = 1
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024   # TRI_ATTN_NOALLOC_SCRATCH_BYTES


class Problem(ctypes.Structure):
    """Mirror of ``tri_attn_problem``."""
    _fields_ = [("abi_version", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("B", ctypes.c_int64), ("N", ctypes.c_int64), ("H", ctypes.c_int64),
                ("D", ctypes.c_int64), ("softmax_scale", ctypes.c_float),
                ("row_begin", ctypes.c_int64), ("row_end", ctypes.c_int64)]


class TriMulProblem(ctypes.Structure):
    """Mirror of ``tri_mul_problem``."""
    _fields_ = [("abi_version", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("B", ctypes.c_int64), ("N", ctypes.c_int64), ("C", ctypes.c_int64)]


class ModuleProblem(ctypes.Structure):
    """Mirror of ``tri_attn_module_problem``."""
    _fields_ = [("abi_version", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("B", ctypes.c_int64), ("N", ctypes.c_int64), ("H", ctypes.c_int64),
                ("D", ctypes.c_int64), ("ln_eps", ctypes.c_float)]


class ModuleParams(ctypes.Structure):
    """Mirror of ``tri_attn_module_params`` (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln_w", "ln_b", "w_qkvg", "w_bias", "w_out")]


class ModuleSaved(ctypes.Structure):
    """Mirror of ``tri_attn_module_saved`` (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("zn", "ln_stats", "q", "k", "v", "g", "bias", "o",
                                                "o_residual", "lse")]


class ModuleGrads(ctypes.Structure):
    """Mirror of ``tri_attn_module_param_grads`` (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln_w", "ln_b", "w_qkvg", "w_bias", "w_out")]


class TriMulModuleProblem(ctypes.Structure):
    """Mirror of ``tri_mul_module_problem``."""
    _fields_ = [("abi_version", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("B", ctypes.c_int64), ("N", ctypes.c_int64), ("C", ctypes.c_int64), ("ln_eps", ctypes.c_float)]


TRI_MUL_MODULE_PARAMS = ("ln_in_w", "ln_in_b", "w_in", "ln_out_w", "ln_out_b", "w_out")
TRI_MUL_MODULE_SAVED = ("zn", "ln_in_stats", "a", "b", "g", "x", "xn", "ln_out_stats")


class TriMulModuleParams(ctypes.Structure):
    """Mirror of ``tri_mul_module_params`` and ``tri_mul_module_param_grads`` (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in TRI_MUL_MODULE_PARAMS]


class TriMulModuleSaved(ctypes.Structure):
    """Mirror of ``tri_mul_module_saved`` (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in TRI_MUL_MODULE_SAVED]


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
    lib.tri_attn_bwd_timed.argtypes = [pp] + [vp] * 14 + [ctypes.c_size_t, ctypes.POINTER(vp), vp]
    lib.tri_attn_bwd_timed.restype = i32
    lib.tri_attn_bwd_noalloc.argtypes = [pp] + [vp] * 13 + [vp]
    lib.tri_attn_bwd_noalloc.restype = i32
    tp = ctypes.POINTER(TriMulProblem)
    lib.tri_mul_abi_version.argtypes = []
    lib.tri_mul_abi_version.restype = i32
    lib.tri_mul_fwd.argtypes = [tp, vp, vp, vp, vp]
    lib.tri_mul_fwd.restype = i32
    lib.tri_mul_bwd.argtypes = [tp, vp, vp, vp, vp, vp, vp]
    lib.tri_mul_bwd.restype = i32
    mp = ctypes.POINTER(ModuleProblem)
    lib.tri_attn_module_abi_version.argtypes = []
    lib.tri_attn_module_abi_version.restype = i32
    lib.tri_attn_module_fwd.argtypes = [mp, vp, vp, ctypes.POINTER(ModuleParams), vp, ctypes.POINTER(ModuleSaved), vp]
    lib.tri_attn_module_fwd.restype = i32
    lib.tri_attn_module_bwd_workspace_bytes.argtypes = [mp]
    lib.tri_attn_module_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tri_attn_module_bwd.argtypes = [mp, vp, vp, ctypes.POINTER(ModuleParams), ctypes.POINTER(ModuleSaved), vp, vp,
                                        ctypes.POINTER(ModuleGrads), vp, ctypes.c_size_t, vp]
    lib.tri_attn_module_bwd.restype = i32
    tp2 = ctypes.POINTER(TriMulModuleProblem)
    lib.tri_mul_module_abi_version.argtypes = []
    lib.tri_mul_module_abi_version.restype = i32
    lib.tri_mul_module_fwd.argtypes = [tp2, vp, vp, ctypes.POINTER(TriMulModuleParams), vp,
                                       ctypes.POINTER(TriMulModuleSaved), vp]
    lib.tri_mul_module_fwd.restype = i32
    lib.tri_mul_module_bwd_workspace_bytes.argtypes = [tp2]
    lib.tri_mul_module_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.tri_mul_module_bwd.argtypes = [tp2, vp, vp, ctypes.POINTER(TriMulModuleParams),
                                       ctypes.POINTER(TriMulModuleSaved), vp, vp,
                                       ctypes.POINTER(TriMulModuleParams), vp, ctypes.c_size_t, vp]
    lib.tri_mul_module_bwd.restype = i32
    if (lib.tri_attn_abi_version() != ABI_VERSION or lib.tri_mul_abi_version() != TRI_MUL_ABI_VERSION
            or lib.tri_attn_module_abi_version() != MODULE_ABI_VERSION
            or lib.tri_mul_module_abi_version() != TRI_MUL_MODULE_ABI_VERSION):
        raise RuntimeError("libtri_attn.so ABI version mismatch")
    if path is None:
        _lib = lib
    return lib


def make_problem(B, N, H, D, *, ending=False, dbias_fp32=False, scale=None, residual="fp32",
                 rows=None, abi_version=ABI_VERSION) -> Problem:
    """rows = (row_begin, row_end): the attention rows of the call (None: all rows)."""
    if residual not in RESIDUAL_DTYPES:
        raise ValueError("residual must be 'fp32' or 'bf16'")
    flags = ((FLAG_ENDING_NODE if ending else 0) | (FLAG_DBIAS_FP32 if dbias_fp32 else 0)
             | (FLAG_RESIDUAL_BF16 if residual == "bf16" else 0))
    r0, r1 = (0, 0) if rows is None else (int(rows[0]), int(rows[1]))
    return Problem(abi_version, flags, B, N, H, D, float(scale or 0.0), r0, r1)


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
    for name, t in (("k", k), ("v", v), ("bias", bias), ("mask", mask)):
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} must be on the device of q")
    return B, N, H, D


def _check_tensor(name, t, shape, dtypes, device):
    """A tensor the library reads or writes: exact shape, dtype, device, contiguity."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be of dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (the device of q)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def tri_attn_fwd(q, k, v, bias, mask=None, *, ending=False, scale=None, save_residual=True,
                 residual="fp32", out=None, rows=None):
    """Forward: returns (o bf16, o_residual or None, lse fp32 [B, N, H, N]); the residual
    O - float(o) is fp32 (exact), or its bf16 rounding with residual="bf16".  `out`, if
    given, is a tuple (o, o_residual, lse) of preallocated outputs written in place
    (o_residual may be None, which then also means save_residual=False).  rows =
    (row_begin, row_end) computes only those attention rows; the other rows of the
    outputs are left as they are (uninitialised when the outputs are allocated here)."""
    B, N, H, D = _check_inputs(q, k, v, bias, mask)
    if residual not in RESIDUAL_DTYPES:
        raise ValueError("residual must be 'fp32' or 'bf16'")
    if out is not None:
        o, res, lse = out
        _check_tensor("o", o, q.shape, (torch.bfloat16,), q.device)
        if res is not None:
            _check_tensor("o_residual", res, q.shape, (RESIDUAL_DTYPES[residual],), q.device)
        _check_tensor("lse", lse, (B, N, H, N), (torch.float32,), q.device)
    lib = load_library()
    prob = make_problem(B, N, H, D, ending=ending, scale=scale, residual=residual, rows=rows)
    if out is None:
        o = torch.empty_like(q)
        res = torch.empty(q.shape, dtype=RESIDUAL_DTYPES[residual], device=q.device) if save_residual else None
        lse = torch.empty((B, N, H, N), dtype=torch.float32, device=q.device)
    st = lib.tri_attn_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask),
                          _ptr(o), _ptr(res), _ptr(lse), _stream(q.device))
    if st != 0:
        raise TriAttnError(st, "tri_attn_fwd")
    return o, res, lse


def bwd_workspace_bytes(B, N, H, D, *, ending=False, dbias_fp32=False, scale=None, rows=None) -> int:
    lib = load_library()
    prob = make_problem(B, N, H, D, ending=ending, dbias_fp32=dbias_fp32, scale=scale, rows=rows)
    return int(lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob)))


def tri_attn_bwd(q, k, v, bias, mask, o, o_residual, lse, d_o, *, ending=False, scale=None,
                 dbias_fp32=False, workspace=None, kernel_events=None, out=None, rows=None):
    """Backward: returns (dq, dk, dv, dbias).  o_residual=None selects the
    uncompensated softmax correction rowsum(dO * float(o)); a bf16 o_residual is
    passed with the bf16-residual flag.  o, o_residual, lse and d_o must match the
    problem of q exactly (shape, dtype, device, contiguity): the kernels read them
    without bounds.  kernel_events, five raw hipEvent_t handles (ints), are recorded
    around each of the four backward kernels (tri_attn_bwd_timed).  `out`, if given,
    is a tuple (dq, dk, dv, dbias) of preallocated outputs written in place;
    `workspace` a uint8 device tensor of at least bwd_workspace_bytes bytes.  rows =
    (row_begin, row_end): gradients of those attention rows only, and dbias the
    range's unreduced partial sum over its rows."""
    B, N, H, D = _check_inputs(q, k, v, bias, mask)
    _check_tensor("o", o, q.shape, (torch.bfloat16,), q.device)
    if o_residual is not None:
        _check_tensor("o_residual", o_residual, q.shape, (torch.bfloat16, torch.float32), q.device)
    _check_tensor("lse", lse, (B, N, H, N), (torch.float32,), q.device)
    _check_tensor("d_o", d_o, q.shape, (torch.bfloat16,), q.device)
    lib = load_library()
    residual = "bf16" if o_residual is not None and o_residual.dtype == torch.bfloat16 else "fp32"
    prob = make_problem(B, N, H, D, ending=ending, dbias_fp32=dbias_fp32, scale=scale,
                        residual=residual, rows=rows)
    nbytes = int(lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    elif (workspace.dtype != torch.uint8 or workspace.device != q.device or not workspace.is_contiguous()
          or workspace.numel() < nbytes):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {nbytes} bytes on {q.device}")
    db_dtype = torch.float32 if dbias_fp32 else torch.bfloat16
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dbias = torch.empty(bias.shape, dtype=db_dtype, device=q.device)
    else:
        dq, dk, dv, dbias = out
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _check_tensor(name, t, q.shape, (torch.bfloat16,), q.device)
        _check_tensor("dbias", dbias, bias.shape, (db_dtype,), q.device)
    args = (ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask),
            _ptr(o), _ptr(o_residual), _ptr(lse), _ptr(d_o),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(workspace), workspace.numel())
    if kernel_events is not None:
        if len(kernel_events) != 5:
            raise ValueError("kernel_events must hold five hipEvent_t handles")
        evs = (ctypes.c_void_p * 5)(*[ctypes.c_void_p(e) for e in kernel_events])
        st = lib.tri_attn_bwd_timed(*args, evs, _stream(q.device))
    else:
        st = lib.tri_attn_bwd(*args, _stream(q.device))
    if st != 0:
        raise TriAttnError(st, "tri_attn_bwd")
    return dq, dk, dv, dbias


def tri_attn_bwd_noalloc(q, k, v, bias, mask, o, o_residual, lse, d_o, out, *, ending=False,
                         scale=None, dbias_fp32=False, rows=None):
    """tri_attn_bwd_noalloc: the backward with its workspace in the library's fixed
    device buffer, for callers that cannot allocate.  `out` = (dq, dk, dv, dbias) must
    be preallocated; nothing is allocated here.  Problems whose workspace exceeds
    NOALLOC_SCRATCH_BYTES raise TriAttnError (TRI_ATTN_ERROR_INSUFFICIENT_WORKSPACE)."""
    B, N, H, D = _check_inputs(q, k, v, bias, mask)
    _check_tensor("o", o, q.shape, (torch.bfloat16,), q.device)
    if o_residual is not None:
        _check_tensor("o_residual", o_residual, q.shape, (torch.bfloat16, torch.float32), q.device)
    _check_tensor("lse", lse, (B, N, H, N), (torch.float32,), q.device)
    _check_tensor("d_o", d_o, q.shape, (torch.bfloat16,), q.device)
    dq, dk, dv, dbias = out
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, (torch.bfloat16,), q.device)
    _check_tensor("dbias", dbias, bias.shape, (torch.float32 if dbias_fp32 else torch.bfloat16,), q.device)
    lib = load_library()
    residual = "bf16" if o_residual is not None and o_residual.dtype == torch.bfloat16 else "fp32"
    prob = make_problem(B, N, H, D, ending=ending, dbias_fp32=dbias_fp32, scale=scale,
                        residual=residual, rows=rows)
    st = lib.tri_attn_bwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask),
                                  _ptr(o), _ptr(o_residual), _ptr(lse), _ptr(d_o),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _stream(q.device))
    if st != 0:
        raise TriAttnError(st, "tri_attn_bwd_noalloc")
    return dq, dk, dv, dbias


# ---- triangle multiplicative update: the contraction (include/tri_mul.h) ----

def make_trimul_problem(B, N, C, *, incoming=False, abi_version=TRI_MUL_ABI_VERSION) -> TriMulProblem:
    return TriMulProblem(abi_version, TRI_MUL_FLAG_INCOMING if incoming else 0, B, N, C)


def _check_trimul(x):
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() != 4 or x.shape[2] != x.shape[3]:
        raise ValueError("triangle multiplication operands are contiguous bf16 CUDA tensors [B, C, N, N]")
    return tuple(x.shape)


def tri_mul_fwd(a, b, *, incoming=False, out=None):
    """z = the outgoing (or incoming) contraction of a and b, all bf16 [B, C, N, N]."""
    B, C, N, _ = _check_trimul(a)
    for name, t in (("b", b),) + ((("out", out),) if out is not None else ()):
        _check_tensor(name, t, a.shape, (torch.bfloat16,), a.device)
    lib = load_library()
    z = torch.empty_like(a) if out is None else out
    st = lib.tri_mul_fwd(ctypes.byref(make_trimul_problem(B, N, C, incoming=incoming)), _ptr(a), _ptr(b),
                         _ptr(z), _stream(a.device))
    if st != 0:
        raise TriAttnError(st, "tri_mul_fwd")
    return z


def tri_mul_bwd(a, b, dz, *, incoming=False, out=None):
    """(da, db) of the contraction for the upstream gradient dz, all bf16 [B, C, N, N]."""
    B, C, N, _ = _check_trimul(a)
    for name, t in (("b", b), ("dz", dz)):
        _check_tensor(name, t, a.shape, (torch.bfloat16,), a.device)
    if out is None:
        da, db = torch.empty_like(a), torch.empty_like(a)
    else:
        da, db = out
        for name, t in (("da", da), ("db", db)):
            _check_tensor(name, t, a.shape, (torch.bfloat16,), a.device)
    lib = load_library()
    st = lib.tri_mul_bwd(ctypes.byref(make_trimul_problem(B, N, C, incoming=incoming)), _ptr(a), _ptr(b),
                         _ptr(dz), _ptr(da), _ptr(db), _stream(a.device))
    if st != 0:
        raise TriAttnError(st, "tri_mul_bwd")
    return da, db


# ---- the triangle-attention module around the core (include/tri_module.h) ----

def make_module_problem(B, N, H, D, *, ending=False, eps=0.0, abi_version=MODULE_ABI_VERSION) -> ModuleProblem:
    return ModuleProblem(abi_version, FLAG_ENDING_NODE if ending else 0, B, N, H, D, float(eps))


def _module_params(params, C, H, dev):
    """params: dict ln_w, ln_b (fp32 [C]), w_qkvg (bf16 [C, 4C]), w_bias (bf16 [C, H]), w_out (bf16 [C, C])."""
    shapes = {"ln_w": ((C,), torch.float32), "ln_b": ((C,), torch.float32), "w_qkvg": ((C, 4 * C), torch.bfloat16),
              "w_bias": ((C, H), torch.bfloat16), "w_out": ((C, C), torch.bfloat16)}
    for n, (shape, dt) in shapes.items():
        _check_tensor(n, params[n], shape, (dt,), dev)
    return ModuleParams(*(params[n].data_ptr() for n in ("ln_w", "ln_b", "w_qkvg", "w_bias", "w_out")))


def _module_dims(z, H):
    if z.dtype != torch.bfloat16 or not z.is_cuda or not z.is_contiguous() or z.dim() != 4 or z.shape[1] != z.shape[2]:
        raise ValueError("z is a contiguous bf16 CUDA tensor [B, N, N, C]")
    B, N, _, C = z.shape
    if C % H:
        raise ValueError("the channel count must be a multiple of H")
    return B, N, C, C // H


def tri_attn_module_fwd(z, mask, params, H, *, ending=False, eps=0.0):
    """Forward of the triangle-attention block: returns (y, saved) where saved is the dict
    of the activations tri_attn_module_bwd needs (all allocated here)."""
    B, N, C, D = _module_dims(z, H)
    dev = z.device
    if mask is not None:
        _check_tensor("mask", mask, (B, N, N), (torch.uint8,), dev)
    p = _module_params(params, C, H, dev)
    e = dict(dtype=torch.bfloat16, device=dev)
    saved = {"zn": torch.empty_like(z), "ln_stats": torch.empty((B, N, N, 2), dtype=torch.float32, device=dev),
             "q": torch.empty((B, N, N, H, D), **e), "k": torch.empty((B, N, N, H, D), **e),
             "v": torch.empty((B, N, N, H, D), **e), "g": torch.empty_like(z),
             "bias": torch.empty((B, H, N, N), **e), "o": torch.empty((B, N, N, H, D), **e),
             "o_residual": torch.empty((B, N, N, H, D), dtype=torch.float32, device=dev),
             "lse": torch.empty((B, N, H, N), dtype=torch.float32, device=dev)}
    y = torch.empty_like(z)
    sv = ModuleSaved(*(saved[n].data_ptr() for n, _ in ModuleSaved._fields_))
    lib = load_library()
    st = lib.tri_attn_module_fwd(ctypes.byref(make_module_problem(B, N, H, D, ending=ending, eps=eps)), _ptr(z),
                                 _ptr(mask), ctypes.byref(p), _ptr(y), ctypes.byref(sv), _stream(dev))
    if st != 0:
        raise TriAttnError(st, "tri_attn_module_fwd")
    return y, saved


def module_bwd_workspace_bytes(B, N, H, D, *, ending=False) -> int:
    return load_library().tri_attn_module_bwd_workspace_bytes(ctypes.byref(make_module_problem(B, N, H, D,
                                                                                                ending=ending)))


def tri_attn_module_bwd(z, mask, params, saved, dy, H, *, ending=False, eps=0.0, workspace=None):
    """Backward of the block: returns (dz, grads) with grads the dict of fp32 parameter
    gradients (ln_w, ln_b, w_qkvg, w_bias, w_out)."""
    B, N, C, D = _module_dims(z, H)
    dev = z.device
    _check_tensor("dy", dy, z.shape, (torch.bfloat16,), dev)
    if mask is not None:
        _check_tensor("mask", mask, (B, N, N), (torch.uint8,), dev)
    p = _module_params(params, C, H, dev)
    sv = ModuleSaved(*(saved[n].data_ptr() for n, _ in ModuleSaved._fields_))
    grads = {n: torch.empty(params[n].shape, dtype=torch.float32, device=dev)
             for n in ("ln_w", "ln_b", "w_qkvg", "w_bias", "w_out")}
    gr = ModuleGrads(*(grads[n].data_ptr() for n, _ in ModuleGrads._fields_))
    dz = torch.empty_like(z)
    prob = make_module_problem(B, N, H, D, ending=ending, eps=eps)
    lib = load_library()
    need = lib.tri_attn_module_bwd_workspace_bytes(ctypes.byref(prob))
    if need == 0:
        raise TriAttnError(2, "tri_attn_module_bwd")
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if workspace is None else workspace
    st = lib.tri_attn_module_bwd(ctypes.byref(prob), _ptr(z), _ptr(mask), ctypes.byref(p), ctypes.byref(sv),
                                 _ptr(dy), _ptr(dz), ctypes.byref(gr), _ptr(ws), ws.numel(), _stream(dev))
    if st != 0:
        raise TriAttnError(st, "tri_attn_module_bwd")
    return dz, grads


# ---- the triangle multiplicative update block (include/tri_mul_module.h) ----

def make_trimul_module_problem(B, N, C, *, incoming=False, eps=0.0,
                               abi_version=TRI_MUL_MODULE_ABI_VERSION) -> TriMulModuleProblem:
    return TriMulModuleProblem(abi_version, TRI_MUL_FLAG_INCOMING if incoming else 0, B, N, C, float(eps))


def _trimul_module_params(params, C, dev):
    shapes = {"ln_in_w": ((C,), torch.float32), "ln_in_b": ((C,), torch.float32),
              "w_in": ((C, 5 * C), torch.bfloat16), "ln_out_w": ((C,), torch.float32),
              "ln_out_b": ((C,), torch.float32), "w_out": ((C, C), torch.bfloat16)}
    for n, (shape, dt) in shapes.items():
        _check_tensor(n, params[n], shape, (dt,), dev)
    return TriMulModuleParams(*(params[n].data_ptr() for n in TRI_MUL_MODULE_PARAMS))


def tri_mul_module_fwd(z, mask, params, *, incoming=False, eps=0.0):
    """Forward of the triangle multiplicative update block: returns (y, saved)."""
    B, N, C, _ = _module_dims(z, 1)
    dev = z.device
    if mask is not None:
        _check_tensor("mask", mask, (B, N, N), (torch.uint8,), dev)
    p = _trimul_module_params(params, C, dev)
    cm = dict(dtype=torch.bfloat16, device=dev)
    saved = {"zn": torch.empty_like(z), "ln_in_stats": torch.empty((B, N, N, 2), dtype=torch.float32, device=dev),
             "a": torch.empty((B, C, N, N), **cm), "b": torch.empty((B, C, N, N), **cm), "g": torch.empty_like(z),
             "x": torch.empty((B, C, N, N), **cm), "xn": torch.empty_like(z),
             "ln_out_stats": torch.empty((B, N, N, 2), dtype=torch.float32, device=dev)}
    y = torch.empty_like(z)
    sv = TriMulModuleSaved(*(saved[n].data_ptr() for n in TRI_MUL_MODULE_SAVED))
    lib = load_library()
    st = lib.tri_mul_module_fwd(ctypes.byref(make_trimul_module_problem(B, N, C, incoming=incoming, eps=eps)),
                                _ptr(z), _ptr(mask), ctypes.byref(p), _ptr(y), ctypes.byref(sv), _stream(dev))
    if st != 0:
        raise TriAttnError(st, "tri_mul_module_fwd")
    return y, saved


def trimul_module_bwd_workspace_bytes(B, N, C, *, incoming=False) -> int:
    return load_library().tri_mul_module_bwd_workspace_bytes(
        ctypes.byref(make_trimul_module_problem(B, N, C, incoming=incoming)))


def tri_mul_module_bwd(z, mask, params, saved, dy, *, incoming=False, eps=0.0, workspace=None):
    """Backward of the block: returns (dz, grads), grads the fp32 parameter gradients."""
    B, N, C, _ = _module_dims(z, 1)
    dev = z.device
    _check_tensor("dy", dy, z.shape, (torch.bfloat16,), dev)
    if mask is not None:
        _check_tensor("mask", mask, (B, N, N), (torch.uint8,), dev)
    p = _trimul_module_params(params, C, dev)
    sv = TriMulModuleSaved(*(saved[n].data_ptr() for n in TRI_MUL_MODULE_SAVED))
    grads = {n: torch.empty(params[n].shape, dtype=torch.float32, device=dev) for n in TRI_MUL_MODULE_PARAMS}
    gr = TriMulModuleParams(*(grads[n].data_ptr() for n in TRI_MUL_MODULE_PARAMS))
    dz = torch.empty_like(z)
    prob = make_trimul_module_problem(B, N, C, incoming=incoming, eps=eps)
    lib = load_library()
    need = lib.tri_mul_module_bwd_workspace_bytes(ctypes.byref(prob))
    if need == 0:
        raise TriAttnError(2, "tri_mul_module_bwd")
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if workspace is None else workspace
    st = lib.tri_mul_module_bwd(ctypes.byref(prob), _ptr(z), _ptr(mask), ctypes.byref(p), ctypes.byref(sv),
                                _ptr(dy), _ptr(dz), ctypes.byref(gr), _ptr(ws), ws.numel(), _stream(dev))
    if st != 0:
        raise TriAttnError(st, "tri_mul_module_bwd")
    return dz, grads


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
                                         d_o.to(torch.bfloat16).contiguous(), ending=ctx.ending,
                                         scale=ctx.scale)
        return dq, dk, dv, dbias, None, None, None


def tri_attn(q, k, v, bias, mask=None, ending=False, scale=None):
    """Differentiable triangle attention (bf16 output)."""
    return TriAttnFunction.apply(q, k, v, bias, mask, ending, scale)


__all__ = ["tri_attn", "tri_attn_fwd", "tri_attn_bwd", "tri_attn_bwd_noalloc", "bwd_workspace_bytes",
           "tri_mul_fwd", "tri_mul_bwd", "make_trimul_problem", "TriMulProblem",
           "tri_attn_module_fwd", "tri_attn_module_bwd", "module_bwd_workspace_bytes", "make_module_problem",
           "ModuleProblem", "ModuleParams", "ModuleSaved", "ModuleGrads",
           "tri_mul_module_fwd", "tri_mul_module_bwd", "trimul_module_bwd_workspace_bytes",
           "make_trimul_module_problem", "TriMulModuleProblem",
           "load_library", "NOALLOC_SCRATCH_BYTES",
           "make_problem", "Problem", "TriAttnError", "TriAttnFunction", "LIB_PATH",
           "EXPORTED_SYMBOLS"]
