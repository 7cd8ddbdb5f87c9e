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
HEADERS = (HEADER, ROOT / "include" / "tri_mul.h", ROOT / "include" / "tri_module.h",
           ROOT / "include" / "tri_mul_module.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, LAUNCH, ABI = 0, 1, 2, 3, 4, 5
ADDR = 1 << 40  # fake, 256-byte-aligned device address


@pytest.fixture(scope="module")
def lib():
    if not ta.LIB_PATH.exists():
        from triangle_attention_amd import build
        build.build()
    return ta.load_library()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        names |= set(re.findall(r"\b(tri_(?:attn|mul)_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_exported_set():
    assert declared_functions() == sorted(ta.EXPORTED_SYMBOLS)


def declaration_comments():
    """The comment block directly above each declared call in the headers."""
    out = {}
    for h in HEADERS:
        text = h.read_text()
        for m in re.finditer(r"/\*((?:(?!\*/).)*)\*/\s*(?:[A-Za-z_][A-Za-z_0-9 ]*\*?\s*)(tri_(?:attn|mul)_[a-z_]+)\s*\(",
                             text, flags=re.S):
            out[m.group(2)] = re.sub(r"\s*\n\s*\*?\s*", " ", m.group(1))   # one line, no leading '*'
    return out


# the allocation-free variant of the backward: its comment names the callers it is
# for (those that cannot allocate) instead of a page passage
NO_ALLOC_VARIANT = "tri_attn_bwd_noalloc"


def test_every_declared_call_cites_the_pages():
    """Each entry point's comment names the page passage that defines it: the Lambda
    post (dev48.org translation) or the biocloudservice page, with a section."""
    comments = declaration_comments()
    assert sorted(comments) == declared_functions()
    for name, c in comments.items():
        if name == NO_ALLOC_VARIANT:
            assert "cannot allocate" in c and "graph capture" in c, name
            continue
        assert ("Lambda post" in c) or ("biocloudservice page" in c), name
        assert re.search(r'"[^"]+"', c), name   # a quoted section title


def test_noalloc_validates_and_rejects_oversized_problems(lib):
    """Host-side checks of the allocation-free backward run before the fixed
    buffer's address is looked up: invalid problems and problems whose workspace
    exceeds the buffer are rejected (no HIP device needed)."""
    lib.tri_attn_bwd_noalloc.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 14
    p = fake_ptrs(13)
    bad = ta.make_problem(1, 64, 4, 32)
    bad.N = 0
    assert lib.tri_attn_bwd_noalloc(ctypes.byref(bad), *p, None) == INVALID
    unsupported = ta.make_problem(1, 64, 4, 128)
    assert lib.tri_attn_bwd_noalloc(ctypes.byref(unsupported), *p, None) == UNSUPPORTED
    big = ta.make_problem(1, 768, 4, 32)
    assert lib.tri_attn_bwd_workspace_bytes(ctypes.byref(big)) > ta.NOALLOC_SCRATCH_BYTES
    assert lib.tri_attn_bwd_noalloc(ctypes.byref(big), *p, None) == WORKSPACE
    small = ta.make_problem(1, 256, 4, 32)
    assert lib.tri_attn_bwd_workspace_bytes(ctypes.byref(small)) <= ta.NOALLOC_SCRATCH_BYTES


def test_noalloc_buffer_size_matches_the_header():
    text = HEADER.read_text()
    m = re.search(r"#define TRI_ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    assert m and int(m.group(1)) * 1024 * 1024 == ta.NOALLOC_SCRATCH_BYTES


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
    ("D", 128, UNSUPPORTED), ("D", 48, UNSUPPORTED), ("D", 8, UNSUPPORTED), ("N", 48, UNSUPPORTED),
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


def test_workspace_is_about_half_a_bf16_score_gradient(lib):
    """The backward never holds the score gradient dS (B N^3 H bf16 values, 3.62 GB at
    crop768): its workspace, dominated by one bf16 dQ partial per 64-key block (N / 64
    partials of B N^2 H D values), is D / 64 of it plus the per-query statistics and the
    dbias partials, about 0.52 at N = 768, H = 4, D = 32."""
    B, N, H, D = 1, 768, 4, 32
    ws = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(B, N, H, D)))
    ds_bytes = B * N ** 3 * H * 2
    partials = (N // 64) * B * N * N * H * D * 2
    assert partials <= ws
    assert 0.5 < ws / ds_bytes < 0.55, ws / ds_bytes


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


def test_head_dim64_is_accepted_with_32_key_blocks(lib):
    """D = 64 passes host validation; its backward keeps one bf16 dQ partial of 64
    channels per 32-key block, so the workspace holds N / 32 of them (and the row
    chunks of B * H * N / 32 workgroup groups)."""
    import bench
    B, N, H, D = 1, 256, 2, 64

    def a256(x):
        return (x + 255) // 256 * 256
    T = N // 32
    C = bench.row_chunks(B * H * T, N)
    want = a256(B * N * H * 2 * N * 4) + a256(T * B * N * N * H * D * 2) + a256(C * B * H * N * N * 4)
    assert lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(B, N, H, D))) == want
    prob = ta.make_problem(1, 64, 2, 64)
    ptrs = fake_ptrs(7)
    ptrs[0] = None  # validation reaches the pointer checks: the size itself is accepted
    assert call_fwd(lib, prob, ptrs) == INVALID


# ---- the Python binding's argument checks (host only: nothing reaches the library) ----

import torch  # noqa: E402


def test_check_tensor_rejects_each_mismatch():
    dev = torch.device("cpu")
    good = torch.zeros((1, 64, 4, 64), dtype=torch.float32)
    ta._check_tensor("lse", good, (1, 64, 4, 64), (torch.float32,), dev)
    with pytest.raises(ValueError, match="shape"):
        ta._check_tensor("lse", torch.zeros((1, 64, 4, 32)), (1, 64, 4, 64), (torch.float32,), dev)
    with pytest.raises(ValueError, match="dtype"):
        ta._check_tensor("lse", good.double(), (1, 64, 4, 64), (torch.float32,), dev)
    with pytest.raises(ValueError, match="contiguous"):
        ta._check_tensor("lse", torch.zeros((1, 64, 64, 4)).transpose(2, 3), (1, 64, 4, 64),
                         (torch.float32,), dev)
    with pytest.raises(ValueError, match="device"):
        ta._check_tensor("lse", good, (1, 64, 4, 64), (torch.float32,), torch.device("meta"))
    with pytest.raises(ValueError, match="tensor"):
        ta._check_tensor("lse", None, (1, 64, 4, 64), (torch.float32,), dev)


@pytest.fixture
def host_only_binding(monkeypatch):
    """The binding with its device checks of q, k, v, bias bypassed and no library:
    any call that got past the argument checks would raise RuntimeError."""
    def no_lib(*a, **k):
        raise RuntimeError("library reached")
    monkeypatch.setattr(ta, "load_library", no_lib)
    monkeypatch.setattr(ta, "_check_inputs", lambda q, k, v, bias, mask: tuple(
        q.shape[i] for i in (0, 1, 3, 4)))
    B, N, H, D = 1, 64, 2, 32
    t = {"q": torch.zeros((B, N, N, H, D), dtype=torch.bfloat16)}
    t.update(k=t["q"], v=t["q"], bias=torch.zeros((B, H, N, N), dtype=torch.bfloat16),
             o=torch.zeros_like(t["q"]), res=torch.zeros((B, N, N, H, D), dtype=torch.float32),
             lse=torch.zeros((B, N, H, N), dtype=torch.float32), do=torch.zeros_like(t["q"]))
    return t


@pytest.mark.parametrize("name,bad,match", [
    ("o", lambda t: t["o"].float(), "o must be of dtype"),
    ("o", lambda t: t["o"][:, :32], "o must have shape"),
    ("res", lambda t: t["res"].double(), "o_residual must be of dtype"),
    ("res", lambda t: t["res"][..., :16], "o_residual must have shape"),
    ("lse", lambda t: t["lse"][:, :32], "lse must have shape"),
    ("lse", lambda t: t["lse"].to(torch.bfloat16), "lse must be of dtype"),
    ("lse", lambda t: t["lse"].transpose(1, 3), "lse must"),
    ("do", lambda t: t["do"].float(), "d_o must be of dtype"),
    ("do", lambda t: t["do"][:, :, :32], "d_o must have shape"),
    ("do", lambda t: t["do"].transpose(1, 2), "d_o must be contiguous"),
])
def test_backward_rejects_mismatched_saved_tensors(host_only_binding, name, bad, match):
    t = dict(host_only_binding)
    t[name] = bad(t)
    with pytest.raises(ValueError, match=match):
        ta.tri_attn_bwd(t["q"], t["k"], t["v"], t["bias"], None, t["o"], t["res"], t["lse"], t["do"])


def test_backward_checks_pass_on_matching_tensors(host_only_binding):
    t = host_only_binding
    with pytest.raises(RuntimeError, match="library reached"):
        ta.tri_attn_bwd(t["q"], t["k"], t["v"], t["bias"], None, t["o"], t["res"], t["lse"], t["do"])
    with pytest.raises(RuntimeError, match="library reached"):   # uncompensated: no residual
        ta.tri_attn_bwd(t["q"], t["k"], t["v"], t["bias"], None, t["o"], None, t["lse"], t["do"])


def test_forward_rejects_mismatched_outputs(host_only_binding):
    t = host_only_binding
    with pytest.raises(ValueError, match="lse must have shape"):
        ta.tri_attn_fwd(t["q"], t["k"], t["v"], t["bias"], None, out=(t["o"], t["res"], t["lse"][:, :8]))
    with pytest.raises(ValueError, match="o_residual must be of dtype"):
        ta.tri_attn_fwd(t["q"], t["k"], t["v"], t["bias"], None, residual="bf16",
                        out=(t["o"], t["res"], t["lse"]))


# ---- attention-row ranges (one GPU's share of a row-sharded problem) ----

@pytest.mark.parametrize("rows,ok", [((0, 0), True), ((0, 64), True), ((10, 20), True), ((63, 64), True),
                                     ((-1, 5), False), ((5, 5), False), ((20, 10), False),
                                     ((0, 65), False), ((64, 64), False)])
def test_row_range_validation(lib, rows, ok):
    prob = ta.make_problem(1, 64, 4, 32, rows=rows)
    need = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(prob))
    assert (need > 0) == ok
    if not ok:
        assert call_fwd(lib, prob) == INVALID
        assert call_bwd(lib, prob, ws_bytes=1 << 40) == INVALID


def test_row_range_workspace_follows_the_range_plan(lib):
    """The dbias partials of a range call are one per row chunk of the range: a
    range of 32 rows (H = 4, N = 256: 16 groups of workgroups, at most 16 chunks)
    needs the same statistics and dQ partials as the whole problem but no more
    dbias partials than chunks of its own rows."""
    import bench
    full = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(1, 256, 4, 32)))
    part = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(1, 256, 4, 32, rows=(100, 132))))

    def a256(x):
        return (x + 255) // 256 * 256
    base = a256(256 * 4 * 2 * 256 * 4) + a256(4 * 256 * 256 * 4 * 32 * 2)
    assert full == base + a256(bench.row_chunks(16, 256) * 4 * 256 * 256 * 4)
    assert part == base + a256(bench.row_chunks(16, 32) * 4 * 256 * 256 * 4)


# ---- the triangle multiplicative update's contraction (include/tri_mul.h) ----

def call_mul_fwd(lib, prob, ptrs=None):
    a, b, z = ptrs or fake_ptrs(3)
    return lib.tri_mul_fwd(ctypes.byref(prob) if prob is not None else None, a, b, z, None)


def call_mul_bwd(lib, prob, ptrs=None):
    a, b, g, da, db = ptrs or fake_ptrs(5)
    return lib.tri_mul_bwd(ctypes.byref(prob), a, b, g, da, db, None)


def test_tri_mul_abi_version(lib):
    assert lib.tri_mul_abi_version() == ta.TRI_MUL_ABI_VERSION


@pytest.mark.parametrize("field,value,expect", [
    ("abi_version", ta.TRI_MUL_ABI_VERSION + 1, ABI), ("B", 0, INVALID), ("N", 0, INVALID), ("C", 0, INVALID),
    ("N", 48, UNSUPPORTED), ("N", 1056, UNSUPPORTED), ("flags", 2, UNSUPPORTED), ("C", 70000, UNSUPPORTED),
])
def test_tri_mul_problem_validation(lib, field, value, expect):
    prob = ta.make_trimul_problem(1, 64, 8)
    setattr(prob, field, value)
    assert call_mul_fwd(lib, prob) == expect
    assert call_mul_bwd(lib, prob) == expect


def test_tri_mul_rejects_null_misaligned_and_aliased_pointers(lib):
    prob = ta.make_trimul_problem(1, 64, 8)
    assert call_mul_fwd(lib, None) == INVALID
    for which in range(3):
        p = fake_ptrs(3)
        p[which] = None
        assert call_mul_fwd(lib, prob, p) == INVALID
        p = fake_ptrs(3)
        p[which] = ctypes.c_void_p(p[which].value + 2)
        assert call_mul_fwd(lib, prob, p) == INVALID
    p = fake_ptrs(3)
    p[2] = ctypes.c_void_p(p[0].value + 64)   # z inside a
    assert call_mul_fwd(lib, prob, p) == INVALID
    for which in range(5):
        p = fake_ptrs(5)
        p[which] = None
        assert call_mul_bwd(lib, prob, p) == INVALID
    p = fake_ptrs(5)
    p[4] = p[3]   # db == da
    assert call_mul_bwd(lib, prob, p) == INVALID
    p = fake_ptrs(5)
    p[3] = p[2]   # da == dz
    assert call_mul_bwd(lib, prob, p) == INVALID


# ---- the modules around the cores (include/tri_module.h, include/tri_mul_module.h) ----

def module_structs(n_params, n_saved, start=1):
    """Distinct fake device addresses, 4 GiB apart, for the pointer structs."""
    addr = [ADDR + (start + i) * (1 << 32) for i in range(n_params + n_saved)]
    return addr[:n_params], addr[n_params:]


def call_attn_module_fwd(lib, prob, z=ADDR, y=ADDR + 7 * (1 << 36), params=None, saved=None):
    pp, sv = module_structs(5, 10)
    p = ta.ModuleParams(*(params or pp))
    s = ta.ModuleSaved(*(saved or sv))
    return lib.tri_attn_module_fwd(ctypes.byref(prob) if prob is not None else None, ctypes.c_void_p(z), None,
                                   ctypes.byref(p), ctypes.c_void_p(y), ctypes.byref(s), None)


@pytest.mark.parametrize("field,value,expect", [("abi_version", ta.MODULE_ABI_VERSION + 1, ABI), ("B", 0, INVALID),
                                                ("H", 3, UNSUPPORTED), ("D", 64, UNSUPPORTED), ("N", 48, UNSUPPORTED),
                                                ("flags", 4, UNSUPPORTED), ("ln_eps", -1.0, INVALID)])
def test_attn_module_problem_validation(lib, field, value, expect):
    prob = ta.make_module_problem(1, 64, 4, 32)
    setattr(prob, field, value)
    assert call_attn_module_fwd(lib, prob) == expect
    assert lib.tri_attn_module_bwd_workspace_bytes(ctypes.byref(prob)) == 0


def test_attn_module_rejects_null_misaligned_and_aliased_pointers(lib):
    prob = ta.make_module_problem(1, 64, 4, 32)
    assert call_attn_module_fwd(lib, None) == INVALID
    pp, sv = module_structs(5, 10)
    bad = list(pp)
    bad[2] += 2  # a misaligned weight matrix
    assert call_attn_module_fwd(lib, prob, params=bad) == INVALID
    bad = list(sv)
    bad[3] = None  # no k
    assert call_attn_module_fwd(lib, prob, saved=bad) == INVALID
    assert call_attn_module_fwd(lib, prob, y=ADDR) == INVALID  # y over z
    bad = list(sv)
    bad[7] = sv[6]  # o over g
    assert call_attn_module_fwd(lib, prob, saved=bad) == INVALID


def test_attn_module_workspace_holds_the_core_workspace(lib):
    for N in (64, 256):
        core = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(1, N, 4, 32)))
        mod = lib.tri_attn_module_bwd_workspace_bytes(ctypes.byref(ta.make_module_problem(1, N, 4, 32)))
        assert mod > core + 5 * N * N * 128 * 2   # + dO, the gate gradient, dq, dk, dv


def call_trimul_module_fwd(lib, prob, z=ADDR, y=ADDR + 7 * (1 << 36), params=None, saved=None):
    pp, sv = module_structs(6, 8)
    p = ta.TriMulModuleParams(*(params or pp))
    s = ta.TriMulModuleSaved(*(saved or sv))
    return lib.tri_mul_module_fwd(ctypes.byref(prob) if prob is not None else None, ctypes.c_void_p(z), None,
                                  ctypes.byref(p), ctypes.c_void_p(y), ctypes.byref(s), None)


@pytest.mark.parametrize("field,value,expect", [("abi_version", ta.TRI_MUL_MODULE_ABI_VERSION + 1, ABI),
                                                ("B", 0, INVALID), ("C", 64, UNSUPPORTED), ("N", 48, UNSUPPORTED),
                                                ("N", 1056, UNSUPPORTED), ("flags", 2, UNSUPPORTED),
                                                ("ln_eps", float("inf"), INVALID)])
def test_trimul_module_problem_validation(lib, field, value, expect):
    prob = ta.make_trimul_module_problem(1, 64, 128)
    setattr(prob, field, value)
    assert call_trimul_module_fwd(lib, prob) == expect
    assert lib.tri_mul_module_bwd_workspace_bytes(ctypes.byref(prob)) == 0


def test_trimul_module_rejects_null_misaligned_and_aliased_pointers(lib):
    prob = ta.make_trimul_module_problem(1, 64, 128)
    assert call_trimul_module_fwd(lib, None) == INVALID
    pp, sv = module_structs(6, 8)
    bad = list(pp)
    bad[0] += 4
    assert call_trimul_module_fwd(lib, prob, params=bad) == INVALID
    assert call_trimul_module_fwd(lib, prob, y=sv[5]) == INVALID  # y over the saved x
    bad = list(sv)
    bad[3] = sv[2]  # b over a
    assert call_trimul_module_fwd(lib, prob, saved=bad) == INVALID
