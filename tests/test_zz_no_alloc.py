"""The allocation-free backward (tri_attn_bwd_noalloc) against tri_attn_bwd (needs an
MI355X).

tri_attn_bwd_noalloc runs the same kernels as tri_attn_bwd with the workspace in the
library's fixed device buffer; its outputs must equal tri_attn_bwd's bitwise.  Two
calls in a row, the second on a smaller problem, so that the second call finds the
first call's contents in the buffer.  Outputs are filled with NaN beforehand.
"""
import ctypes
import sys

import pytest
import torch

import seeded_inputs as si

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def nan_like(t):
    x = torch.empty_like(t)
    x.view(torch.uint8).fill_(0xFF)
    return x


@pytest.fixture(scope="module")
def ta():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import triangle_attention_amd as mod
    mod.load_library()
    return mod


def one_case(ta, B, N, H, D, mask_kind, ending, seed):
    print(f"[no-alloc] B={B} N={N} H={H} D={D} mask={mask_kind} ending={ending}", flush=True)
    sys.stdout.flush()
    dev = torch.device("cuda:0")
    inp = si.make_problem(B, N, H, D, seed, mask=mask_kind)
    g = {k: v.to(dev) for k, v in inp.items()}
    mask = g["mask"] if mask_kind != "none" else None
    o, res, lse = ta.tri_attn_fwd(g["q"], g["k"], g["v"], g["bias"], mask, ending=ending)
    ref = ta.tri_attn_bwd(g["q"], g["k"], g["v"], g["bias"], mask, o, res, lse, g["do"], ending=ending)
    out = tuple(nan_like(t) for t in ref)
    got = ta.tri_attn_bwd_noalloc(g["q"], g["k"], g["v"], g["bias"], mask, o, res, lse, g["do"], out,
                                  ending=ending)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dbias"), ref, got):
        assert torch.equal(bits(a), bits(b)), name


def test_noalloc_matches_the_workspace_backward_twice(ta):
    one_case(ta, 1, 256, 4, 32, "pad32", False, 501)      # the largest workload that fits
    one_case(ta, 2, 96, 3, 32, "random", True, 502)       # then a smaller one


def test_noalloc_rejects_a_problem_beyond_the_buffer(ta):
    dev = torch.device("cuda:0")
    B, N, H, D = 1, 768, 4, 32
    lib = ta.load_library()
    need = lib.tri_attn_bwd_workspace_bytes(ctypes.byref(ta.make_problem(B, N, H, D)))
    assert need > ta.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, N, N, H, D), dtype=torch.bfloat16, device=dev)
    bias = torch.zeros((B, H, N, N), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((B, N, H, N), dtype=torch.float32, device=dev)
    out = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), torch.empty_like(bias))
    with pytest.raises(ta.TriAttnError) as e:
        ta.tri_attn_bwd_noalloc(q, q, q, bias, None, q, None, lse, q, out)
    assert e.value.status == 3
