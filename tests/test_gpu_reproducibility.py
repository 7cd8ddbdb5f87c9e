"""Run-to-run reproducibility of the HIP path (needs an MI355X).

The protocol of the TurboPairFormer reproducibility check (dev48.org page,
"reproducibility" section): 600 cases with fixed inputs, each run five times; a case
passes only if the gradients of q, k, v and the pair bias are bitwise identical
over the five runs.  Here the forward outputs (o, its residual, lse) are compared
too.  The cases are small (N <= 128) and drawn from a fixed seed over batch size,
N, head count, key-mask kind (none given as no mask at all, a ones mask, padded
keys, random keys), orientation, compensated or uncompensated D, softmax scale,
bf16 or fp32 dbias, bf16 or fp32 saved residual and head dimension 16 or 32.
Before every run the outputs and the backward workspace are filled with a byte
pattern (NaN in the first run, other patterns after), so that a value the kernels
read before writing it, or never write, would differ between the runs.
"""
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si

pytestmark = pytest.mark.gpu

N_CASES, N_RUNS = 600, 5


@pytest.fixture(scope="module")
def ta():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import triangle_attention_amd as mod
    mod.load_library()
    return mod


FILLS = (0xFF, 0x00, 0x7F, 0xA5, 0x5A)  # 0xff bytes: NaN in bf16 and fp32


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def filled(shape, dtype, dev, byte):
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def test_reproducibility_sweep(ta):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(600)
    names = ("o", "res", "lse", "dq", "dk", "dv", "dbias")
    failures = []
    for case in range(N_CASES):
        B = int(rng.choice([1, 2]))
        N = int(rng.choice([32, 64, 96, 128]))
        H = int(rng.integers(1, 5))
        kind = str(rng.choice(["absent", "none", "pad32", "random"]))
        ending = bool(rng.integers(0, 2))
        compensated = bool(rng.integers(0, 2))
        scale = None if rng.integers(0, 2) else float(rng.uniform(0.1, 0.4))
        dbias_fp32 = bool(rng.integers(0, 2))
        residual = "fp32" if rng.integers(0, 2) else "bf16"
        D = int(rng.choice([16, 32]))
        inp = si.make_problem(B, N, H, D, 20000 + case, mask="none" if kind == "absent" else kind)
        g = {k: v.to(dev) for k, v in inp.items()}
        mask = None if kind == "absent" else g["mask"]
        if case % 100 == 0:
            print(f"[reproducibility] case {case}: B={B} N={N} H={H} D={D} mask={kind} ending={ending} "
                  f"compensated={compensated} scale={scale} dbias_fp32={dbias_fp32} "
                  f"residual={residual}", flush=True)
            sys.stdout.flush()
        first = None
        shp = tuple(inp["q"].shape)
        ws_bytes = ta.bwd_workspace_bytes(B, N, H, D, ending=ending, dbias_fp32=dbias_fp32, scale=scale)
        for run in range(N_RUNS):
            # outputs and workspace start as NaN in the first run and as other byte
            # patterns in the later ones: a value read before it is written, or never
            # written, then differs between runs
            fill = FILLS[run]
            fo = (filled(shp, torch.bfloat16, dev, fill), filled(shp, ta.RESIDUAL_DTYPES[residual], dev, fill),
                  filled((B, N, H, N), torch.float32, dev, fill))
            o, res, lse = ta.tri_attn_fwd(g["q"], g["k"], g["v"], g["bias"], mask, ending=ending,
                                          scale=scale, residual=residual, out=fo)
            bo = tuple(filled(shp, torch.bfloat16, dev, fill) for _ in range(3)) + (
                filled((B, H, N, N), torch.float32 if dbias_fp32 else torch.bfloat16, dev, fill),)
            ws = filled((ws_bytes,), torch.uint8, dev, fill)
            grads = ta.tri_attn_bwd(g["q"], g["k"], g["v"], g["bias"], mask, o,
                                    res if compensated else None, lse, g["do"], ending=ending,
                                    scale=scale, dbias_fp32=dbias_fp32, workspace=ws, out=bo)
            out = dict(zip(names, (o, res, lse) + tuple(grads)))
            if first is None:
                first = out
                continue
            for n in names:
                if not torch.equal(bits(first[n]), bits(out[n])):
                    failures.append((case, n))
        torch.cuda.synchronize()
    print(f"[reproducibility] {N_CASES} cases x {N_RUNS} runs: {len(failures)} differing outputs", flush=True)
    assert not failures, failures[:20]
