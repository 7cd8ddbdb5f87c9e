#!/usr/bin/env python3
"""Triangle-attention forward+backward throughput on one MI355X.

Workload: the crop-768 Pairformer configuration (B=1, N=768, H=4, D=32, bf16
q, k, v, dO and bias drawn N(0,1) from a fixed seed, all keys attended,
starting node).  One step = tri_attn_fwd followed by tri_attn_bwd (every
kernel of the path) on inputs already resident in HBM.  The metric is
algorithmic TFLOP/s: 14 * D flop per valid score element (two forward and five
backward products; exp and the bias-gradient additions are not counted).

The JSON line also carries
  roofline     : the backward main kernel (the dominant one), timed with HIP
                 events recorded by the library on the launch stream, against
                 the MI355X dense bf16 MFMA peak; its "traffic" is the HBM bytes
                 per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary in
                 profiles/ (calibrated against a plain device copy), or null when
                 that summary was taken on a different kernel source or build flags;
  cpu_baseline : the FP64 oracle run on the whole crop768 problem on this host's
                 cores (one timed forward and backward, ~40 s on 16 threads), with
                 the thread count and CPU model;
  mfma_probe   : the sustained bf16 matrix-core rate this device reaches with
                 independent back-to-back 32x32x16 products, and the backward main
                 kernel's and the whole step's fractions of it;
  phases       : median and 90th-percentile forward, backward and step times over
                 the timed steps (events on the launch stream), the same for each
                 of the backward's four kernels (events the library records
                 between them), the algorithmic bytes of one step and the rate they
                 imply, the pair-bias and bias-gradient bytes of a step with the
                 measured rate of the dbias reduction, and whether the outputs of
                 the first and last timed steps are bitwise identical;
  workloads    : the other reported crop sizes (384 and 640, 768 in the ending
                 node orientation, and 768 at head dimensions 16 and 64 with the same
                 128 pair channels), each timed over fewer steps: median time per
                 step, forward and backward, TFLOP/s and fraction of the MFMA peak;
  module       : the triangle-attention module around the core (LayerNorm, the q, k, v,
                 bias and gate projections, the core, the gated output projection, and
                 the backward to dz and the parameter gradients) at crop 768: median
                 forward and backward times;
  tri_mul      : the triangle multiplicative update's contraction at the crop-768
                 shape with 128 channels (tri_mul_fwd + tri_mul_bwd, outgoing and
                 incoming edges): median times, TFLOP/s and fraction of the peak; and
                 the whole block around it (LayerNorms, gated projections, output
                 gate) at the same shape;
  accuracy     : the crop768 outputs of the last timed step against the FP64 oracle
                 run on the whole problem (forward max-abs and rel-RMSE, lse max-abs,
                 and the rel-RMSE of each gradient with the residual-compensated
                 correction next to the uncompensated one, the latter from one more
                 backward without the residual), and the same gradient comparison at
                 crop640 (peaked rows) on sampled rows.
The whole-problem oracle run is the cpu_baseline's timed work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time
from pathlib import Path

import torch

MFMA_PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBS = 8000.0


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch has already loaded (the
    library records them on the launch stream; torch's own Event objects are
    created lazily and cannot be handed to it before their first record)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e: int) -> None:
        self.hip.hipEventDestroy(e)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


ROOT = Path(__file__).resolve().parent
KERNEL_SOURCE = ROOT / "triangle_attention_amd" / "csrc" / "tri_attn.hip"


def build_hash() -> str:
    """sha256 of the kernel source and the compiler flags it is built with."""
    from triangle_attention_amd.build import FLAGS
    return hashlib.sha256(KERNEL_SOURCE.read_bytes() + " ".join(FLAGS).encode()).hexdigest()


def measured_traffic(workload: str, ending: bool, residual: str = "fp32"):
    """HBM bytes per launch of the backward main kernel from the committed rocprofv3
    counter summary, if it was taken on this kernel source, these build flags and
    this workload."""
    if ending or residual != "fp32":
        return None
    f = ROOT / "profiles" / f"traffic_bwd_main_{workload}.md"
    if not f.exists():
        return None
    text = f.read_text()
    sha = re.search(r"build_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not sha or not val:
        return None
    if sha.group(1) != build_hash():
        return None
    return int(val.group(1))


def algorithmic_bytes(B: int, N: int, H: int, D: int, masked: bool, residual_bytes: int = 4) -> int:
    """Bytes one fwd+bwd step must move: the forward reads q, k, v, bias (and the
    mask) and writes o, its residual and lse; the backward reads q, k, v, o, the
    residual, dO, lse, bias (and the mask) and writes dq, dk, dv and dbias."""
    E = B * N * N * H * D
    return (24 + 2 * residual_bytes) * E + 14 * B * H * N * N + (2 * B * N * N if masked else 0)


def row_chunks(groups: int, N: int, cus: int = 256) -> int:
    """Row chunks per (batch, head, block) in the library's launch plan (one workgroup
    per CU at a time): one round of workgroups over the MI355X's 256 compute units, or,
    where one round would leave more than 15 % of them idle, the chunk count that
    minimises rows per CU plus two rows per round (at least one chunk, at most N)."""
    one = max(1, min(N, cus // groups))
    c = one
    if groups * one * 100 < cus * 85 and groups < cus:
        best_cost = None
        for C in range(one, min(N, 16 * one) + 1):
            rounds = -(-groups * C // cus)
            cost = rounds * -(-N // C) + 2 * rounds
            if best_cost is None or cost < best_cost:
                best_cost, c = cost, C
    per = -(-N // c)
    return -(-N // per)


def block_size(D: int) -> int:
    """Queries per forward workgroup and keys per backward workgroup in the library's
    launch plan: 64, or 32 at head dimension 64."""
    return 32 if D == 64 else 64


def bias_dbias_bytes(B: int, N: int, H: int, dbias_bytes: int = 2, D: int = 32) -> dict:
    """Pair-bias and bias-gradient HBM bytes of one step.  Every forward workgroup
    (b, h, query block, row chunk) and every backward workgroup (b, h, key block, row
    chunk) stages its bias block once; the backward main kernel writes one fp32
    dbias partial per row chunk, which the dbias reduction reads back before writing
    dbias."""
    nb = B * H * N * N
    blocks = -(-N // block_size(D))
    c_fwd = row_chunks(B * H * blocks, N)
    c_bwd = row_chunks(B * H * blocks, N)
    return {"bias_tensor_bytes": 2 * nb,
            "bias_staged_bytes": (c_fwd + c_bwd) * 2 * nb,
            "dbias_partial_bytes": c_bwd * 4 * nb,
            "dbias_reduction_bytes": c_bwd * 4 * nb + dbias_bytes * nb}


def mfma_probe_tflops(blocks: int = 1024, iters: int = 20000) -> float:
    """Sustained bf16 matrix-core rate of this device: `blocks` workgroups of four
    waves (four per SIMD at 1024) issuing independent 32x32x16 products back to
    back (libmfma_probe.so, built with the library), timed with events on the
    current stream."""
    import ctypes
    from triangle_attention_amd.build import PROBE_LIB
    if not PROBE_LIB.exists():
        raise RuntimeError(f"{PROBE_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(str(PROBE_LIB))
    lib.mfma_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.mfma_probe_launch.restype = ctypes.c_int
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(n):
        if lib.mfma_probe_launch(ctypes.c_void_p(out.data_ptr()), blocks, n, stream) != 0:
            raise RuntimeError("mfma probe launch failed")

    launch(iters // 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launch(iters)
    e1.record()
    torch.cuda.synchronize()
    flops = blocks * 4 * iters * 4 * 32768
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12


def quantiles(xs):
    xs = sorted(xs)
    pick = lambda q: xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]
    return {"median": round(pick(0.5), 4), "p90": round(pick(0.9), 4)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def rel_rmse(x, ref) -> float:
    import numpy as np
    den = float(np.linalg.norm(ref))
    return float(np.linalg.norm(np.asarray(x, np.float64) - ref) / (den if den > 0 else 1.0))


def to_np(t):
    return t.detach().float().cpu().double().numpy()


def oracle_whole(inp):
    """The FP64 oracle on the whole problem (forward, then every row's gradients, then
    every pair-bias-gradient row), timed on this host: (reference dict, cpu_baseline)."""
    import oracle
    import seeded_inputs as si

    B, N, _, H, D = inp["q"].shape
    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    t0 = time.perf_counter()
    ref = oracle.forward_backward(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"])
    t = time.perf_counter() - t0
    flops = si.flop_count(B, N, H, D, inp["mask"])
    base = {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": int(os.environ.get("OMP_NUM_THREADS", threads)),
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": (f"the whole workload: all {B * N} attention rows (forward, lse and q/k/v gradients) "
                   f"and all {B * H * N} pair-bias-gradient rows, {t:.1f} s"),
    }
    return ref, base


def accuracy_whole(out, unc, ref) -> dict:
    """Forward errors and per-gradient rel-RMSE (compensated / uncompensated) of one
    step's outputs against the whole-problem oracle."""
    import numpy as np
    o = to_np(out["o"])
    lse = to_np(out["lse"])
    fin = np.isfinite(ref["lse"])
    acc = {"reference": "FP64 oracle, whole problem",
           "o_max_abs": float(np.max(np.abs(o - ref["o"]))),
           "o_rel_rmse": rel_rmse(o, ref["o"]),
           "lse_max_abs": float(np.max(np.abs(lse[fin] - ref["lse"][fin]))) if fin.any() else 0.0,
           "grad_rel_rmse": {}}
    del o, lse
    for n in ("dq", "dk", "dv", "dbias"):
        acc["grad_rel_rmse"][n] = {"compensated": rel_rmse(to_np(out[n]), ref[n]),
                                   "uncompensated": rel_rmse(to_np(unc[n]), ref[n])}
    acc["bounds"] = {"o_max_abs": 2e-2, "o_rel_rmse": 1e-2, "grad_rel_rmse": 2e-2}
    return acc


def accuracy_sampled(out, unc, inp, rows: int, dbias_rows: int) -> dict:
    """Per-gradient rel-RMSE, compensated and uncompensated, on `rows` sampled attention
    rows and `dbias_rows` sampled pair-bias-gradient rows."""
    import numpy as np
    import oracle
    B, N, _, H, D = inp["q"].shape
    rng = np.random.default_rng(1)
    sel_rows = sorted((0, int(r)) for r in rng.choice(N, size=min(rows, N), replace=False))
    sel_db = sorted({(0, int(h), int(j)) for h, j in zip(rng.integers(0, H, dbias_rows),
                                                         rng.integers(0, N, dbias_rows))})
    p = oracle.Problem(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"])
    ref = p.rows(sel_rows)
    ref["dbias"] = p.dbias(sel_db)

    def pick(x, n):
        if n == "dbias":
            return np.stack([to_np(x[b, h, j]) for (b, h, j) in sel_db])
        return np.stack([to_np(x[b, r]) for (b, r) in sel_rows])
    acc = {"reference": f"FP64 oracle, {len(sel_rows)} sampled attention rows and {len(sel_db)} "
                        "sampled pair-bias-gradient rows",
           "o_rel_rmse": rel_rmse(pick(out["o"], "o"), ref["o"]), "grad_rel_rmse": {}}
    for n in ("dq", "dk", "dv", "dbias"):
        acc["grad_rel_rmse"][n] = {"compensated": rel_rmse(pick(out[n], n), ref[n]),
                                   "uncompensated": rel_rmse(pick(unc[n], n), ref[n])}
    return acc


def time_workload(args, workload: str, ending: bool, steps: int, warmup: int, keep_outputs: bool = False):
    """Time `steps` fwd+bwd steps of one workload after `warmup` untimed ones."""
    import seeded_inputs as si
    import triangle_attention_amd as ta

    w = si.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    log(f"workload {w.name}{' (ending node)' if ending else ''}: {w.description}")
    inp = si.make_workload(w.name)
    g = {k: v.to(dev) for k, v in inp.items()}
    mask = g["mask"] if w.mask != "none" else None
    ta.load_library()
    ws = torch.empty(ta.bwd_workspace_bytes(w.B, w.N, w.H, w.D, ending=ending),
                     dtype=torch.uint8, device=dev)

    def fwd():
        return ta.tri_attn_fwd(g["q"], g["k"], g["v"], g["bias"], mask, ending=ending,
                               residual=args.residual)

    def bwd(o, res, lse, events=None):
        return ta.tri_attn_bwd(g["q"], g["k"], g["v"], g["bias"], mask, o, res, lse, g["do"],
                               ending=ending, workspace=ws, kernel_events=events)

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"warmup {warmup}")
    for _ in range(warmup):
        bwd(*fwd())
    torch.cuda.synchronize()

    hip = HipEvents()
    # five events per step around the backward's four kernels (statistics, main, dQ
    # reduction, dbias reduction), recorded by the library on the launch stream
    ev = [[hip.create() for _ in range(5)] for _ in range(steps)]
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    log(f"timing {steps} steps")
    outs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        marks[i][0].record()
        fo = fwd()
        marks[i][1].record()
        grads = bwd(*fo, events=ev[i])
        marks[i][2].record()
        if i == 0 or i == steps - 1:
            outs.append(fo + tuple(grads))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    kern = {name: [hip.elapsed_ms(e[i], e[i + 1]) for e in ev]
            for i, name in enumerate(("bwd_prep", "bwd_main", "reduce_dq", "reduce_dbias"))}
    for e in ev:
        for x in e:
            hip.destroy(x)
    res = {
        "w": w, "inp": inp, "ms": ms,
        "fwd_ms": [m[0].elapsed_time(m[1]) for m in marks],
        "bwd_ms": [m[1].elapsed_time(m[2]) for m in marks],
        "step_ms": [m[0].elapsed_time(m[2]) for m in marks],
        "kern": kern,
        "same": all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                                y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
                    for x, y in zip(outs[0], outs[-1])),
        "flops": si.flop_count(w.B, w.N, w.H, w.D, inp["mask"]),
    }
    if keep_outputs:
        o, r, lse, dq, dk, dv, db = outs[-1]
        res["out"] = {"o": o, "res": r, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dbias": db}
        # one more backward without the residual: the uncompensated correction
        udq, udk, udv, udb = bwd(o, None, lse)
        torch.cuda.synchronize()
        res["unc"] = {"dq": udq, "dk": udk, "dv": udv, "dbias": udb}
    del g, ws, outs
    log(f"{ms:.3f} ms/step, backward main kernel {statistics.mean(kern['bwd_main']):.3f} ms")
    return res


def time_trimul(args, workload: str, incoming: bool, steps: int, warmup: int) -> dict:
    """Time `steps` forward + backward calls of the triangle-multiplication contraction
    (tri_mul_fwd, then tri_mul_bwd: three N^3 products per channel) after `warmup`."""
    import seeded_inputs as si
    import triangle_attention_amd as ta

    w = si.TRIMUL_WORKLOADS[workload]
    dev = torch.device("cuda:0")
    log(f"workload {w.name} ({'incoming' if incoming else 'outgoing'} edges): {w.description}")
    inp = si.make_trimul_workload(w.name)
    a, b, g = (inp[n].to(dev) for n in ("a", "b", "g"))
    z, da, db = torch.empty_like(a), torch.empty_like(a), torch.empty_like(a)
    for _ in range(warmup):
        ta.tri_mul_fwd(a, b, incoming=incoming, out=z)
        ta.tri_mul_bwd(a, b, g, incoming=incoming, out=(da, db))
    torch.cuda.synchronize()
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    first = None
    for i in range(steps):
        marks[i][0].record()
        ta.tri_mul_fwd(a, b, incoming=incoming, out=z)
        marks[i][1].record()
        ta.tri_mul_bwd(a, b, g, incoming=incoming, out=(da, db))
        marks[i][2].record()
        if i == 0:
            torch.cuda.synchronize()
            first = [x.clone() for x in (z, da, db)]
    torch.cuda.synchronize()
    fwd = statistics.median(m[0].elapsed_time(m[1]) for m in marks)
    bwd = statistics.median(m[1].elapsed_time(m[2]) for m in marks)
    flops = si.trimul_flop_count(w.B, w.N, w.C)
    v = flops / ((fwd + bwd) * 1e-3) / 1e12
    return {"ms_per_step": round(fwd + bwd, 4), "fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4),
            "TFLOPs": round(v, 2), "mfma_peak_frac": round(v / MFMA_PEAK_BF16_TFLOPS, 4),
            "flops_per_step": flops, "steps": steps,
            "deterministic_first_vs_last_step": all(
                torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(first, (z, da, db)))}


def module_bytes(B: int, N: int, H: int) -> dict:
    """Algorithmic HBM bytes of one module step outside the core: each bf16 position
    tensor ([B, N, N, 128], E bytes) read or written once per kernel that needs it.
    Forward: projections read z and write zn, q, k, v, g (+ statistics and the bias);
    the gated output reads g, o and writes y.  Backward: dy, g, o in and dO, dg out;
    dq, dk, dv, dg, z in and dz out (+ dbias, statistics); the weight gradients read
    zn, dq, dk, dv, dg, g, o, dy (+ dbias)."""
    P = B * N * N
    E = P * 128 * 2
    nb = B * H * N * N
    fwd = 6 * E + 8 * P + 2 * nb + 3 * E
    bwd = 5 * E + 6 * E + 4 * nb + 8 * P + 8 * E + 4 * nb
    return {"forward": fwd, "backward": bwd, "total": fwd + bwd}


def time_module(args, workload: str, steps: int, warmup: int) -> dict:
    """Time `steps` forward + backward calls of the triangle-attention module (the core
    included) after `warmup`; events on the launch stream."""
    import seeded_inputs as si
    import triangle_attention_amd as ta

    w = si.MODULE_WORKLOADS[workload]
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: {w.description}")
    inp = {n: t.to(dev) for n, t in si.make_module_workload(w.name).items()}
    mask = inp["mask"] if w.mask != "none" else None
    params = {n: inp[n] for n in ("ln_w", "ln_b", "w_qkvg", "w_bias", "w_out")}
    ws = torch.empty(ta.module_bwd_workspace_bytes(w.B, w.N, w.H, w.D), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        y, saved = ta.tri_attn_module_fwd(inp["z"], mask, params, w.H)
        ta.tri_attn_module_bwd(inp["z"], mask, params, saved, inp["dy"], w.H, workspace=ws)
    torch.cuda.synchronize()
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    outs = []
    for i in range(steps):
        marks[i][0].record()
        y, saved = ta.tri_attn_module_fwd(inp["z"], mask, params, w.H)
        marks[i][1].record()
        dz, grads = ta.tri_attn_module_bwd(inp["z"], mask, params, saved, inp["dy"], w.H, workspace=ws)
        marks[i][2].record()
        if i == 0 or i == steps - 1:
            outs.append([y, dz] + [grads[n] for n in sorted(grads)])
    torch.cuda.synchronize()
    fwd = statistics.median(m[0].elapsed_time(m[1]) for m in marks)
    bwd = statistics.median(m[1].elapsed_time(m[2]) for m in marks)
    flops = si.flop_count(w.B, w.N, w.H, w.D, inp["mask"].cpu() if mask is not None else None)
    nb = module_bytes(w.B, w.N, w.H)
    same = all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
               for x, y in zip(outs[0], outs[-1]))
    return {"ms_per_step": round(fwd + bwd, 4), "fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4),
            "core_TFLOPs_equivalent": round(flops / ((fwd + bwd) * 1e-3) / 1e12, 2),
            "module_bytes_outside_core": nb["total"], "steps": steps,
            "deterministic_first_vs_last_step": same}


def time_trimul_module(args, workload: str, incoming: bool, steps: int, warmup: int) -> dict:
    """Time `steps` forward + backward calls of the triangle multiplicative update block
    (LayerNorms, gated projections, the contraction) after `warmup`."""
    import seeded_inputs as si
    import triangle_attention_amd as ta

    w = si.TRIMUL_MODULE_WORKLOADS[workload]
    dev = torch.device("cuda:0")
    log(f"workload {w.name} ({'incoming' if incoming else 'outgoing'} edges): {w.description}")
    inp = {n: t.to(dev) for n, t in si.make_trimul_module_workload(w.name).items()}
    mask = inp["mask"] if w.mask != "none" else None
    params = {n: inp[n] for n in ("ln_in_w", "ln_in_b", "w_in", "ln_out_w", "ln_out_b", "w_out")}
    ws = torch.empty(ta.trimul_module_bwd_workspace_bytes(w.B, w.N, w.C, incoming=incoming), dtype=torch.uint8,
                     device=dev)
    for _ in range(warmup):
        y, saved = ta.tri_mul_module_fwd(inp["z"], mask, params, incoming=incoming)
        ta.tri_mul_module_bwd(inp["z"], mask, params, saved, inp["dy"], incoming=incoming, workspace=ws)
    torch.cuda.synchronize()
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    outs = []
    for i in range(steps):
        marks[i][0].record()
        y, saved = ta.tri_mul_module_fwd(inp["z"], mask, params, incoming=incoming)
        marks[i][1].record()
        dz, grads = ta.tri_mul_module_bwd(inp["z"], mask, params, saved, inp["dy"], incoming=incoming, workspace=ws)
        marks[i][2].record()
        if i == 0 or i == steps - 1:
            outs.append([y, dz] + [grads[n] for n in sorted(grads)])
    torch.cuda.synchronize()
    fwd = statistics.median(m[0].elapsed_time(m[1]) for m in marks)
    bwd = statistics.median(m[1].elapsed_time(m[2]) for m in marks)
    same = all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
               for x, y in zip(outs[0], outs[-1]))
    flops = si.trimul_flop_count(w.B, w.N, w.C)
    return {"ms_per_step": round(fwd + bwd, 4), "fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4),
            "contraction_TFLOPs_equivalent": round(flops / ((fwd + bwd) * 1e-3) / 1e12, 2), "steps": steps,
            "deterministic_first_vs_last_step": same}


def run_workload(args, workload: str, ending: bool, with_extras: bool) -> dict:
    """Time fwd+bwd steps of one workload and return its JSON line as a dict."""
    t = time_workload(args, workload, ending, args.steps, args.warmup, keep_outputs=with_extras)
    w, kern, flops = t["w"], t["kern"], t["flops"]
    ms = t["ms"]
    main_ms = statistics.mean(kern["bwd_main"])
    nbytes = algorithmic_bytes(w.B, w.N, w.H, w.D, w.mask != "none", 4 if args.residual == "fp32" else 2)
    value = flops / (ms * 1e-3) / 1e12
    bwd_main_flops = flops * 10 / 14   # S, dP, dV, dK, dQ products of the backward
    achieved = bwd_main_flops / (main_ms * 1e-3) / 1e12
    bd = bias_dbias_bytes(w.B, w.N, w.H, D=w.D)
    red_ms = statistics.median(kern["reduce_dbias"])
    bd["reduce_dbias_ms"] = round(red_ms, 4)
    bd["reduce_dbias_GBps"] = round(bd["dbias_reduction_bytes"] / (red_ms * 1e-3) / 1e9, 1)
    bd["bias_and_dbias_bytes_per_step"] = bd["bias_staged_bytes"] + 2 * bd["dbias_partial_bytes"] + 2 * w.B * w.H * w.N * w.N
    line = {
        "metric": "triangle-attn fwd+bwd TFLOP/s at N=768 bf16; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} ({w.description})", "B": w.B, "N": w.N, "H": w.H,
                   "D": w.D, "orientation": "ending" if ending else "starting",
                   "residual": args.residual,
                   "mfma_peak_frac": round(value / MFMA_PEAK_BF16_TFLOPS, 4)},
        "roofline": {"kernel": "bwd_main_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name, ending, args.residual),
                     "avg_ms": round(main_ms, 4)},
        "phases": {"fwd_ms": quantiles(t["fwd_ms"]), "bwd_ms": quantiles(t["bwd_ms"]),
                   "step_ms": quantiles(t["step_ms"]),
                   "bwd_kernels_ms": {n: quantiles(v) for n, v in kern.items()},
                   "bias_dbias": bd,
                   "algorithmic_bytes_per_step": nbytes,
                   "algorithmic_GBps": round(nbytes / (statistics.median(t["step_ms"]) * 1e-3) / 1e9, 1),
                   "deterministic_first_vs_last_step": bool(t["same"])},
    }
    if not with_extras:
        return line
    out, unc, inp = t.pop("out"), t.pop("unc"), t["inp"]
    del t
    # the other reported workloads: crop 384 and 640, 768 in the ending orientation, and
    # 768 at head dimensions 16 and 64 (the same 128 pair channels)
    others = {}
    for wl, end in (("crop384", False), ("crop640", False), ("crop768", True), ("crop768_h8d16", False),
                    ("crop768_h2d64", False)):
        o = time_workload(args, wl, end, args.other_steps, min(args.warmup, 3),
                          keep_outputs=(wl == "crop640"))
        v = o["flops"] / (statistics.median(o["step_ms"]) * 1e-3) / 1e12
        key = f"{wl}_ending" if end else wl
        others[key] = {"ms_per_step": round(statistics.median(o["step_ms"]), 4),
                       "fwd_ms": round(statistics.median(o["fwd_ms"]), 4),
                       "bwd_ms": round(statistics.median(o["bwd_ms"]), 4),
                       "bwd_main_ms": round(statistics.median(o["kern"]["bwd_main"]), 4),
                       "TFLOPs": round(v, 2), "mfma_peak_frac": round(v / MFMA_PEAK_BF16_TFLOPS, 4),
                       "steps": args.other_steps,
                       "deterministic_first_vs_last_step": bool(o["same"])}
        if wl == "crop640":
            log("accuracy at crop640 (sampled oracle rows)")
            acc640 = accuracy_sampled(o["out"], o["unc"], o["inp"], args.acc_rows, args.acc_dbias_rows)
        del o
        torch.cuda.empty_cache()
    line["workloads"] = others
    # the triangle multiplicative update's contraction at the crop-768 shape, C = 128
    line["tri_mul"] = {f"trimul_crop768_{d}": time_trimul(args, "trimul_crop768", d == "incoming",
                                                          args.other_steps, 3)
                       for d in ("outgoing", "incoming")}
    # the module around the core (LayerNorm, projections, gating) at the crop-768 shape
    line["module"] = {"module_crop768": time_module(args, "module_crop768", args.other_steps, 3)}
    torch.cuda.empty_cache()
    line["tri_mul"]["trimul_block_crop768_outgoing"] = time_trimul_module(args, "trimul_block_crop768", False,
                                                                          args.other_steps, 3)
    torch.cuda.empty_cache()
    log("matrix-core probe")
    probe = mfma_probe_tflops()
    line["mfma_probe"] = {"TFLOPs": round(probe, 1),
                          "what": "sustained v_mfma_f32_32x32x16_bf16 rate of this device "
                                  "(four waves per SIMD, independent accumulators)",
                          "bwd_main_frac": round(achieved / probe, 4),
                          "step_frac": round(value / probe, 4)}
    if not args.no_cpu_baseline:
        log("cpu baseline: the FP64 oracle on the whole workload")
        ref, base = oracle_whole(inp)
        line["cpu_baseline"] = base
        log("accuracy against the oracle")
        line["accuracy"] = accuracy_whole(out, unc, ref)
        line["accuracy"]["crop640_sampled"] = acc640
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="crop768")
    ap.add_argument("--ending", action="store_true", help="ending-node orientation")
    ap.add_argument("--residual", choices=("fp32", "bf16"), default="fp32",
                    help="precision of the saved rounding residual of o")
    ap.add_argument("--other-steps", type=int, default=20,
                    help="timed steps of each of the other reported workloads")
    ap.add_argument("--acc-rows", type=int, default=64,
                    help="sampled attention rows of the crop640 accuracy comparison")
    ap.add_argument("--acc-dbias-rows", type=int, default=256,
                    help="sampled pair-bias-gradient rows of the crop640 accuracy comparison")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the whole-problem oracle run (and with it the crop768 accuracy block)")
    ap.add_argument("--quick", action="store_true",
                    help="only the timed workload: no other workloads, probe, oracle or accuracy")
    ap.add_argument("--all", action="store_true",
                    help="one JSON line per workload: crop384, crop640, crop768 starting and ending node")
    ap.add_argument("--calib-copy", action="store_true",
                    help="copy a 256 MiB device buffer once before the warmup (a known-size kernel "
                         "that calibrates the rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU runs are not "
                                   "supported (use --gpus 1)", "n_gpus": args.gpus}))
        sys.exit(2)

    if args.all:
        # one line per workload the reporting plan names: crops 384, 640 and 768, the
        # last in both orientations; the oracle baseline with the crop768 line only
        for wl, ending in (("crop384", False), ("crop640", False), ("crop768", False), ("crop768", True)):
            line = run_workload(args, wl, ending, False)
            print(json.dumps(line), flush=True)
        return
    if args.workload.startswith("module_"):
        # the whole module (LayerNorm, projections, gating, core) alone: a profiling aid
        r = time_module(args, args.workload, args.steps, args.warmup)
        print(json.dumps({"metric": "tri_attn_module_fwd_bwd_ms", "value": r["ms_per_step"], "unit": "ms",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": r["ms_per_step"], "higher_is_better": False, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": args.workload}, "detail": r}), flush=True)
        return
    if args.workload.startswith("trimul_block_"):
        # the whole triangle multiplicative update block alone: a profiling aid
        r = time_trimul_module(args, args.workload, args.ending, args.steps, args.warmup)
        print(json.dumps({"metric": "tri_mul_module_fwd_bwd_ms", "value": r["ms_per_step"], "unit": "ms",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": r["ms_per_step"], "higher_is_better": False, "dtype": "bf16",
                          "data": "synthetic",
                          "config": {"workload": args.workload, "edges": "incoming" if args.ending else "outgoing"},
                          "detail": r}), flush=True)
        return
    if args.workload.startswith("trimul_"):
        # the triangle-multiplication contraction alone (a profiling aid, not the metric)
        d = "incoming" if args.ending else "outgoing"
        r = time_trimul(args, args.workload, args.ending, args.steps, args.warmup)
        print(json.dumps({"metric": "tri_mul_fwd_bwd_TFLOPs", "value": r["TFLOPs"], "unit": "TFLOP/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": r["ms_per_step"], "higher_is_better": True, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": args.workload, "edges": d},
                          "detail": r}), flush=True)
        return
    extras = not args.quick and args.workload == "crop768" and not args.ending
    line = run_workload(args, args.workload, args.ending, extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
