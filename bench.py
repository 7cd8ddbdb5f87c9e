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
  cpu_baseline : the FP64 oracle timed on this host on a bounded sample of the
                 same workload (sampled attention rows and bias-gradient rows),
                 scaled to the whole workload, with the host's thread count and
                 CPU model;
  mfma_probe   : the sustained bf16 matrix-core rate this device reaches with
                 independent back-to-back 32x32x16 products, and the backward main
                 kernel's and the whole step's fractions of it;
  phases       : median and 90th-percentile forward, backward and step times over
                 the timed steps (events on the launch stream), the same for each
                 of the backward's four kernels (events the library records
                 between them), the algorithmic bytes of one step and the rate they
                 imply, the pair-bias and bias-gradient bytes of a step with the
                 measured rate of the dbias reduction, and whether the outputs of
                 the first and last timed steps are bitwise identical.
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
    """Row chunks per (batch, head, block) in the library's launch plan: one round of
    workgroups over the MI355X's 256 compute units (at least one chunk, at most N)."""
    c = max(1, min(N, cus // groups))
    per = -(-N // c)
    return -(-N // per)


def bias_dbias_bytes(B: int, N: int, H: int, dbias_bytes: int = 2) -> dict:
    """Pair-bias and bias-gradient HBM bytes of one step.  Every forward workgroup
    (b, h, 64-query block, row chunk) and every backward workgroup (b, h, 64-key
    block, row chunk) stages its bias block once; the backward main kernel writes
    one fp32 dbias partial per row chunk, which the dbias reduction reads back
    before writing dbias."""
    nb = B * H * N * N
    blocks = -(-N // 64)
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


def cpu_baseline(inp, rows: int, dbias_rows: int):
    """Oracle time on `rows` attention rows (o, lse, dq, dk, dv) plus `dbias_rows`
    bias-gradient rows, scaled to the full problem."""
    import numpy as np
    import oracle
    import seeded_inputs as si

    B, N, _, H, D = inp["q"].shape
    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    p = oracle.Problem(inp["q"], inp["k"], inp["v"], inp["bias"], inp["mask"], inp["do"])
    rng = np.random.default_rng(0)
    sel_rows = [(0, int(r)) for r in rng.choice(N, size=min(rows, N), replace=False)]
    sel_db = [(0, int(h), int(j)) for h, j in zip(rng.integers(0, H, dbias_rows),
                                                  rng.integers(0, N, dbias_rows))]
    t0 = time.perf_counter()
    p.rows(sel_rows)
    t1 = time.perf_counter()
    p.dbias(sel_db)
    t2 = time.perf_counter()
    t_full = (t1 - t0) * (B * N / len(sel_rows)) + (t2 - t1) * (B * H * N / len(sel_db))
    flops = si.flop_count(B, N, H, D, inp["mask"])
    return {
        "value": flops / t_full / 1e12,
        "unit": "TFLOP/s",
        "cores": int(os.environ.get("OMP_NUM_THREADS", threads)),
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": (f"{len(sel_rows)} of {B * N} attention rows (forward and q/k/v gradients, "
                   f"{t1 - t0:.1f} s) and {len(sel_db)} of {B * H * N} bias-gradient rows "
                   f"({t2 - t1:.1f} s), scaled to the whole workload; est. {t_full:.0f} s"),
    }


def run_workload(args, workload: str, ending: bool, with_cpu_baseline: bool) -> dict:
    """Time fwd+bwd steps of one workload and return its JSON line as a dict."""
    import seeded_inputs as si
    import triangle_attention_amd as ta

    w = si.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: {w.description}")
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

    def step(events=None):
        return bwd(*fwd(), events=events)

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hip = HipEvents()
    # five events per step around the backward's four kernels (statistics, main, dQ
    # reduction, dbias reduction), recorded by the library on the launch stream
    ev = [[hip.create() for _ in range(5)] for _ in range(args.steps)]
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    outs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        marks[i][0].record()
        fo = fwd()
        marks[i][1].record()
        grads = bwd(*fo, events=ev[i])
        marks[i][2].record()
        if i == 0 or i == args.steps - 1:
            outs.append(fo + tuple(grads))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    kern = {name: [hip.elapsed_ms(e[i], e[i + 1]) for e in ev]
            for i, name in enumerate(("bwd_prep", "bwd_main", "reduce_dq", "reduce_dbias"))}
    main_ms = statistics.mean(kern["bwd_main"])
    for e in ev:
        for x in e:
            hip.destroy(x)
    log(f"{ms:.3f} ms/step, backward main kernel {main_ms:.3f} ms")

    fwd_ms = [m[0].elapsed_time(m[1]) for m in marks]
    bwd_ms = [m[1].elapsed_time(m[2]) for m in marks]
    step_ms = [m[0].elapsed_time(m[2]) for m in marks]
    same = all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
               for x, y in zip(outs[0], outs[-1]))
    nbytes = algorithmic_bytes(w.B, w.N, w.H, w.D, w.mask != "none", 4 if args.residual == "fp32" else 2)
    flops = si.flop_count(w.B, w.N, w.H, w.D, inp["mask"])
    value = flops / (ms * 1e-3) / 1e12
    bwd_main_flops = flops * 10 / 14   # S, dP, dV, dK, dQ products of the backward
    achieved = bwd_main_flops / (main_ms * 1e-3) / 1e12
    bd = bias_dbias_bytes(w.B, w.N, w.H)
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
        "phases": {"fwd_ms": quantiles(fwd_ms), "bwd_ms": quantiles(bwd_ms), "step_ms": quantiles(step_ms),
                   "bwd_kernels_ms": {n: quantiles(v) for n, v in kern.items()},
                   "bias_dbias": bd,
                   "algorithmic_bytes_per_step": nbytes,
                   "algorithmic_GBps": round(nbytes / (statistics.median(step_ms) * 1e-3) / 1e9, 1),
                   "deterministic_first_vs_last_step": bool(same)},
    }
    log("matrix-core probe")
    probe = mfma_probe_tflops()
    line["mfma_probe"] = {"TFLOPs": round(probe, 1),
                          "what": "sustained v_mfma_f32_32x32x16_bf16 rate of this device "
                                  "(four waves per SIMD, independent accumulators)",
                          "bwd_main_frac": round(achieved / probe, 4),
                          "step_frac": round(value / probe, 4)}
    if with_cpu_baseline:
        log("cpu baseline (oracle sample)")
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows, args.cpu_dbias_rows)
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
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--cpu-dbias-rows", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
            line = run_workload(args, wl, ending, not args.no_cpu_baseline and wl == "crop768" and not ending)
            print(json.dumps(line), flush=True)
        return
    line = run_workload(args, args.workload, args.ending, not args.no_cpu_baseline)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
