"""Compile the gfx950 HIP library in-tree: triangle_attention_amd/libtri_attn.so."""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
ROOT = HERE.parent
SRC = HERE / "csrc" / "tri_attn.hip"
# the triangle multiplicative update's contraction, built into the same library
TRI_MUL_SRC = HERE / "csrc" / "tri_mul.hip"
# the triangle-attention module around the core (LayerNorm, projections, gating)
MODULE_SRC = HERE / "csrc" / "tri_module.hip"
LIB = HERE / "libtri_attn.so"
# the matrix-core rate probe bench.py reports next to the published peak
PROBE_SRC = HERE / "csrc" / "mfma_probe.hip"
PROBE_LIB = HERE / "libmfma_probe.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU forms are disabled for all device code (-packed-fp32-ops).
# MFMA results start in architectural VGPRs (-amdgpu-mfma-vgpr-form): the
# per-tile score, dP and dQ products are read by VALU code, and only the
# long-lived backward accumulators (dbias, dK, dV) end up in AGPRs.  The
# iterative ILP machine-scheduling strategy orders the backward main kernel's
# single wave (one per SIMD, so nothing else hides its latencies) better than the
# default occupancy-driven one: 3-5 % less backward time at N = 384..768.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
         "-Wno-unused-command-line-argument"]


def _compile(srcs, lib: Path, verbose: bool) -> None:
    tmp = lib.with_suffix(".so.tmp")
    cmd = [HIPCC, *FLAGS, "-I", str(ROOT / "include"), "-o", str(tmp), *[str(s) for s in srcs]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {lib}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> Path:
    """Compile the library and the matrix-core probe; returns the library's path."""
    _compile([SRC, TRI_MUL_SRC, MODULE_SRC], LIB, verbose)
    _compile([PROBE_SRC], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
