"""Seeded synthetic inputs for triangle attention.

This module only draws random tensors and builds key masks. It holds none of
the method's arithmetic, so both the HIP path (through its tests and the bench)
and the FP64 oracle can take their inputs from it without sharing any code.

Shapes follow the Pairformer pair representation that the TurboPairFormer pages
describe (crop sizes 384/640/768, "Результаты тестирования" / "crop size不是一个普通参数"):
  q, k, v, dO : [B, N, N, H, D] bfloat16, element [b, i, j, h, c], c contiguous
  bias        : [B, H, N, N]    bfloat16, element [b, h, j, k] (shared by all rows i)
  mask        : [B, N, N]       uint8,    element [b, i, k], nonzero = key k attends

The pages train on real OpenFold3 pair activations at those crop sizes; no dataset
or trained weights are used here. i.i.d. normal tensors of the same shapes stand in
for them, rounded to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

# tensor tags: each tensor of a workload draws from its own generator,
# seeded with seed * 16 + tag
_TAG = {"q": 0, "k": 1, "v": 2, "do": 3, "bias": 4, "length": 5, "tm_a": 6, "tm_b": 7, "tm_g": 8,
        "md_z": 9, "md_ln": 10, "md_wqkvg": 11, "md_wb": 12, "md_wo": 13, "md_dy": 14,
        "tb_z": 15, "tb_ln": 16, "tb_win": 17, "tb_wout": 18, "tb_dy": 19, "tb_mask": 20}


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based position in the workload list; seed = 1000 + index
    B: int
    N: int
    H: int
    D: int
    bias_std: float
    mask: str           # "none" | "pad32" | "ragged512"
    description: str

    @property
    def seed(self) -> int:
        return 1000 + self.index


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny64", 1, 1, 64, 4, 32, 1.0, "none",
                 "B=1 N=64 H=4 d=32, all keys valid"),
        Workload("pad256", 2, 1, 256, 4, 32, 1.0, "pad32",
                 "B=1 N=256 H=4 d=32, last 32 keys of every row masked"),
        Workload("crop384", 3, 1, 384, 4, 32, 1.0, "none",
                 "B=1 N=384 H=4 d=32, all keys valid"),
        Workload("crop640", 4, 1, 640, 4, 32, 4.0, "ragged512",
                 "B=1 N=640 H=4 d=32, bias ~ N(0, 4^2), seeded valid length in [512, 640]"),
        Workload("crop768", 5, 1, 768, 4, 32, 1.0, "none",
                 "B=1 N=768 H=4 d=32, all keys valid (starting and ending node)"),
        Workload("crop768_h8d16", 6, 1, 768, 8, 16, 1.0, "none",
                 "B=1 N=768 H=8 d=16 (the same 128 pair channels as H=4 d=32), all keys valid"),
        Workload("crop768_h2d64", 7, 1, 768, 2, 64, 1.0, "none",
                 "B=1 N=768 H=2 d=64 (the same 128 pair channels as H=4 d=32), all keys valid"),
    ]
}


def _gen(seed: int, tag: str) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 16 + _TAG[tag])
    return g


def _randn_bf16(shape, seed: int, tag: str, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=_gen(seed, tag), dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16)


def make_mask(B: int, N: int, kind: str, seed: int) -> torch.Tensor:
    """Key mask [B, N, N] uint8 (mask[b, i, k] != 0: key k is attended in row i)."""
    m = torch.ones((B, N, N), dtype=torch.uint8)
    if kind == "none":
        return m
    if kind == "pad32":
        m[:, :, N - 32:] = 0
        return m
    if kind == "ragged512":
        lengths = valid_lengths(B, N, kind, seed)
        for b in range(B):
            m[b, :, lengths[b]:] = 0
        return m
    if kind == "random":
        g = _gen(seed, "length")
        m = (torch.rand((B, N, N), generator=g) < 0.8).to(torch.uint8)
        return m
    raise ValueError(f"unknown mask kind {kind!r}")


def valid_lengths(B: int, N: int, kind: str, seed: int) -> list[int]:
    """Per-batch valid key length; for "ragged512" drawn uniformly from [512, N]."""
    if kind == "ragged512":
        g = _gen(seed, "length")
        return [int(x) for x in torch.randint(512, N + 1, (B,), generator=g)]
    if kind == "pad32":
        return [N - 32] * B
    return [N] * B


def make_problem(B: int, N: int, H: int, D: int, seed: int, *,
                 bias_std: float = 1.0, mask: str = "none") -> dict:
    """Seeded bf16 inputs of one triangle-attention problem (CPU tensors)."""
    shp = (B, N, N, H, D)
    return {
        "q": _randn_bf16(shp, seed, "q"),
        "k": _randn_bf16(shp, seed, "k"),
        "v": _randn_bf16(shp, seed, "v"),
        "do": _randn_bf16(shp, seed, "do"),
        "bias": _randn_bf16((B, H, N, N), seed, "bias", bias_std),
        "mask": make_mask(B, N, mask, seed),
    }


def make_workload(name: str) -> dict:
    w = WORKLOADS[name]
    return make_problem(w.B, w.N, w.H, w.D, w.seed, bias_std=w.bias_std, mask=w.mask)


def flop_count(B: int, N: int, H: int, D: int, mask: torch.Tensor | None) -> int:
    """Algorithmic fwd+bwd FLOP count: 2 forward and 5 backward products of
    2*D flop per valid (b, i, h, j, k) score element (exp and the bias-gradient
    adds are not counted)."""
    valid = N * N * B if mask is None else int(mask.to(torch.int64).sum())
    return 14 * D * H * N * valid


# Triangle multiplicative update's contraction: the projected factors a, b and the
# upstream gradient g, channel-major [B, C, N, N] bf16, N(0, 1) entries.  The crop
# sizes are those of the attention workloads, with C = 128 channels.
@dataclass(frozen=True)
class TriMulWorkload:
    name: str
    index: int
    B: int
    N: int
    C: int
    description: str

    @property
    def seed(self) -> int:
        return 2000 + self.index


TRIMUL_WORKLOADS = {
    w.name: w
    for w in [
        TriMulWorkload("trimul_tiny64", 1, 1, 64, 16, "B=1 N=64 C=16"),
        TriMulWorkload("trimul_crop384", 2, 1, 384, 128, "B=1 N=384 C=128"),
        TriMulWorkload("trimul_crop640", 3, 1, 640, 128, "B=1 N=640 C=128"),
        TriMulWorkload("trimul_crop768", 4, 1, 768, 128, "B=1 N=768 C=128"),
    ]
}


def make_trimul(B: int, N: int, C: int, seed: int) -> dict:
    """Seeded bf16 factors a, b and upstream gradient g, each [B, C, N, N] (CPU)."""
    shp = (B, C, N, N)
    return {"a": _randn_bf16(shp, seed, "tm_a"), "b": _randn_bf16(shp, seed, "tm_b"),
            "g": _randn_bf16(shp, seed, "tm_g")}


def make_trimul_workload(name: str) -> dict:
    w = TRIMUL_WORKLOADS[name]
    return make_trimul(w.B, w.N, w.C, w.seed)


def trimul_flop_count(B: int, N: int, C: int) -> int:
    """Forward + backward flops of the contraction: three N^3 products per channel."""
    return 3 * 2 * B * C * N ** 3


# Triangle-attention module around the core: the pair tensor z [B, N, N, C] (C = H * D
# channels), its key mask, the LayerNorm scale and offset (fp32, [C]), the projection
# weights w_qkvg [C, 4 C], w_bias [C, H] and w_out [C, C] (bf16, N(0, 1/C) entries, so
# that every projection has unit variance) and the upstream gradient dy [B, N, N, C].
@dataclass(frozen=True)
class ModuleWorkload:
    name: str
    index: int
    B: int
    N: int
    H: int
    D: int
    mask: str
    description: str

    @property
    def seed(self) -> int:
        return 3000 + self.index


MODULE_WORKLOADS = {
    w.name: w
    for w in [
        ModuleWorkload("module_tiny64", 1, 1, 64, 4, 32, "pad32", "B=1 N=64 H=4 d=32 (C=128), last 32 keys masked"),
        ModuleWorkload("module_crop384", 2, 1, 384, 4, 32, "none", "B=1 N=384 H=4 d=32 (C=128)"),
        ModuleWorkload("module_crop768", 3, 1, 768, 4, 32, "none", "B=1 N=768 H=4 d=32 (C=128)"),
    ]
}


def make_module(B: int, N: int, H: int, D: int, seed: int, mask: str = "none") -> dict:
    """Seeded inputs and parameters of one module problem (CPU tensors)."""
    C = H * D
    ln = torch.randn((2, C), generator=_gen(seed, "md_ln"), dtype=torch.float32) * 0.1
    return {
        "z": _randn_bf16((B, N, N, C), seed, "md_z"),
        "mask": make_mask(B, N, mask, seed),
        "ln_w": 1.0 + ln[0],
        "ln_b": ln[1].clone(),
        "w_qkvg": _randn_bf16((C, 4 * C), seed, "md_wqkvg", C ** -0.5),
        "w_bias": _randn_bf16((C, H), seed, "md_wb", C ** -0.5),
        "w_out": _randn_bf16((C, C), seed, "md_wo", C ** -0.5),
        "dy": _randn_bf16((B, N, N, C), seed, "md_dy"),
    }


def make_module_workload(name: str) -> dict:
    w = MODULE_WORKLOADS[name]
    return make_module(w.B, w.N, w.H, w.D, w.seed, w.mask)


# Triangle multiplicative update block: the pair tensor z [B, N, N, C], a pair mask
# [B, N, N] (uint8, 1 = kept), the two LayerNorms' scales and offsets (fp32 [C]), the
# input projections w_in [C, 5 C] (a gate, a, b gate, b, output gate) and the output
# projection w_out [C, C] (bf16, N(0, 1/C) entries) and the upstream gradient dy.
@dataclass(frozen=True)
class TriMulModuleWorkload:
    name: str
    index: int
    B: int
    N: int
    C: int
    mask: str
    description: str

    @property
    def seed(self) -> int:
        return 4000 + self.index


TRIMUL_MODULE_WORKLOADS = {
    w.name: w
    for w in [
        TriMulModuleWorkload("trimul_block_tiny64", 1, 1, 64, 128, "pad32",
                             "B=1 N=64 C=128, the last 32 positions of every row masked"),
        TriMulModuleWorkload("trimul_block_crop768", 2, 1, 768, 128, "none", "B=1 N=768 C=128"),
    ]
}


def make_trimul_module(B: int, N: int, C: int, seed: int, mask: str = "none") -> dict:
    """Seeded inputs and parameters of one triangle-multiplication block (CPU tensors)."""
    ln = torch.randn((4, C), generator=_gen(seed, "tb_ln"), dtype=torch.float32) * 0.1
    if mask == "random":
        m = (torch.rand((B, N, N), generator=_gen(seed, "tb_mask")) < 0.8).to(torch.uint8)
    else:
        m = make_mask(B, N, mask, seed)
    return {
        "z": _randn_bf16((B, N, N, C), seed, "tb_z"),
        "mask": m,
        "ln_in_w": 1.0 + ln[0], "ln_in_b": ln[1].clone(),
        "ln_out_w": 1.0 + ln[2], "ln_out_b": ln[3].clone(),
        "w_in": _randn_bf16((C, 5 * C), seed, "tb_win", C ** -0.5),
        "w_out": _randn_bf16((C, C), seed, "tb_wout", C ** -0.5),
        "dy": _randn_bf16((B, N, N, C), seed, "tb_dy"),
    }


def make_trimul_module_workload(name: str) -> dict:
    w = TRIMUL_MODULE_WORKLOADS[name]
    return make_trimul_module(w.B, w.N, w.C, w.seed, w.mask)
