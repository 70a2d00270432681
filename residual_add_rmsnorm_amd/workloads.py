"""Seeded synthetic inputs for the fused epilogue and the QK norm.

This module only draws numbers: a CPU ``torch.Generator`` seeded per workload,
normal draws scaled to the stated spread, optional outliers, and a cast to
bf16 (round to nearest even). It holds none of the method's arithmetic, so both
the HIP path and the CPU oracle can take their inputs from it.

Draw order, per workload (each array drawn in fp32, multiplied by its outlier
mask when the workload has outliers, then cast to bf16):
  1. partials p = 0..P-1: randn(T, H) * sigma, then for each buffer right after
     it, mask = rand(T, H) < outlier_frac and masked elements *= outlier_mult;
  2. residual: randn(T, H);
  3. weight: 1 + 0.1 * randn(H).
QK workloads: qkv = randn(T, row) with its outlier mask; wq = 1 + 0.1 randn(q);
wk = 1 + 0.1 randn(kv); then tp_world - 1 further shard rows drawn like qkv
(the other ranks' local rows, used only to form the sum of shard means).
The MLA all-gather workload draws like a QK workload: the gathered rows
(q_lora_rank | kv_lora_rank | rope), then the x and y gammas. The sharded
workload: this rank's rows, the weight, then tp_world - 1 further ranks' rows.
The reduce-scatter workload: P partials of token_num rows, add_in, residual
and weight (add_in and residual cover the slice only).

The shapes follow the pages' workloads: a 7168-wide decode step, 8192-wide
prefill with per-token FP8, 7168-wide block-FP8 with 1x128 groups, and the
MiniMax-M2 attention shard (global q 6144 / k 1024, from the tokenspeed
``trtllm.py`` page, section "MiniMax QK fused AR + RMSNorm"), and MLA rows of
q_lora_rank 1536 | kv_lora_rank 512 | rope 64 = 2112, the largest hidden width
the same page's "AllGather fusion" section accepts.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                      # "norm", "quant_token", "quant_block", "quant_static",
                                   # "rs", "qk", "sharded", "mla"
    T: int
    H: int = 0                     # hidden width (fused epilogue)
    P: int = 0                     # number of partial buffers
    sigma: float = 1.0             # spread of the partials
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    group_size: int = 128          # block FP8 group width
    row_stride: int = 0            # QK: elements between rows of qkv
    q_size: int = 0
    kv_size: int = 0
    tp_world: int = 1              # QK mode B: shards folded into the rsqrt
    token_num: int = 0             # reduce-scatter: tokens in each partial buffer
    token_offset: int = 0          # reduce-scatter: first token of this GPU's slice
    pattern: int = 0               # reduce-scatter: fusion pattern code
    static_scale: float = 0.0      # static FP8: the per-tensor dequantisation scale
    eps: float = 1e-6
    seed: int = 0
    want_norm: bool = True         # FP8 kinds: also write bf16 norm_out (MLA: x_norm_out)
    description: str = ""

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=int(T))

    # ---- algorithmic bytes: each input read once, each output written once,
    # the weight counted once per launch.
    def bytes_per_token(self) -> int:
        if self.kind == "qk":
            read = (self.q_size + self.kv_size) * 2
            write = (self.q_size + self.kv_size) * 2
            var = 8 if self.tp_world > 1 else 0
            return read + write + var
        if self.kind == "sharded":
            return self.q_size * 2 + 4 + self.q_size * 2          # row + var_in, out
        if self.kind == "rs":
            read = (self.P + 2) * self.H * 2                      # partials, add_in, residual
            return read + self.H * 2 + self.H + 4 * (self.H // self.group_size)
        if self.kind == "mla":
            read = (self.q_size + self.kv_size) * 2
            write = self.kv_size * 2 + self.q_size + 4 * (self.q_size // self.group_size)
            if self.want_norm:
                write += self.q_size * 2
            return read + write
        read = (self.P + 1) * self.H * 2
        write = self.H * 2                                   # residual_out
        if self.kind == "norm" or self.want_norm:
            write += self.H * 2                              # norm_out
        if self.kind == "quant_token":
            write += self.H + 4
        elif self.kind == "quant_static":
            write += self.H
        elif self.kind == "quant_block":
            write += self.H + 4 * (self.H // self.group_size)
        return read + write

    def weight_bytes(self) -> int:
        if self.kind in ("qk", "mla", "sharded"):
            return (self.q_size + self.kv_size) * 2
        return self.H * 2 + (4 if self.kind == "quant_static" else 0)

    def algorithmic_bytes(self, T: Optional[int] = None) -> int:
        T = self.T if T is None else T
        return T * self.bytes_per_token() + self.weight_bytes()


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", "norm", T=16, H=1024, P=1, sigma=1.0,
        description="fused add+RMSNorm T=16 H=1024 P=1, bf16 outputs"),
    "decode": Workload(
        "decode", "norm", T=128, H=7168, P=4, sigma=0.5,
        description="decode step T=128 H=7168 P=4, bf16 outputs"),
    "prefill_fp8_token": Workload(
        "prefill_fp8_token", "quant_token", T=8192, H=8192, P=8, sigma=0.35,
        outlier_frac=0.001, outlier_mult=64.0, want_norm=False,
        description="prefill T=8192 H=8192 P=8, 0.1% x64 outliers, per-token e4m3 + fp32 scale"),
    "fp8_block": Workload(
        "fp8_block", "quant_block", T=16384, H=7168, P=2, sigma=0.7, group_size=128,
        want_norm=False,
        description="T=16384 H=7168 P=2, e4m3 with one fp32 scale per 1x128 group"),
    "qk_local": Workload(
        "qk_local", "qk", T=4096, row_stride=8192, q_size=6144, kv_size=1024,
        outlier_frac=0.01, outlier_mult=50.0, tp_world=1,
        description="MiniMax QK RMSNorm T=4096, row 8192 = q 6144 | k 1024 | v 1024, local means"),
    "qk_sharded": Workload(
        "qk_sharded", "qk", T=4096, row_stride=8192, q_size=6144, kv_size=1024,
        outlier_frac=0.01, outlier_mult=50.0, tp_world=4,
        description="MiniMax QK RMSNorm T=4096, supplied sum of 4 shard means, tp_world=4"),
    "sharded_post": Workload(
        "sharded_post", "sharded", T=16384, row_stride=2048, q_size=2048, tp_world=4,
        outlier_frac=0.01, outlier_mult=50.0,
        description="sharded-hidden RMSNorm post stage, T=16384 rows of 2048 (8192 over 4 "
                    "ranks), supplied sum of 4 local means"),
    "static_fp8": Workload(
        "static_fp8", "quant_static", T=8192, H=8192, P=8, sigma=0.35, outlier_frac=0.001,
        outlier_mult=64.0, want_norm=False, static_scale=0.02,
        description="prefill T=8192 H=8192 P=8 with a static per-tensor e4m3 scale 0.02"),
    "rs_fp8_block": Workload(
        "rs_fp8_block", "rs", T=2048, H=7168, P=8, sigma=0.5, token_num=16384,
        token_offset=6144, pattern=7,
        description="reduce-scatter epilogue, slice of 2048 of 16384 tokens, H=7168, P=8 "
                    "peers + add_in, 1x128 e4m3"),
    "mla_ag_fp8": Workload(
        "mla_ag_fp8", "mla", T=8192, row_stride=2112, q_size=1536, kv_size=512,
        outlier_frac=0.001, outlier_mult=64.0, want_norm=False,
        description="MLA all-gather epilogue T=8192 rows of 1536 | 512 | 64: y bf16, "
                    "x as 1x128 e4m3 + fp32 scales"),
}


def _draw(gen: torch.Generator, shape, sigma: float, frac: float, mult: float) -> torch.Tensor:
    a = torch.randn(shape, generator=gen, dtype=torch.float32)
    if sigma != 1.0:
        a.mul_(sigma)
    if frac > 0.0:
        mask = torch.rand(shape, generator=gen, dtype=torch.float32) < frac
        a[mask] *= mult
    return a.to(torch.bfloat16)


@dataclass
class NormInputs:
    workload: Workload
    partials: List[torch.Tensor]   # P x bf16 [T, H] (CPU)
    residual: torch.Tensor         # bf16 [T, H]
    weight: torch.Tensor           # bf16 [H]
    add_in: Optional[torch.Tensor] = None  # reduce-scatter: bf16 [T, H]


@dataclass
class QkInputs:
    workload: Workload
    qkv: torch.Tensor              # bf16 [T, row_stride] (CPU)
    q_weight: torch.Tensor         # bf16 [q_size]
    k_weight: torch.Tensor         # bf16 [kv_size]
    shards: List[torch.Tensor] = field(default_factory=list)  # tp_world-1 more [T, row_stride]


def make_inputs(w: Workload, T: Optional[int] = None, seed: Optional[int] = None):
    """Draws the inputs of workload ``w`` (optionally with another token count
    or seed) as CPU tensors."""
    if T is not None:
        w = w.with_tokens(T)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else int(seed))
    if w.kind == "sharded":
        x = _draw(gen, (w.T, w.row_stride), 1.0, w.outlier_frac, w.outlier_mult)
        weight = (1.0 + 0.1 * torch.randn(w.q_size, generator=gen)).to(torch.bfloat16)
        shards = [_draw(gen, (w.T, w.row_stride), 1.0, w.outlier_frac, w.outlier_mult)
                  for _ in range(w.tp_world - 1)]
        return QkInputs(w, x, weight, weight[:0], shards)
    if w.kind == "rs":
        partials = [_draw(gen, (w.token_num, w.H), w.sigma, w.outlier_frac, w.outlier_mult)
                    for _ in range(w.P)]
        add_in = _draw(gen, (w.T, w.H), w.sigma, 0.0, 1.0)
        residual = _draw(gen, (w.T, w.H), 1.0, 0.0, 1.0)
        weight = (1.0 + 0.1 * torch.randn(w.H, generator=gen)).to(torch.bfloat16)
        return NormInputs(w, partials, residual, weight, add_in)
    if w.kind in ("qk", "mla"):
        qkv = _draw(gen, (w.T, w.row_stride), 1.0, w.outlier_frac, w.outlier_mult)
        wq = (1.0 + 0.1 * torch.randn(w.q_size, generator=gen)).to(torch.bfloat16)
        wk = (1.0 + 0.1 * torch.randn(w.kv_size, generator=gen)).to(torch.bfloat16)
        shards = [_draw(gen, (w.T, w.row_stride), 1.0, w.outlier_frac, w.outlier_mult)
                  for _ in range(w.tp_world - 1)]
        return QkInputs(w, qkv, wq, wk, shards)
    partials = [_draw(gen, (w.T, w.H), w.sigma, w.outlier_frac, w.outlier_mult)
                for _ in range(w.P)]
    residual = _draw(gen, (w.T, w.H), 1.0, 0.0, 1.0)
    weight = (1.0 + 0.1 * torch.randn(w.H, generator=gen)).to(torch.bfloat16)
    return NormInputs(w, partials, residual, weight)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (same memory order, CPU copy)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bf16 tensor")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 CPU tensor."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
