"""Seeded synthetic inputs shared by the HIP path's tests, the benchmark and the oracle.

This module only draws random numbers and describes workload shapes. It holds
none of the attention arithmetic: no scores, no softmax, no rotation, no merge.
Both the fp64 oracle and the HIP kernels consume exactly the tensors produced
here, so that input quantisation is never counted as kernel error.

Recipe (one generator per workload, seed fixed in advance):
  q, then k, then v are drawn in that order as float32 N(0, 1) from
  ``torch.Generator(device).manual_seed(seed)`` and cast with
  round-to-nearest-even to the workload's dtype.  Layout is contiguous
  [B, H, N, D] row-major.  Small cases draw on the CPU; full-size workloads
  draw on the GPU (the 2 x 537M-element decode cache takes ~40 s on the CPU),
  and the oracle is then handed exact copies of the slices it needs.

The shapes follow the workloads the pages measure on: the AttnFuse listing's
causal forward at B=4 H=12 N=4096 D=64 fp16 (its Tables 1-3), its RoPE+causal
and sliding-window (W=256) variants (Tables 2, 4, 6, 7), and its flash-decoding
geometry of 32 query heads sharing 8 KV heads of width 128 (Table 8), plus a
tiny fp32 single-head case that the oracle finishes in well under a second.
"""
from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["Workload", "WORKLOADS", "TABLE8_DECODE", "by_name", "gen_qkv", "gen_normal", "alibi_slopes", "gen_grad_out",
           "LN_WORKLOAD", "gen_layernorm", "TOPK_WORKLOAD", "gen_logits"]

_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    D: int
    dtype: str          # "f32" | "f16" | "bf16"
    scale: float
    mask: str           # "none" | "causal" | "sliding"
    window: int = 0
    rope_base: float = 0.0
    num_splits: int = 0  # >0: split-KV decode with this many chunks
    seed: int = 0

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DT[self.dtype]

    def shapes(self):
        return ((self.B, self.Hq, self.Nq, self.D),
                (self.B, self.Hkv, self.Nk, self.D),
                (self.B, self.Hkv, self.Nk, self.D))


WORKLOADS = [
    Workload("tiny_dense_f32_n256_d64", B=1, Hq=1, Hkv=1, Nq=256, Nk=256, D=64,
             dtype="f32", scale=1.0 / math.sqrt(64), mask="none", seed=1),
    Workload("causal_f16_b4h12_n4096_d64", B=4, Hq=12, Hkv=12, Nq=4096, Nk=4096, D=64,
             dtype="f16", scale=1.0 / 8.0, mask="causal", seed=2),
    Workload("rope_causal_f16_b4h12_n2048_d64", B=4, Hq=12, Hkv=12, Nq=2048, Nk=2048, D=64,
             dtype="f16", scale=1.0 / 8.0, mask="causal", rope_base=10000.0, seed=3),
    Workload("sliding256_bf16_b8h16_n8192_d128", B=8, Hq=16, Hkv=16, Nq=8192, Nk=8192, D=128,
             dtype="bf16", scale=1.0 / math.sqrt(128), mask="sliding", window=256, seed=4),
    Workload("gqa_decode_bf16_b16_32q8kv_nk32768_d128", B=16, Hq=32, Hkv=8, Nq=1, Nk=32768,
             D=128, dtype="bf16", scale=1.0 / math.sqrt(128), mask="none", num_splits=64,
             seed=5),
]


# AttnFuse Table 8's flash-decoding geometries (query length 1; the table
# states neither batch nor dtype): 32q/8kv/128 with 4096 and 16384 cached
# keys and 64q/8kv/128 with 32768, each at batch 1 and 16, bf16 like the
# decode workload above.  num_splits = 0: the library's chunk-count rule.
TABLE8_DECODE = [
    Workload(f"decode_bf16_b{B}_{Hq}q8kv_nk{Nk}_d128", B=B, Hq=Hq, Hkv=8, Nq=1, Nk=Nk, D=128, dtype="bf16",
             scale=1.0 / math.sqrt(128), mask="none", num_splits=0, seed=seed)
    for seed, (B, Hq, Nk) in enumerate([(1, 32, 4096), (16, 32, 4096), (1, 64, 32768), (16, 64, 32768),
                                        (1, 32, 16384), (16, 32, 16384)], start=11)
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS + TABLE8_DECODE:
        if w.name == name:
            return w
    raise KeyError(name)


def gen_normal(shape, dtype: torch.dtype, gen: torch.Generator) -> torch.Tensor:
    """float32 N(0,1) draw, then a round-to-nearest-even cast to ``dtype``."""
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=gen.device)
    return x.to(dtype) if dtype != torch.float32 else x


def gen_qkv(B, Hq, Hkv, Nq, Nk, D, dtype, seed, device="cpu"):
    """Draw (q, k, v) in the fixed order q, k, v with a generator on ``device``.

    ``dtype`` is a torch dtype or one of "f32", "f16", "bf16".
    Returns contiguous tensors of shapes [B,Hq,Nq,D], [B,Hkv,Nk,D], [B,Hkv,Nk,D].
    """
    if isinstance(dtype, str):
        dtype = _DT[dtype]
    g = torch.Generator(device=device).manual_seed(int(seed))
    q = gen_normal((B, Hq, Nq, D), dtype, g)
    k = gen_normal((B, Hkv, Nk, D), dtype, g)
    v = gen_normal((B, Hkv, Nk, D), dtype, g)
    return q, k, v


def gen_grad_out(shape, dtype, seed, device="cpu"):
    """dO for a backward: N(0,1) float32 from its own generator, cast to ``dtype``."""
    if isinstance(dtype, str):
        dtype = _DT[dtype]
    g = torch.Generator(device=device).manual_seed(int(seed))
    return gen_normal(shape, dtype, g)


def alibi_slopes(H: int):
    """The usual geometric ALiBi slope schedule 2^(-8h/H), h = 1..H (a fixed input)."""
    return [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]


def gen_workload(w: Workload, seed: int | None = None, device="cpu"):
    return gen_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, w.torch_dtype,
                   w.seed if seed is None else seed, device=device)


# LayerNorm (the second cascaded reduction): the pages' workload tables for
# it are missing, so the shape is chosen: the hidden states of the Llama-3-8B
# step of AttnFuse Table 9 (width 4096) for B=4 sequences of 4096 tokens.
LN_WORKLOAD = dict(name="layernorm_bf16_r16384_h4096", rows=16384, H=4096, dtype="bf16", eps=1e-5, seed=6)


def gen_layernorm(rows, H, dtype, seed, device="cpu"):
    """(x [rows, H], gamma [H], beta [H]).  Rows get their own offset in
    [-8, 8) and spread in [0.5, 2) (so the mean is large next to the spread,
    the case a one-pass sum of squares gets wrong); gamma = 1 + 0.1 N(0,1),
    beta = 0.1 N(0,1).  Draw order: x noise, offsets, spreads, gamma, beta."""
    if isinstance(dtype, str):
        dtype = _DT[dtype]
    g = torch.Generator(device=device).manual_seed(int(seed))
    z = torch.randn((rows, H), generator=g, dtype=torch.float32, device=device)
    off = torch.rand((rows, 1), generator=g, dtype=torch.float32, device=device) * 16.0 - 8.0
    spread = torch.rand((rows, 1), generator=g, dtype=torch.float32, device=device) * 1.5 + 0.5
    gamma = 1.0 + 0.1 * torch.randn((H,), generator=g, dtype=torch.float32, device=device)
    beta = 0.1 * torch.randn((H,), generator=g, dtype=torch.float32, device=device)
    return (z * spread + off).to(dtype), gamma.to(dtype), beta.to(dtype)


# Softmax -> TopK (the max/+ cascade): the pages give no shape, so the chosen
# one is a mixture-of-experts router: 16384 tokens over 256 experts, top 8.
TOPK_WORKLOAD = dict(name="softmax_topk_bf16_r16384_e256_k8", rows=16384, E=256, k=8, dtype="bf16", seed=7)


def gen_logits(rows, E, dtype, seed, device="cpu"):
    """Router logits: 2 * N(0,1) float32, cast to ``dtype`` (bf16 makes ties common)."""
    if isinstance(dtype, str):
        dtype = _DT[dtype]
    g = torch.Generator(device=device).manual_seed(int(seed))
    return (2.0 * torch.randn((rows, E), generator=g, dtype=torch.float32, device=device)).to(dtype)
