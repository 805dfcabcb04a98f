"""Seeded synthetic inputs for the attention forward and backward passes.

This module only draws and encodes inputs; it holds none of the attention
arithmetic. Both the HIP path (through its binding) and the CPU oracle
consume exactly the tensors made here, so the two sides see identical bits.

Recipe (the same for every configuration):
  * one CPU ``torch.Generator`` seeded with ``seed``;
  * ``torch.randn`` in float32, drawn in the order Q, K, V, each of shape
    [batch, heads, n, d_k] (the per-head [n x d_k] matrices of the
    "Queries, keys and values" slide of "Case study: FlashAttention",
    with a leading batch axis);
  * an optional multiplier per tensor (the fp8 workload scales Q and K by 4
    so that raw scores reach large magnitudes);
  * a cast to the storage dtype with round-to-nearest-even.

For the backward pass the output gradient dO is the fourth draw of the same
generator (after Q, K, V), of the same shape, N(0,1), cast the same way.

For fp8 (OCP e4m3fn, largest finite value 448) each tensor gets one fp32
descale s = amax(|x|) / 448; the stored code is x / s clamped to [-448, 448]
and rounded to nearest even. The value a code stands for is code * s.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

E4M3_MAX = 448.0

# Storage dtype names used across the repository.
DTYPES = ("f32", "f16", "bf16", "fp8")

_TORCH_DTYPE = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8": torch.float8_e4m3fn,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-forward problem: shape, dtype, mask and input law."""

    name: str
    batch: int
    heads: int
    n: int
    d_k: int
    dtype: str
    causal: bool
    qk_mult: float = 1.0  # Q and K are drawn N(0,1) * qk_mult; V is N(0,1)

    @property
    def scale(self) -> float:
        """Score scale 1/sqrt(d_k), rounded to fp32 (the value the kernel gets)."""
        return float(torch.tensor(1.0 / math.sqrt(self.d_k), dtype=torch.float32))

    @property
    def out_dtype(self) -> str:
        return "bf16" if self.dtype == "fp8" else self.dtype


# The five workloads: a tiny fp32 correctness case, an fp16 multi-head causal
# case, the Llama-3-8B layer shape (h=32, d_k=128, n=8192; bf16, causal), its
# 32k long-context variant, and an fp8 variant without a mask.
WORKLOADS = {
    "single_head_f32": Workload("single_head_f32", 1, 1, 256, 64, "f32", False),
    "mha_f16_causal": Workload("mha_f16_causal", 2, 32, 2048, 128, "f16", True),
    "llama3_8b_bf16_causal": Workload("llama3_8b_bf16_causal", 1, 32, 8192, 128, "bf16", True),
    "long_ctx_bf16_causal": Workload("long_ctx_bf16_causal", 1, 32, 32768, 128, "bf16", True),
    "fp8_e4m3_nomask": Workload("fp8_e4m3_nomask", 1, 32, 8192, 128, "fp8", False, qk_mult=4.0),
    # grids far below the chip's 256 CUs: the cases the split-KV path is for
    "two_heads_bf16": Workload("two_heads_bf16", 1, 2, 4096, 128, "bf16", False),
    "four_heads_long_bf16_causal": Workload("four_heads_long_bf16_causal", 1, 4, 16384, 128, "bf16", True),
}


@dataclasses.dataclass
class Inputs:
    """Host (CPU) tensors in storage dtype plus the fp8 descales (1.0 otherwise)."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    dtype: str
    q_descale: float = 1.0
    k_descale: float = 1.0
    v_descale: float = 1.0

    def bits(self, which: str):
        """Raw storage bits of q, k or v as a NumPy array (uint8/16/32)."""
        t = getattr(self, which)
        view = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16, "fp8": torch.uint8}[self.dtype]
        raw = t.contiguous().view(view).numpy()
        unsigned = {"f32": "uint32", "f16": "uint16", "bf16": "uint16", "fp8": "uint8"}[self.dtype]
        return raw.view(unsigned)

    def to(self, device) -> "Inputs":
        return Inputs(self.q.to(device), self.k.to(device), self.v.to(device), self.dtype,
                      self.q_descale, self.k_descale, self.v_descale)


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor fp8 e4m3fn encoding: returns (codes, fp32 descale)."""
    amax = float(x.abs().max())
    s = float(torch.tensor(amax / E4M3_MAX if amax > 0 else 1.0, dtype=torch.float32))
    codes = (x / s).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return codes, s


def make_inputs(batch: int, heads: int, n: int, d_k: int, dtype: str, seed: int,
                qk_mult: float = 1.0, v_mult: float = 1.0) -> Inputs:
    """Draw Q, K, V with the recipe in the module docstring."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    g = torch.Generator().manual_seed(int(seed))
    shape = (batch, heads, n, d_k)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if qk_mult != 1.0:
        q = q * qk_mult
        k = k * qk_mult
    if v_mult != 1.0:
        v = v * v_mult
    if dtype == "fp8":
        q8, qs = quantize_e4m3(q)
        k8, ks = quantize_e4m3(k)
        v8, vs = quantize_e4m3(v)
        return Inputs(q8, k8, v8, dtype, qs, ks, vs)
    td = _TORCH_DTYPE[dtype]
    return Inputs(q.to(td), k.to(td), v.to(td), dtype)


def make_inputs_with_grad(batch: int, heads: int, n: int, d_k: int, dtype: str, seed: int):
    """Q, K, V as ``make_inputs`` plus dO, the generator's fourth draw (f16 / bf16 / f32)."""
    if dtype not in ("f32", "f16", "bf16"):
        raise ValueError("the backward inputs are f32, f16 or bf16")
    g = torch.Generator().manual_seed(int(seed))
    shape = (batch, heads, n, d_k)
    td = _TORCH_DTYPE[dtype]
    q, k, v, do = (torch.randn(shape, generator=g, dtype=torch.float32).to(td) for _ in range(4))
    return Inputs(q, k, v, dtype), do


def workload_inputs(w: Workload, seed: int) -> Inputs:
    return make_inputs(w.batch, w.heads, w.n, w.d_k, w.dtype, seed, qk_mult=w.qk_mult)


def torch_dtype(dtype: str) -> torch.dtype:
    return _TORCH_DTYPE[dtype]


def from_bits(bits, dtype: str) -> torch.Tensor:
    """Build a CPU tensor of storage dtype from raw bits (inverse of Inputs.bits)."""
    import numpy as np

    signed = {"f32": np.int32, "f16": np.int16, "bf16": np.int16, "fp8": np.uint8}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(bits).view(signed).copy())
    view = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "fp8": torch.float8_e4m3fn}[dtype]
    return t.view(view)


def sample_rows(n: int, count: int, seed: int) -> "list[int]":
    """Seeded query-row sample: the first and last rows plus random ones, sorted."""
    g = torch.Generator().manual_seed(int(seed) + 7919)
    edge = min(count // 4, n)
    rows = set(range(edge)) | set(range(max(0, n - edge), n))
    if n > len(rows):
        extra = torch.randint(0, n, (max(0, count - len(rows)),), generator=g).tolist()
        rows |= set(extra)
    return sorted(rows)
