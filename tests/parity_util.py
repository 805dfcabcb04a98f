"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and measure their difference.

The oracle side decodes the exact stored bits of q, k, v to float64 itself
(oracle.formats); the GPU side goes through the C ABI binding only.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import transformer_attention_08_amd as fa
import workload

# Tolerances on max |O_gpu - O_ref| (absolute, N(0,1) inputs) per input type,
# and on LSE.
O_TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 1e-2, "fp8": 6e-2}
LSE_TOL = 1e-3


def gpu_forward(inp: workload.Inputs, causal: bool, scale: float, device="cuda"):
    """O and LSE from the HIP path as float64 NumPy arrays."""
    d = inp.to(device)
    if inp.dtype == "fp8":
        o, lse = fa.forward_fp8(d.q, d.k, d.v, inp.q_descale, inp.k_descale, inp.v_descale,
                                causal=causal, scale=scale)
    else:
        o, lse = fa.forward(d.q, d.k, d.v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().to(torch.float64).numpy(), lse.cpu().to(torch.float64).numpy()


def oracle_inputs(inp: workload.Inputs):
    q = oracle.decode(inp.bits("q"), inp.dtype, inp.q_descale)
    k = oracle.decode(inp.bits("k"), inp.dtype, inp.k_descale)
    v = oracle.decode(inp.bits("v"), inp.dtype, inp.v_descale)
    return q, k, v


def oracle_forward(inp: workload.Inputs, causal: bool, scale: float, rows=None):
    q, k, v = oracle_inputs(inp)
    return oracle.attention(q, k, v, scale, causal, rows=rows)


def half_ulp(x: np.ndarray, fmt: str) -> np.ndarray:
    """Half a unit in the last place of |x| in the output format (0 for f32)."""
    mant = {"bf16": 7, "f16": 10, "f32": 23}[fmt]
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    if fmt == "f16":
        e = np.maximum(e, -14)
    return 0.5 * np.exp2(e - mant)


def report(o_gpu, lse_gpu, o_ref, lse_ref, out_fmt):
    err = np.abs(o_gpu - o_ref)
    resid = err - half_ulp(o_ref, out_fmt)
    return {
        "o_max": float(err.max()) if err.size else 0.0,
        "o_resid": float(resid.max()) if err.size else 0.0,
        "lse_max": float(np.abs(lse_gpu - lse_ref).max()) if lse_ref.size else 0.0,
        "finite": bool(np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all()),
    }
