"""GPU parity of the backward pass (fa_backward) against the gradient oracle.

Inputs: Q, K, V and dO are the seeded draws of workload.make_inputs_with_grad.
O and LSE, which the backward takes from the forward, come either from the
oracle (O rounded once to the input type, LSE to fp32) or from the HIP
forward itself (the chain a training step runs); the expected gradients are
always the oracle's, from Q, K, V and dO alone.

Bar: per gradient tensor, max |g_gpu - g_ref| <= tol * max(max |g_ref|, 1e-3)
with tol = 1e-2 for bf16 and 2e-3 for f16. The pages give no error bound for
the backward; the bar is derived from the arithmetic: a CPU model of the
kernel's rounding points (P and dS rounded to the input type for the MFMAs,
O given in the input type, fp32 accumulation, outputs rounded once) on these
input laws reaches 4.9e-3 (bf16) and 7.8e-4 (f16) of max |g_ref|, and the bar
is about twice that.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_08_amd as fa
import workload
from parity_util import gpu_forward, oracle_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f16": 2e-3}
TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def say(*a):
    print(*a, flush=True)


def decode(t: torch.Tensor, dtype: str) -> np.ndarray:
    bits = t.contiguous().view(torch.int16).numpy().view("uint16")
    return oracle.decode(bits, dtype)


def forward_from_oracle(inp, causal, scale):
    q, k, v = oracle_inputs(inp)
    o, lse = oracle.attention(q, k, v, scale, causal)
    return torch.from_numpy(o).to(TDT[inp.dtype]), torch.from_numpy(lse).to(torch.float32)


def run_backward(inp, do, o, lse, causal, scale):
    dev = "cuda"
    d = inp.to(dev)
    dq, dk, dv = fa.backward(d.q, d.k, d.v, o.to(dev), lse.to(dev), do.to(dev), causal=causal,
                             scale=scale)
    torch.cuda.synchronize()
    return [decode(t.cpu(), inp.dtype) for t in (dq, dk, dv)]


def compare(got, ref, dtype, tag=""):
    out = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        err = float(np.abs(g - r).max()) if r.size else 0.0
        ref_max = float(np.abs(r).max()) if r.size else 0.0
        bar = TOL[dtype] * max(ref_max, 1e-3)
        out[name] = (err, ref_max)
        assert np.isfinite(g).all(), (tag, name)
        assert err <= bar, (tag, name, err, ref_max, bar)
    say("   ", tag, {k: "err %.2e (max %.2f)" % v for k, v in out.items()})


SMALL_N = [1, 2, 17, 64, 65, 127, 130, 257, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", SMALL_N)
def test_ragged_shapes_oracle_forward(n, causal, d, dtype):
    b, h = (1, 8) if n % 2 else (2, 3)
    say(f"backward n={n} d={d} causal={causal} dtype={dtype} b={b} h={h}")
    inp, do = workload.make_inputs_with_grad(b, h, n, d, dtype, seed=3 * n + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = forward_from_oracle(inp, causal, scale)
    got = run_backward(inp, do, o, lse, causal, scale)
    q, k, v = oracle_inputs(inp)
    ref = oracle.attention_backward(q, k, v, decode(do, dtype), scale, causal)
    compare(got, ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_chain_with_gpu_forward(causal, dtype):
    b, h, n, d = 1, 4, 700, 128
    say(f"forward + backward chain n={n} causal={causal} dtype={dtype}")
    inp, do = workload.make_inputs_with_grad(b, h, n, d, dtype, seed=17)
    scale = float(np.float32(1 / math.sqrt(d)))
    dev = inp.to("cuda")
    o, lse = fa.forward(dev.q, dev.k, dev.v, causal=causal, scale=scale)
    got = run_backward(inp, do, o.cpu(), lse.cpu(), causal, scale)
    q, k, v = oracle_inputs(inp)
    ref = oracle.attention_backward(q, k, v, decode(do, dtype), scale, causal)
    compare(got, ref, dtype, "chain")


def test_zero_scale_and_deterministic():
    b, h, n, d = 1, 2, 200, 64
    inp, do = workload.make_inputs_with_grad(b, h, n, d, "bf16", seed=5)
    o, lse = forward_from_oracle(inp, True, 0.0)
    got = run_backward(inp, do, o, lse, True, 0.0)
    q, k, v = oracle_inputs(inp)
    ref = oracle.attention_backward(q, k, v, decode(do, "bf16"), 0.0, True)
    assert np.abs(got[0]).max() == 0 and np.abs(got[1]).max() == 0  # dQ = dK = 0 at scale 0
    compare(got, ref, "bf16", "scale 0")
    again = run_backward(inp, do, o, lse, True, 0.0)
    for a_, b_ in zip(got, again):
        assert np.array_equal(a_, b_)


def test_workspace_holds_d_and_lse():
    b, h, n, d = 1, 2, 300, 128
    inp, do = workload.make_inputs_with_grad(b, h, n, d, "bf16", seed=6)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = forward_from_oracle(inp, True, scale)
    dev = inp.to("cuda")
    ws = torch.empty(fa.backward_workspace_size(b, h, n), dtype=torch.uint8, device="cuda")
    fa.backward(dev.q, dev.k, dev.v, o.cuda(), lse.cuda(), do.cuda(), causal=True, scale=scale,
                workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu()
    rows = b * h * n
    dsum = w[:rows * 4].view(torch.float32).double().numpy().reshape(b, h, n)
    off = -(-rows * 4 // 256) * 256
    nl2 = w[off:off + rows * 4].view(torch.float32).double().numpy().reshape(b, h, n)
    ref_d = (decode(do, "bf16") * decode(o, "bf16")).sum(-1)
    assert np.abs(dsum - ref_d).max() <= 1e-4 * max(1.0, np.abs(ref_d).max())
    assert np.abs(nl2 + lse.double().numpy() / math.log(2)).max() <= 1e-5 * np.abs(nl2).max()


def test_llama_shape_sampled_rows_and_keys():
    """b=1, h=32, n=8192, d_k=128, bf16, causal: the GPU forward's O and LSE feed
    the GPU backward; dQ rows and dK / dV key columns of two heads are compared
    with the oracle, and the invariants are checked on every head."""
    b, h, n, d = 1, 32, 8192, 128
    say("backward llama shape, sampled")
    inp, do = workload.make_inputs_with_grad(b, h, n, d, "bf16", seed=0)
    scale = float(np.float32(1 / math.sqrt(d)))
    dev = inp.to("cuda")
    dog = do.cuda()
    o, lse = fa.forward(dev.q, dev.k, dev.v, causal=True, scale=scale)
    dq, dk, dv = fa.backward(dev.q, dev.k, dev.v, o, lse, dog, causal=True, scale=scale)
    torch.cuda.synchronize()
    # invariants on every head and column: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i
    sk = dk.double().sum(dim=2).abs() / dk.double().abs().sum(dim=2)
    sv = (dv.double().sum(dim=2) - dog.double().sum(dim=2)).abs() / dv.double().abs().sum(dim=2)
    say(f"    invariants: max |sum dK| / sum |dK| = {sk.max().item():.2e}, dV: {sv.max().item():.2e}")
    assert sk.max().item() <= 1e-2 and sv.max().item() <= 1e-2
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, 255, 4096, n - 1], rng.integers(0, n, 59)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 4096, n - 1], rng.integers(0, n, 59)]))
    dq_c, dk_c, dv_c = (decode(t.cpu(), "bf16") for t in (dq, dk, dv))
    q, k, v = oracle_inputs(inp)
    g = decode(do, "bf16")
    for hh in (0, 31):
        say(f"    head {hh}")
        ref_dq, _ = oracle.backward_rows(q[0, hh], k[0, hh], v[0, hh], g[0, hh], scale, True, rows)
        lse_h, dsum_h = oracle.head_statistics(q[0, hh], k[0, hh], v[0, hh], g[0, hh], scale, True)
        ref_dk, ref_dv = oracle.backward_key_columns(q[0, hh], k[0, hh], v[0, hh], g[0, hh], scale, True,
                                                     cols, lse_h, dsum_h)
        compare([dq_c[0, hh][rows], dk_c[0, hh][cols], dv_c[0, hh][cols]], [ref_dq, ref_dk, ref_dv],
                "bf16", f"head {hh}")


def test_paired_dq_tiles_without_mask():
    """32 heads, n = 4096, d_k 64, no mask: the dQ pass pairs query tiles
    (32 x 16 / 2 = 256 workgroups); sampled dQ rows and dK / dV key columns of
    two heads against the oracle."""
    b, h, n, d = 1, 32, 4096, 64
    say("backward, paired dQ tiles, no mask")
    inp, do = workload.make_inputs_with_grad(b, h, n, d, "bf16", seed=13)
    scale = float(np.float32(1 / math.sqrt(d)))
    dev = inp.to("cuda")
    o, lse = fa.forward(dev.q, dev.k, dev.v, causal=False, scale=scale)
    dq, dk, dv = fa.backward(dev.q, dev.k, dev.v, o, lse, do.cuda(), causal=False, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, 255, 256, 2047, 2048, n - 1], rng.integers(0, n, 40)]))
    cols = np.unique(np.concatenate([[0, 127, n - 1], rng.integers(0, n, 40)]))
    dq_c, dk_c, dv_c = (decode(t.cpu(), "bf16") for t in (dq, dk, dv))
    q, k, v = oracle_inputs(inp)
    g = decode(do, "bf16")
    for hh in (0, 17):
        ref_dq, _ = oracle.backward_rows(q[0, hh], k[0, hh], v[0, hh], g[0, hh], scale, False, rows)
        lse_h, dsum_h = oracle.head_statistics(q[0, hh], k[0, hh], v[0, hh], g[0, hh], scale, False)
        ref_dk, ref_dv = oracle.backward_key_columns(q[0, hh], k[0, hh], v[0, hh], g[0, hh], scale, False,
                                                     cols, lse_h, dsum_h)
        compare([dq_c[0, hh][rows], dk_c[0, hh][cols], dv_c[0, hh][cols]], [ref_dq, ref_dk, ref_dv],
                "bf16", f"head {hh}")
