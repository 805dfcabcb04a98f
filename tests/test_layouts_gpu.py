"""GPU tests of the strided (fa_forward_strided) and ragged-batch
(fa_forward_varlen) layouts.

Both run the forward kernels on the same values in the same order as the
dense fa_forward, only at other addresses, so their outputs must equal the
dense outputs bit for bit; the dense path is itself checked against the
oracle in test_parity_gpu.py, and a few cases here are also compared with the
oracle directly.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_08_amd as fa
import workload
from parity_util import LSE_TOL, O_TOL, oracle_inputs

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def say(*a):
    print(*a, flush=True)


def draw(b, h, n, d, dtype, seed):
    """Seeded [b, h, n, d] inputs; e4m3 ones are N(0,1) rounded to e4m3 (the
    strided and ragged entries take e4m3 with unit descales)."""
    if dtype != "fp8":
        return workload.make_inputs(b, h, n, d, dtype, seed)
    f = workload.make_inputs(b, h, n, d, "f32", seed)
    return workload.Inputs(f.q.to(TD["fp8"]), f.k.to(TD["fp8"]), f.v.to(TD["fp8"]), "fp8")


def same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype == torch.float8_e4m3fn else a,
                       b.view(torch.uint8) if b.dtype == torch.float8_e4m3fn else b)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 64), (65, 128), (300, 64), (1000, 128)])
def test_bshd_equals_dense_bitwise(n, d, causal, dtype):
    b, h = 2, 3
    say(f"bshd n={n} d={d} causal={causal} dtype={dtype}")
    inp = draw(b, h, n, d, dtype, seed=n + d).to("cuda")
    scale = float(np.float32(1 / math.sqrt(d)))
    o1, l1 = fa.forward(inp.q, inp.k, inp.v, causal=causal, scale=scale)
    qs, ks, vs = (t.transpose(1, 2).contiguous() for t in (inp.q, inp.k, inp.v))
    o2, l2 = fa.forward_strided(qs, ks, vs, layout="bshd", causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert tuple(o2.shape) == (b, n, h, d)
    assert same(o1, o2.transpose(1, 2)) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_rows_and_mixed_output_layout(dtype):
    """q, k, v are column slices of wider row buffers (row strides 192, 256 and
    128 + 64), O is written in the [b, n, h, d] layout."""
    b, h, n, d = 2, 4, 333, 128
    inp = draw(b, h, n, d, dtype, seed=9).to("cuda")
    o1, l1 = fa.forward(inp.q, inp.k, inp.v, causal=True)
    wide = []
    for t, w in ((inp.q, 192), (inp.k, 256), (inp.v, 192)):
        big = torch.full((b, h, n, w), float("nan"), dtype=t.dtype, device="cuda")
        big[..., 32:32 + d] = t
        wide.append(big[..., 32:32 + d])
    o2, l2 = fa.forward_strided(*wide, layout="bhsd", out_layout="bshd", causal=True)
    torch.cuda.synchronize()
    assert same(o1, o2.transpose(1, 2)) and torch.equal(l1, l2)


def test_bshd_llama_shape_bitwise():
    b, h, n, d = 1, 32, 8192, 128
    say("bshd llama shape")
    inp = workload.make_inputs(b, h, n, d, "bf16", seed=0).to("cuda")
    o1, l1 = fa.forward(inp.q, inp.k, inp.v, causal=True)
    qs, ks, vs = (t.transpose(1, 2).contiguous() for t in (inp.q, inp.k, inp.v))
    o2, l2 = fa.forward_strided(qs, ks, vs, layout="bshd", causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.transpose(1, 2)) and torch.equal(l1, l2)


def pack(inp, lens):
    """[1, h, total, d] draws -> packed [total, h, d] tensors and cu_seqlens."""
    q, k, v = (t[0].transpose(0, 1).contiguous() for t in (inp.q, inp.k, inp.v))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return q, k, v, cu


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_equals_per_sequence_calls(d, causal, dtype):
    lens = [1, 17, 0, 300, 64, 129, 1000, 2]
    total, h = sum(lens), 3
    say(f"varlen d={d} causal={causal} dtype={dtype} lens={lens}")
    inp = draw(1, h, total, d, dtype, seed=d + 5)
    q, k, v, cu = pack(inp, lens)
    qd, kd, vd, cud = (t.cuda() for t in (q, k, v, cu))
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = fa.forward_varlen(qd, kd, vd, cud, max(lens), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (total, h, d) and tuple(lse.shape) == (h, total)
    for bi, ln in enumerate(lens):
        if ln == 0:
            continue
        s0 = int(cu[bi])
        sl = slice(s0, s0 + ln)
        qs, ks, vs = (t[sl].transpose(0, 1).unsqueeze(0).contiguous() for t in (qd, kd, vd))
        o1, l1 = fa.forward(qs, ks, vs, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert same(o1[0], o[sl].transpose(0, 1)), (bi, ln)
        assert torch.equal(l1[0], lse[:, sl]), (bi, ln)
    # the longest sequence also against the oracle
    s0, ln = int(cu[6]), lens[6]
    one = workload.Inputs(*(t[s0:s0 + ln].transpose(0, 1).unsqueeze(0).contiguous() for t in (q, k, v)), dtype)
    o_ref, l_ref = oracle.attention(*oracle_inputs(one), scale, causal)
    o_g = o[s0:s0 + ln].transpose(0, 1).float().cpu().double().numpy()
    assert np.abs(o_g - o_ref[0]).max() <= O_TOL[dtype]
    assert np.abs(lse[:, s0:s0 + ln].cpu().double().numpy() - l_ref[0]).max() <= LSE_TOL


def test_varlen_length_mix_at_scale():
    """32 heads, d_k 128, bf16, causal; 12 sequences whose lengths follow a
    seeded log-normal mix (16 .. 8192 rows, about 24k rows in all)."""
    rng = np.random.default_rng(7)
    lens = np.clip(np.exp(rng.normal(7.3, 1.0, 12)).astype(int), 16, 8192).tolist()
    total, h, d = int(sum(lens)), 32, 128
    say(f"varlen mix: total {total}, lens {lens}")
    inp = workload.make_inputs(1, h, total, d, "bf16", seed=1)
    q, k, v, cu = pack(inp, lens)
    qd, kd, vd, cud = (t.cuda() for t in (q, k, v, cu))
    o, lse = fa.forward_varlen(qd, kd, vd, cud, max(lens), causal=True)
    torch.cuda.synchronize()
    for bi, ln in enumerate(lens):
        s0 = int(cu[bi])
        sl = slice(s0, s0 + ln)
        qs, ks, vs = (t[sl].transpose(0, 1).unsqueeze(0).contiguous() for t in (qd, kd, vd))
        o1, l1 = fa.forward(qs, ks, vs, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], o[sl].transpose(0, 1)) and torch.equal(l1[0], lse[:, sl]), (bi, ln)


def test_varlen_empty_sequences_around_one():
    h, d = 2, 64
    inp = draw(1, h, 5, d, "bf16", seed=3)
    q, k, v, cu = pack(inp, [0, 0, 5, 0])
    o, lse = fa.forward_varlen(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), 5, causal=True)
    o1, l1 = fa.forward(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[0], o.transpose(0, 1)) and torch.equal(l1[0], lse)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_varlen_equals_per_sequence_calls(d, causal, dtype):
    lens = [1, 17, 0, 300, 64, 129, 700, 2]
    total, h = sum(lens), 3
    say(f"backward varlen d={d} causal={causal} dtype={dtype} lens={lens}")
    inp, do = workload.make_inputs_with_grad(1, h, total, d, dtype, seed=d + 7)
    q, k, v, cu = pack(inp, lens)
    g = do[0].transpose(0, 1).contiguous()
    qd, kd, vd, gd, cud = (t.cuda() for t in (q, k, v, g, cu))
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = fa.forward_varlen(qd, kd, vd, cud, max(lens), causal=causal, scale=scale)
    dq, dk, dv = fa.backward_varlen(qd, kd, vd, o, lse, gd, cud, max(lens), causal=causal, scale=scale)
    torch.cuda.synchronize()
    for bi, ln in enumerate(lens):
        if ln == 0:
            continue
        s0 = int(cu[bi])
        sl = slice(s0, s0 + ln)
        one = [t[sl].transpose(0, 1).unsqueeze(0).contiguous() for t in (qd, kd, vd, o, gd)]
        l1 = lse[:, sl].unsqueeze(0).contiguous()
        r = fa.backward(one[0], one[1], one[2], one[3], l1, one[4], causal=causal, scale=scale)
        torch.cuda.synchronize()
        for name, a_, b_ in zip(("dq", "dk", "dv"), r, (dq, dk, dv)):
            assert torch.equal(a_[0], b_[sl].transpose(0, 1)), (bi, ln, name)
    # the longest sequence against the gradient oracle (bar of test_backward_gpu)
    s0, ln = int(cu[6]), lens[6]
    sl = slice(s0, s0 + ln)
    dec = lambda t: oracle.decode(t.cpu().contiguous().view(torch.int16).numpy().view("uint16"), dtype)
    qs, ks, vs, gs = (dec(t[sl].transpose(0, 1).unsqueeze(0)) for t in (qd, kd, vd, gd))
    ref = oracle.attention_backward(qs, ks, vs, gs, scale, causal)
    tol = {"bf16": 1e-2, "f16": 2e-3}[dtype]
    for name, gt, rf in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        got = dec(gt[sl].transpose(0, 1).unsqueeze(0))
        assert np.abs(got - rf).max() <= tol * max(np.abs(rf).max(), 1e-3), name
