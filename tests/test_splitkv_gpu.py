"""GPU parity of the split-KV forward (fa_forward_splitkv).

The merged output is compared with the oracle like the plain forward; each
key block's partial result (O_g, LSE_g in the workspace) is compared with the
oracle's own softmax state over that block's keys alone (oracle.tile_state),
so both the per-block kernels and the log-sum-exp merge are pinned
separately. The block rule (keys per block) is the one include/fa.h states.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_08_amd as fa
import workload
from parity_util import LSE_TOL, O_TOL, oracle_forward, report

pytestmark = pytest.mark.gpu

OUT_FMT = {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8": "bf16"}


def say(*a):
    print(*a, flush=True)


def block_keys(n, splits):
    per = -(-n // splits)
    return 128 * -(-per // 128)


def make(b, h, n, d, dtype, seed):
    """Seeded inputs; e4m3 ones are N(0,1) rounded to e4m3 with descale 1,
    since fa_forward_splitkv takes e4m3 with unit descales."""
    if dtype != "fp8":
        return workload.make_inputs(b, h, n, d, dtype, seed)
    f = workload.make_inputs(b, h, n, d, "f32", seed)
    e = torch.float8_e4m3fn
    return workload.Inputs(f.q.to(e), f.k.to(e), f.v.to(e), "fp8")


def run_split(inp, splits, causal, scale):
    d = inp.to("cuda")
    o, lse, ws = fa.forward_splitkv(d.q, d.k, d.v, splits, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse, ws


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,splits", [(201, 2), (300, 3), (1000, 7), (2048, 64), (130, 256)])
def test_merged_result_matches_oracle(n, splits, causal, dtype):
    b, h, d = 1, 3, (64 if n % 2 else 128)
    say(f"splitkv n={n} splits={splits} causal={causal} dtype={dtype} d={d}")
    inp = make(b, h, n, d, dtype, seed=n + splits)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse, _ = run_split(inp, splits, causal, scale)
    o_ref, lse_ref = oracle_forward(inp, causal, scale)
    r = report(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref, OUT_FMT[dtype])
    say("   ", r)
    assert r["finite"] and r["lse_max"] <= LSE_TOL and r["o_max"] <= O_TOL[dtype], r


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_partials_match_oracle_block_states(dtype, causal):
    b, h, n, d, splits = 2, 2, 700, 64, 4
    say(f"partials dtype={dtype} causal={causal}")
    inp = workload.make_inputs(b, h, n, d, dtype, seed=11)
    scale = float(np.float32(0.125))
    _, _, ws = run_split(inp, splits, causal, scale)
    bk = block_keys(n, splits)
    used = -(-n // bk)
    rows = b * h * n
    o_bytes = used * rows * d * 4
    lse_off = -(-o_bytes // 256) * 256
    wsc = ws.cpu()
    part_o = wsc[:o_bytes].view(torch.float32).reshape(used, b, h, n, d).double().numpy()
    part_l = wsc[lse_off:lse_off + used * rows * 4].view(torch.float32).reshape(used, b, h, n).double().numpy()
    qd = oracle.decode(inp.bits("q"), dtype)
    kd = oracle.decode(inp.bits("k"), dtype)
    vd = oracle.decode(inp.bits("v"), dtype)
    qi = np.arange(n)
    for g in range(used):
        k0, k1 = g * bk, min(n, (g + 1) * bk)
        excl = (np.arange(k0, k1)[None, :] > qi[:, None]) if causal else None
        for bi in range(b):
            for hi in range(h):
                st = oracle.tile_state(qd[bi, hi], kd[bi, hi, k0:k1], vd[bi, hi, k0:k1], scale, excl)
                m, l, o = st
                seen = l > 0
                o_ref = np.zeros_like(o)
                o_ref[seen] = o[seen] / l[seen][:, None]
                lse_ref = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
                go, gl = part_o[g, bi, hi], part_l[g, bi, hi]
                assert np.array_equal(np.isneginf(gl), ~seen), (g, bi, hi)
                assert (go[~seen] == 0).all()
                assert np.abs(gl[seen] - lse_ref[seen]).max(initial=0) <= LSE_TOL
                assert np.abs(go[seen] - o_ref[seen]).max(initial=0) <= O_TOL[dtype]


def test_split_equals_unsplit_within_rounding():
    say("split vs unsplit")
    inp = workload.make_inputs(1, 8, 3000, 128, "bf16", seed=3)
    d = inp.to("cuda")
    o1, l1 = fa.forward(d.q, d.k, d.v, causal=True)
    o2, l2, _ = fa.forward_splitkv(d.q, d.k, d.v, 5, causal=True)
    torch.cuda.synchronize()
    # both are within the bf16 bar of the exact result; they differ by at most
    # a few output roundings
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_one_block_is_the_plain_forward_bitwise():
    say("splits=1")
    inp = workload.make_inputs(1, 8, 500, 128, "bf16", seed=4)
    d = inp.to("cuda")
    o1, l1 = fa.forward(d.q, d.k, d.v, causal=True)
    o2, l2, _ = fa.forward_splitkv(d.q, d.k, d.v, 1, causal=True)
    o3, l3, _ = fa.forward_splitkv(d.q, d.k, d.v, 64, causal=True)   # 500 keys -> 128-key blocks
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isfinite(o3).all()


def test_long_rows_sampled():
    w = workload.Workload("llama_8heads", 1, 8, 8192, 128, "bf16", True)
    rows = workload.sample_rows(w.n, 256, 5)
    say(f"splitkv 8 heads n=8192 causal, {len(rows)} sampled rows")
    inp = workload.workload_inputs(w, 5)
    o, lse, _ = run_split(inp, 4, True, w.scale)
    o_ref, lse_ref = oracle_forward(inp, True, w.scale, rows=rows)
    r = report(o.cpu().double().numpy()[:, :, rows], lse.cpu().double().numpy()[:, :, rows], o_ref,
               lse_ref, "bf16")
    say("   ", r)
    assert r["lse_max"] <= LSE_TOL and r["o_max"] <= O_TOL["bf16"], r


def test_chosen_split_count_on_two_heads():
    """splits=None takes fa_splitkv_splits' count for the device (8 for two
    heads of 4096 keys on 256 compute units); the merged result meets the
    oracle on sampled rows of both heads."""
    b, h, n, d = 1, 2, 4096, 128
    chosen = fa.splitkv_splits(b, h, n, False)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert chosen == fa.splitkv_splits(b, h, n, False, cus)
    say(f"splitkv chosen splits={chosen} on {cus} compute units")
    assert chosen > 1
    inp = workload.make_inputs(b, h, n, d, "bf16", seed=21)
    scale = float(np.float32(1 / math.sqrt(d)))
    dv = inp.to("cuda")
    o, lse, ws = fa.forward_splitkv(dv.q, dv.k, dv.v, None, causal=False, scale=scale)
    torch.cuda.synchronize()
    assert ws.numel() == fa.splitkv_workspace_size(b, h, n, d, chosen)
    rows = workload.sample_rows(n, 256, 21)
    o_ref, lse_ref = oracle_forward(inp, False, scale, rows=rows)
    r = report(o.cpu().double().numpy()[:, :, rows], lse.cpu().double().numpy()[:, :, rows], o_ref,
               lse_ref, "bf16")
    say("   ", r)
    assert r["lse_max"] <= LSE_TOL and r["o_max"] <= O_TOL["bf16"], r
