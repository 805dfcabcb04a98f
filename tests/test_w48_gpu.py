"""GPU parity of the 384-row forward kernels (fwd_w48, fwd_w48_packed)
against the fp64 oracle.

fa_forward runs f16 / bf16 heads of d_k 128 on 48-row-per-wave kernels when
there are two or more 384-row tiles per compute unit (heads x tiles >= 512
on a 256-CU device): causal heads of 6144 <= n < 16384 with the tiles packed
into groups of near-equal length (one workgroup per group; with a multiple
of 8 heads, each workgroup may take two or more heads in turn), heads of
n >= 16384 with one workgroup per tile, and heads without the mask from
6144 rows with one workgroup per tile where that grid fills its rounds of
workgroups nearly as well as the 256-row kernel's. Tiles are laid out from the last row back, so a ragged n leaves a
partial first tile whose missing rows lie before row 0, and the softmax
takes no chunk max unless a lane's sum of p passes 2^64 (bf16) or 2^15
(f16). The shapes below take each path; rows are a seeded sample (the first
and last rows of every head plus random ones), computed by the oracle row by
row.
"""
import math

import numpy as np
import pytest
import torch

import workload
from parity_util import O_TOL, LSE_TOL, gpu_forward, oracle_forward, report

pytestmark = pytest.mark.gpu

OUT_FMT = {"f16": "f16", "bf16": "bf16"}
D = 128
SCALE = float(np.float32(1 / math.sqrt(D)))


def say(*a):
    print(*a, flush=True)


def check_rows(inp, causal, rows):
    o, lse = gpu_forward(inp, causal, SCALE)
    o, lse = o[:, :, rows], lse[:, :, rows]
    o_ref, lse_ref = oracle_forward(inp, causal, SCALE, rows=rows)
    r = report(o, lse, o_ref, lse_ref, OUT_FMT[inp.dtype])
    say("   ", r)
    assert r["finite"]
    assert r["lse_max"] <= LSE_TOL, r
    assert r["o_max"] <= O_TOL[inp.dtype], r


def _dev(t):
    return t.to("cuda")


@pytest.mark.parametrize("dtype,causal,heads,n", [
    ("bf16", True, 12, 16384),    # one workgroup per tile; 43 tiles, the first holds 256 rows
    ("bf16", False, 12, 16500),   # one workgroup per tile; first tile holds 372 rows
    ("f16", True, 12, 17000),     # one workgroup per tile; first tile holds 104 rows
    ("f16", False, 10, 20000),    # one workgroup per tile, 53 tiles x 10 heads
    ("bf16", True, 32, 16384),    # one workgroup per tile, heads one at a time per XCD
    ("f16", True, 12, 16200),     # packed, 21 groups per head (12 heads: no XCD grouping); first tile 72 rows
    ("f16", True, 32, 8192),      # packed, 8 groups per head, one head per workgroup
    ("bf16", True, 64, 8200),     # packed, 8 groups per head, two heads in turn; first tile 136 rows
    ("bf16", True, 32, 6144),     # packed, 16 full tiles in 8 groups of two
    ("f16", True, 32, 7000),      # packed, 19 tiles; first tile holds 88 rows
    ("bf16", False, 32, 6144),    # no mask, one workgroup per tile (512 = two full rounds)
    ("f16", False, 32, 12000),    # no mask, one workgroup per tile; first tile holds 96 rows
])
def test_w48_sampled_rows(dtype, causal, heads, n):
    say(f"w48 [1, {heads}, {n}, {D}] {dtype} causal={causal}")
    inp = workload.make_inputs(1, heads, n, D, dtype, seed=n + heads)
    rows = workload.sample_rows(n, 768, seed=n)
    check_rows(inp, causal, rows)


def growing_scores(heads, n, dtype, seed, rise=120.0):
    """Q and K whose scores rise along the keys by about `rise` (natural-log
    units) from key 0 to key n - 1, with N(0, 1) noise on every element: each
    later 32-key chunk outscores the reference the first chunk set, so lane
    sums of p pass the bound several times per row (every ~44 units in bf16,
    ~10 in f16) and the chunk takes its true max."""
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(D, generator=g, dtype=torch.float64)
    u = u / u.norm()
    c = 8.0
    t = torch.arange(n, dtype=torch.float64) * (rise / (SCALE * c) / n)
    q = c * u + torch.randn(1, heads, n, D, generator=g, dtype=torch.float64)
    k = t[:, None] * u + torch.randn(1, heads, n, D, generator=g, dtype=torch.float64)
    v = torch.randn(1, heads, n, D, generator=g, dtype=torch.float64)
    td = workload.torch_dtype(dtype)
    return workload.Inputs(q.to(td), k.to(td), v.to(td), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal,n", [(True, 16500), (False, 16500), (True, 16200)])
def test_w48_growing_scores(dtype, causal, n):
    heads = 12
    say(f"w48 growing scores [1, {heads}, {n}, {D}] {dtype} causal={causal}")
    inp = growing_scores(heads, n, dtype, seed=21)
    rows = workload.sample_rows(n, 512, seed=21)
    check_rows(inp, causal, rows)


@pytest.mark.parametrize("heads,n,causal", [
    (12, 16500, True),   # one workgroup per tile
    (12, 16200, True),   # packed
    (32, 6144, False),   # no mask, one workgroup per tile
])
def test_w48_strided_is_bitwise_dense(heads, n, causal):
    """[batch, n, heads, d_k] inputs and output give bitwise the dense result."""
    import transformer_attention_08_amd as fa
    say(f"w48 strided [1, {n}, {heads}, {D}] bf16 causal={causal}")
    inp = workload.make_inputs(1, heads, n, D, "bf16", seed=31)
    q, k, v = _dev(inp.q), _dev(inp.k), _dev(inp.v)
    o1, l1 = fa.forward(q, k, v, causal=causal)
    qs, ks, vs = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    o2, l2 = fa.forward_strided(qs, ks, vs, layout="bshd", causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.transpose(1, 2)) and torch.equal(l1, l2)


@pytest.mark.parametrize("n", [17000, 16200])
def test_w48_deterministic_and_lse_null(n):
    import transformer_attention_08_amd as fa
    heads = 12
    say(f"w48 determinism, lse null [1, {heads}, {n}, {D}] f16 causal")
    inp = workload.make_inputs(1, heads, n, D, "f16", seed=32)
    q, k, v = _dev(inp.q), _dev(inp.k), _dev(inp.v)
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True)
    o3, l3 = fa.forward(q, k, v, causal=True, want_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert l3 is None and torch.equal(o1, o3)


@pytest.mark.parametrize("n", [16500, 16200])
def test_w48_writes_only_rows_of_the_heads(n):
    """The partial first tile's missing rows (before row 0) and the rows past
    n are never written: sentinels on both sides of O and LSE survive."""
    import transformer_attention_08_amd as fa
    heads = 12
    say(f"w48 no write outside [1, {heads}, {n}, {D}] bf16 causal")
    inp = workload.make_inputs(1, heads, n, D, "bf16", seed=33)
    pad = 384 * D
    size = heads * n * D
    big = torch.full((pad + size + pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    o = big[pad: pad + size].view(1, heads, n, D)
    lbig = torch.full((384 + heads * n + 384,), 7.0, dtype=torch.float32, device="cuda")
    lse = lbig[384: 384 + heads * n].view(1, heads, n)
    fa.forward(_dev(inp.q), _dev(inp.k), _dev(inp.v), causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert (big[:pad] == 7.0).all() and (big[pad + size:] == 7.0).all()
    assert (lbig[:384] == 7.0).all() and (lbig[384 + heads * n:] == 7.0).all()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
