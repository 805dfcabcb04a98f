"""The entry points under HIP graph capture: fa_forward and
fa_forward_splitkv allocate nothing and only enqueue kernels on the caller's
stream, so a captured call replays. Each replay runs after eager work that
overwrites the outputs, and must reproduce the eager result bit for bit."""
import pytest
import torch

import transformer_attention_08_amd as fa
import workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the graph (kernel code objects loaded)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("causal", [False, True])
def test_forward_replays(causal):
    say(f"graph replay, fa_forward causal={causal}")
    d = workload.make_inputs(1, 8, 1000, 128, "bf16", seed=31).to("cuda")
    o_ref, lse_ref = fa.forward(d.q, d.k, d.v, causal=causal)
    out, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    g = _capture(lambda: fa.forward(d.q, d.k, d.v, causal=causal, out=out, lse=lse))
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(lse, lse_ref), rep


@pytest.mark.parametrize("heads,n,causal", [(32, 8192, True), (12, 16500, False)])
def test_384_row_kernels_replay(heads, n, causal):
    """The 384-row kernels: the packed causal launch (its host-built plan of
    tile groups travels in the captured kernel arguments) and one workgroup
    per tile."""
    say(f"graph replay, fa_forward [1, {heads}, {n}, 128] causal={causal}")
    d = workload.make_inputs(1, heads, n, 128, "bf16", seed=33).to("cuda")
    o_ref, lse_ref = fa.forward(d.q, d.k, d.v, causal=causal)
    out, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    q2, k2, v2 = (x[:, :, :6000].contiguous() for x in (d.q, d.k, d.v))
    g = _capture(lambda: fa.forward(d.q, d.k, d.v, causal=causal, out=out, lse=lse))
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        # eager work between replays: a call of another shape (another plan)
        fa.forward(q2, k2, v2, causal=True)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(lse, lse_ref), rep


def test_splitkv_replays():
    say("graph replay, fa_forward_splitkv (blocks + merge)")
    d = workload.make_inputs(1, 2, 2048, 128, "bf16", seed=32).to("cuda")
    splits = 4
    o_ref, lse_ref, _ = fa.forward_splitkv(d.q, d.k, d.v, splits)
    out, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    ws = torch.empty(fa.splitkv_workspace_size(1, 2, 2048, 128, splits), dtype=torch.uint8, device="cuda")
    g = _capture(lambda: fa.forward_splitkv(d.q, d.k, d.v, splits, out=out, lse=lse, workspace=ws))
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(lse, lse_ref), rep
