"""fa_forward_splitkv_noalloc: the split-KV forward for callers that cannot
allocate, with its partials in the library's fixed per-GPU scratch array.

Called through the C ABI (ctypes, no binding logic in between) and compared
with fa_forward_splitkv on a caller workspace: the same kernels on the same
block count, so the results must be equal bit for bit -- on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
partials; nothing in it may leak into the second result). Sizes beyond the
scratch are refused before any launch. The first call on a device loads the
code object holding the array (the runtime reserves its 128 MiB then, for
the rest of the process); every call after that allocates no device memory.
"""
import math

import numpy as np
import pytest
import torch

import transformer_attention_08_amd as fa
import workload
from parity_util import LSE_TOL, O_TOL, oracle_forward, report

pytestmark = pytest.mark.gpu

OUT_FMT = {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8": "bf16"}


def say(*a):
    print(*a, flush=True)


def c_noalloc(lib, q, k, v, o, lse, causal, scale, splits):
    b, h, n, d = q.shape
    return lib.fa_forward_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                          lse.data_ptr(), b, h, n, d, scale, 1 if causal else 0,
                                          fa._DTYPE_CODE[q.dtype], splits,
                                          torch.cuda.current_stream().cuda_stream)


def c_workspace(lib, q, k, v, o, lse, causal, scale, splits):
    b, h, n, d = q.shape
    need = fa.splitkv_workspace_size(b, h, n, d, splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    st = lib.fa_forward_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                b, h, n, d, scale, 1 if causal else 0, fa._DTYPE_CODE[q.dtype], splits,
                                ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    return st, ws


_WARM = []


def warm_up(lib):
    """The first call on a device loads the code object that holds the
    scratch array (the runtime then reserves its 128 MiB, held until the
    process ends) and looks up its address; after that no call allocates."""
    if _WARM:
        return
    q = torch.zeros(1, 1, 512, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = torch.empty_like(q), torch.empty(1, 1, 512, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    assert c_noalloc(lib, q, q, q, o, lse, False, 0.125, 2) == 0
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    say(f"    first call on the device: {(free0 - free1) / 2**20:.1f} MiB reserved")
    assert free0 - free1 <= fa.noalloc_scratch_bytes() + (4 << 20)
    _WARM.append(True)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_equals_workspace_entry_on_two_calls(dtype, causal):
    lib = fa.load_library()
    warm_up(lib)
    # first a larger call, then a smaller one (fewer heads, shorter rows, other block count)
    for (b, h, n, d, splits, seed) in ((1, 4, 2000, 128, 8, 71), (1, 2, 700, 64, 3, 72)):
        say(f"no-alloc split-KV [{b}, {h}, {n}, {d}] {dtype} causal={causal} splits={splits}")
        inp = workload.make_inputs(b, h, n, d, dtype, seed=seed)
        dev = inp.to("cuda")
        scale = float(np.float32(1 / math.sqrt(d)))
        o_ref = torch.empty(b, h, n, d, dtype=dev.q.dtype, device="cuda")
        l_ref = torch.empty(b, h, n, dtype=torch.float32, device="cuda")
        st, ws = c_workspace(lib, dev.q, dev.k, dev.v, o_ref, l_ref, causal, scale, splits)
        assert st == 0
        o = torch.full_like(o_ref, 7.0)
        lse = torch.full_like(l_ref, 7.0)
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        st = c_noalloc(lib, dev.q, dev.k, dev.v, o, lse, causal, scale, splits)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        assert st == 0, (st, lib.fa_last_hip_error())
        assert free0 == free1, (free0, free1)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        # and the oracle's bars, as for the workspace entry
        o_or, l_or = oracle_forward(inp, causal, scale)
        r = report(o.cpu().double().numpy(), lse.cpu().double().numpy(), o_or, l_or, OUT_FMT[dtype])
        say("   ", r)
        assert r["finite"] and r["lse_max"] <= LSE_TOL and r["o_resid"] <= O_TOL[dtype], r


def test_noalloc_refuses_partials_beyond_its_scratch():
    lib = fa.load_library()
    warm_up(lib)
    cap = int(lib.fa_noalloc_scratch_bytes())
    assert cap == fa.noalloc_scratch_bytes() == 128 << 20
    b, h, n, d = 1, 32, 8192, 128
    # 2 blocks of the Llama shape need 2 * 262144 rows * 516 bytes > 128 MiB
    assert fa.splitkv_workspace_size(b, h, n, d, 2) > cap
    q = torch.zeros(b, h, n, d, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((b, h, n), 7.0, dtype=torch.float32, device="cuda")
    st = c_noalloc(lib, q, q, q, o, lse, True, 0.0884, 2)
    torch.cuda.synchronize()
    assert st == 10  # FA_ERR_SCRATCH, before any launch: nothing written
    assert (o == 7.0).all() and (lse == 7.0).all()
    # one block needs no scratch at all: the plain forward
    st = c_noalloc(lib, q[:, :2, :100], q[:, :2, :100], q[:, :2, :100], o[:, :2, :100].contiguous(),
                   lse[:, :2, :100].contiguous(), True, 0.0884, 1)
    assert st == 0


def test_noalloc_through_the_binding():
    # the binding with caller-given outputs; another call after the ones above
    inp = workload.make_inputs(1, 2, 4096, 128, "bf16", seed=73)
    dev = inp.to("cuda")
    o = torch.empty_like(dev.q)
    lse = torch.empty(1, 2, 4096, dtype=torch.float32, device="cuda")
    splits = fa.splitkv_splits(1, 2, 4096, False)
    say(f"binding: two heads of 4096, {splits} blocks")
    assert fa.splitkv_workspace_size(1, 2, 4096, 128, splits) <= fa.noalloc_scratch_bytes()
    fa.forward_splitkv_noalloc(dev.q, dev.k, dev.v, splits, causal=False, out=o, lse=lse)
    o2, l2, _ = fa.forward_splitkv(dev.q, dev.k, dev.v, splits, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
