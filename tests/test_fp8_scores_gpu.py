"""Why the e4m3 forward widens Q and K to bf16 instead of using the fp8 MFMA.

The e4m3 workload ([1, 32, 8192, 128], no mask, Q and K drawn N(0,1) x 4,
per-tensor descales) has scaled scores up to about 100, so a relative error
of the raw scores of a few 1e-5 moves the log-sum-exp by more than its 1e-3
bar. This test computes the raw scores S = Q8 K8^T of sampled rows of two
heads with both matrix paths (libfa_probe.so: v_mfma_f32_32x32x16_fp8_fp8 on
the codes, and v_mfma_f32_32x32x16_bf16 on the codes widened exactly to
bf16), forms the LSE of each in float64 on the host, and compares it with
the oracle's LSE of the same rows. The bf16 path meets the bar with a wide
margin; the fp8 path does not. If the fp8 path ever met it, the choice made
in the e4m3 kernel should be revisited.
"""
import ctypes

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
import workload
from parity_util import LSE_TOL

pytestmark = pytest.mark.gpu

ROWS = 512


def say(*a):
    print(*a, flush=True)


def test_fp8_mfma_scores_miss_the_lse_bar_bf16_scores_meet_it():
    from transformer_attention_08_amd import build as _b

    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.fa_probe_fp8_scores.restype = ctypes.c_int
    lib.fa_probe_fp8_scores.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    w = workload.WORKLOADS["fp8_e4m3_nomask"]
    inp = workload.workload_inputs(w, seed=0)
    c = float(w.scale) * inp.q_descale * inp.k_descale  # raw score -> scaled score
    rows = np.arange(ROWS)
    worst = {"fp8": 0.0, "bf16": 0.0, "s_rel_fp8": 0.0, "s_rel_bf16": 0.0}
    for h in (0, 13):
        q8 = inp.q[0, h].contiguous().cuda()
        k8 = inp.k[0, h].contiguous().cuda()
        out8 = torch.empty(ROWS, w.n, dtype=torch.float32, device="cuda")
        out16 = torch.empty_like(out8)
        rc = lib.fa_probe_fp8_scores(q8.data_ptr(), k8.data_ptr(), w.n, ROWS, out8.data_ptr(), out16.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        s8 = out8.double().cpu().numpy()
        s16 = out16.double().cpu().numpy()
        qd = oracle.decode(inp.bits("q")[0:1, h:h + 1], "fp8", 1.0)[0, 0]
        kd = oracle.decode(inp.bits("k")[0:1, h:h + 1], "fp8", 1.0)[0, 0]
        exact = qd[:ROWS] @ kd.T  # raw scores of the codes, exact in float64
        vd = oracle.decode(inp.bits("v")[0:1, h:h + 1], "fp8", inp.v_descale)
        _, lse_ref = oracle.attention(oracle.decode(inp.bits("q")[0:1, h:h + 1], "fp8", inp.q_descale),
                                      oracle.decode(inp.bits("k")[0:1, h:h + 1], "fp8", inp.k_descale),
                                      vd, w.scale, False, rows=rows)
        lse_ref = lse_ref[0, 0]
        for tag, s in (("fp8", s8), ("bf16", s16)):
            err = float(np.abs(logsumexp(c * s, axis=1) - lse_ref).max())
            rel = float((np.abs(s - exact) / np.maximum(np.abs(exact), 1.0)).max())
            worst[tag] = max(worst[tag], err)
            worst["s_rel_" + tag] = max(worst["s_rel_" + tag], rel)
        say(f"    head {h}: max scaled score {float(np.abs(c * exact).max()):.1f}")
    say("   ", {k: f"{v:.3e}" for k, v in worst.items()})
    assert worst["bf16"] <= LSE_TOL / 10, worst
    assert worst["fp8"] > LSE_TOL, worst
