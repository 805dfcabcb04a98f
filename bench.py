"""Throughput of the fused attention forward pass on one MI355X.

One step = one fa_forward call over the whole workload: the Llama-3-8B layer
shape (batch 1, 32 heads, n = 8192, d_k = 128, bf16, causal) by default.
Inputs are seeded synthetic N(0,1) tensors, resident in HBM before timing.
FLOPs follow the two-GEMM count 4*b*h*n^2*d_k, halved for a causal mask.

Prints one JSON line with the throughput, the roofline position of the
kernel (achieved TFLOP/s against the dense MFMA peak of its dtype, plus the
HBM traffic measured by rocprofv3 counters when the stored measurement
belongs to the current kernel source) and the CPU oracle timed on a bounded
sample of the same workload on this host's cores. A second pass times ten
calls one by one with 512 MiB of other device memory read before each, so
that no input is served from the L2s or the 256 MB Infinity Cache
(`cold_cache`).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--n N] [--splits S] [--no-cpu-baseline] [--no-cold-cache]
    python bench.py --backward      # fa_backward on the workload
    python bench.py --unfused       # the unfused contrast (S, P in memory)
    python bench.py --layout bshd   # [batch, n, heads, d_k] inputs (fa_forward_strided)
    python bench.py --varlen 16     # a ragged batch of 16 sequences (fa_forward_varlen)
    python bench.py --copy-calibration      # plain copy of known size (counter scale)
    python bench.py --traffic-record F W CF CW   # the stored HBM traffic record from counter files
    python bench.py --mfma-rate             # issue rate of the 32x32x16 and 16x16x32 MFMAs
    python bench.py --lds-rate              # LDS read bandwidth (16-byte and transposing reads)
    python bench.py --coissue               # MFMA beside vector work, with register or LDS operands
    python bench.py --valu-rate             # vector ALU rates: exp, fma, add, pack, max3, alone and paired
    python bench.py --copy-rate             # global -> LDS copies, straight or through registers
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % of bf16 MFMA peak (h32, n8192, d_k128, causal)"
# Dense MFMA peaks of MI355X, TFLOP/s (256 CUs x FLOP/clk/CU x 2.4 GHz; the
# published 2.5 PFLOP/s bf16/fp16, 5.0 fp8 and 157.3 fp32 figures).
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
# the kernel each input type runs on
KERNEL_OF_DTYPE = {"bf16": "fwd_direct", "f16": "fwd_direct", "fp8": "fwd_direct8", "f32": "fwd_mfma32"}
# f16 / bf16 heads of d_k 128 run on the 384-row kernels (unsplit, dense
# batches, two or more 384-row tiles per CU): causal heads of W48_PACK_MIN_N
# <= n < W48_MIN_N on fwd_w48_packed (while every head gets two or more
# workgroups), heads of n >= W48_MIN_N on fwd_w48, and heads without the mask
# from W48_PACK_MIN_N rows on fwd_w48 where its grid fills its rounds at
# least 91% as well as fwd_direct's; the same rule as the forward dispatch in
# fa_fwd.hip
W48_PACK_MIN_N, W48_MIN_N, W48_ROWS = 6144, 16384, 384


def fwd_kernel(w, split: bool, ragged: bool = False) -> str:
    """Name of the forward kernel fa_forward launches for workload w."""
    if w.dtype in ("bf16", "f16") and w.d_k == 128 and not split and not ragged:
        import torch
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        bh, tiles = w.batch * w.heads, -(-w.n // W48_ROWS)
        if bh * tiles >= 2 * cus:
            if (w.causal and W48_PACK_MIN_N <= w.n < W48_MIN_N and tiles <= 255
                    and 2 <= cus // bh <= 255):
                return "fwd_w48_packed"
            if w.n >= W48_MIN_N:
                return "fwd_w48"
            if not w.causal and w.n >= W48_PACK_MIN_N:
                dt = -(-w.n // 256)
                dpair = dt % 2 == 0 and bh * (dt // 2) >= cus
                wd, w48 = bh * (dt // 2 if dpair else dt), bh * tiles
                if 100 * w48 * -(-wd // cus) >= 91 * wd * -(-w48 // cus):
                    return "fwd_w48"
    return KERNEL_OF_DTYPE[w.dtype]
# the files the forward kernels and their launch shape are compiled from; a
# stored traffic measurement is valid only for the sources it was taken on
KERNEL_SOURCES = ("transformer_attention_08_amd/csrc/fa_fwd.hip",
                  "transformer_attention_08_amd/csrc/fa_device.h",
                  "transformer_attention_08_amd/csrc/fa_kernels.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama3_8b_bf16_causal.json")


def algorithmic_flops(w) -> float:
    """The two GEMMs, 2*n*n*d_k FLOP each per head; halved under a causal mask."""
    f = 4.0 * w.batch * w.heads * w.n * w.n * w.d_k
    return f / 2 if w.causal else f


def min_hbm_bytes(w) -> int:
    """Read Q, K, V once; write O and the fp32 LSE once."""
    elt = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
    rows = w.batch * w.heads * w.n
    return rows * w.d_k * (3 * elt[w.dtype] + elt[w.out_dtype]) + 4 * rows


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload_name: str):
    """HBM bytes per launch from the committed counter summary, if current."""
    if workload_name != "llama3_8b_bf16_causal" or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def host_threads():
    """(cores this process may run on, threads of the BLAS that NumPy calls)."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
                   or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return cores, int(blas)


def cpu_baseline(w, inp, budget_s: float = 15.0):
    """The fp64 oracle on whole heads of the same inputs, as many heads as fit
    the time budget (at least one); TFLOP/s under the same FLOP count."""
    import numpy as np

    import oracle

    cores, blas = host_threads()
    qb, kb, vb = inp.bits("q"), inp.bits("k"), inp.bits("v")
    done, elapsed = 0, 0.0
    while done < w.heads * w.batch:
        bi, hi = divmod(done, w.heads)
        q = oracle.decode(qb[bi:bi + 1, hi:hi + 1], w.dtype, inp.q_descale)
        k = oracle.decode(kb[bi:bi + 1, hi:hi + 1], w.dtype, inp.k_descale)
        v = oracle.decode(vb[bi:bi + 1, hi:hi + 1], w.dtype, inp.v_descale)
        t0 = time.perf_counter()
        oracle.attention(q, k, v, w.scale, w.causal)
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed >= budget_s or elapsed / done * (done + 1) > 2 * budget_s:
            break
    fl = 4.0 * done * w.n * w.n * w.d_k / (2 if w.causal else 1)
    return {"value": fl / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"{done} of {w.batch * w.heads} heads, all {w.n} rows each, fp64 NumPy, "
                      f"{elapsed:.1f} s; the products run on {blas} BLAS threads, the exponentials "
                      f"(NumPy exp) on one thread, heads one after another"}


def cpu_baseline_backward(w, inp, do, budget_s: float = 15.0):
    """The fp64 gradient oracle on whole heads of the same inputs (S, P, dP, dS
    materialised), as many heads as fit the time budget (at least one);
    TFLOP/s under the backward FLOP count."""
    import oracle

    cores, blas = host_threads()
    qb, kb, vb = inp.bits("q"), inp.bits("k"), inp.bits("v")
    gb = do.contiguous().view(__import__("torch").int16).numpy().view("uint16")
    done, elapsed = 0, 0.0
    while done < w.heads * w.batch:
        bi, hi = divmod(done, w.heads)
        q, k, v, g = (oracle.decode(x[bi:bi + 1, hi:hi + 1], w.dtype) for x in (qb, kb, vb, gb))
        t0 = time.perf_counter()
        oracle.attention_backward(q, k, v, g, w.scale, w.causal)
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed >= budget_s or elapsed / done * (done + 1) > 2 * budget_s:
            break
    fl = 10.0 * done * w.n * w.n * w.d_k / (2 if w.causal else 1)
    return {"value": fl / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"{done} of {w.batch * w.heads} heads, all {w.n} rows each, fp64 NumPy "
                      f"(S, P, dP, dS materialised), {elapsed:.1f} s; the products run on {blas} BLAS "
                      f"threads, the exponentials on one thread"}


def traffic_record(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out=TRAFFIC_FILE):
    """Write the HBM traffic record of the forward at the Llama shape from four
    rocprofv3 counter files: FETCH_SIZE and WRITE_SIZE of `bench.py --steps 3
    --warmup 1 --no-cpu-baseline --no-cold-cache`, and the same two counters
    of `bench.py --copy-calibration` (a 1 GiB device copy), which scale the
    counters' KiB to bytes. The record carries the hash of the kernel sources
    it was taken on; bench.py reports it only while the hash matches."""
    import csv

    def vals(path, kern):
        rows = list(csv.DictReader(open(path)))
        v = [float(r["Counter_Value"]) for r in rows if kern in r["Kernel_Name"]]
        if not v:
            raise RuntimeError(f"no {kern} dispatch in {path}")
        return v

    # the forward kernel the counted run launched (one name across the file)
    names = {r["Kernel_Name"] for r in csv.DictReader(open(fetch_csv)) if "::fwd_" in r["Kernel_Name"]}
    if len(names) != 1:
        raise RuntimeError(f"expected one forward kernel in {fetch_csv}, found {sorted(names)}")
    kname = re.search(r"::(fwd_\w+)<", names.pop()).group(1)
    fv, wv = vals(fetch_csv, f"::{kname}<"), vals(write_csv, f"::{kname}<")
    cfv, cwv = vals(copy_fetch_csv, "copyBuffer"), vals(copy_write_csv, "copyBuffer")
    fetch, write = sum(fv) / len(fv), sum(wv) / len(wv)
    cfk, cwk = sum(cfv) / len(cfv), sum(cwv) / len(cwv)
    nb = 1 << 30
    rf, wf = nb / (cfk * 1024), nb / (cwk * 1024)
    rd, wr = fetch * 1024 * rf, write * 1024 * wf
    import workload
    mn = min_hbm_bytes(workload.WORKLOADS["llama3_8b_bf16_causal"])
    bench_cmd = "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-cold-cache"
    t = {
        "kernel": f"{kname}<bf16, d_k 128, causal>",
        "workload": "llama3_8b_bf16_causal [1, 32, 8192, 128]",
        "kernel_source_hash": kernel_source_hash(),
        "kernel_sources": list(KERNEL_SOURCES),
        "fetch_size_kib_per_dispatch": round(fetch, 1),
        "write_size_kib_per_dispatch": round(write, 1),
        "dispatches_counted": len(fv),
        "copy_calibration": {"bytes_read": nb, "bytes_written": nb, "fetch_size_kib": round(cfk, 4),
                             "write_size_kib": round(cwk, 4), "read_factor": rf, "write_factor": wf},
        "hbm_read_bytes_per_launch": int(rd), "hbm_write_bytes_per_launch": int(wr),
        "hbm_bytes_per_launch": int(rd + wr), "min_hbm_bytes": mn, "ratio_to_min": round((rd + wr) / mn, 2),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o pmc -- {bench_cmd}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o pmc -- {bench_cmd}",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o pmc -- python3 bench.py --copy-calibration",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o pmc -- python3 bench.py --copy-calibration",
            "python3 bench.py --traffic-record <the four pmc_counter_collection.csv files, in that order>"],
    }
    with open(out, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    print(json.dumps({"traffic_record": out, "hbm_bytes_per_launch": t["hbm_bytes_per_launch"],
                      "ratio_to_min": t["ratio_to_min"]}))


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch

    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


MFMA_KINDS = ((0, "v_mfma_f32_32x32x16_bf16", 32 * 32 * 16 * 2),
              (1, "v_mfma_f32_16x16x32_bf16", 16 * 16 * 32 * 2),
              (2, "v_mfma_f32_32x32x16_f16", 32 * 32 * 16 * 2),
              (3, "v_mfma_f32_16x16x32_f16", 16 * 16 * 32 * 2))


def mfma_rate(iters: int = 2000, blocks: int = 256):
    """Issue rate of the 16-bit MFMAs with independent accumulators (the
    libfa_probe.so kernel: one workgroup per CU, 1 or 2 waves per SIMD, no
    memory traffic in the timed loop). One JSON line per variant: shader
    cycles per MFMA on a SIMD, FLOP per cycle per SIMD (1024 at the dense
    peak), and the shader clock from the wave's own cycle and 100 MHz
    counters."""
    import ctypes

    import torch

    from transformer_attention_08_amd import build as _b

    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.fa_probe_mfma_rate.restype = ctypes.c_int
    lib.fa_probe_mfma_rate.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3
    dev = torch.device("cuda:0")
    sink = torch.zeros(512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for kind, name, flop in MFMA_KINDS:
        for wps in (1, 2):
            for nacc in (1, 2, 4, 8):
                out = torch.zeros(2 * blocks * 4 * wps, dtype=torch.int64, device=dev)
                for _ in range(2):  # the first launch warms the clock
                    rc = lib.fa_probe_mfma_rate(kind, nacc, wps, blocks, iters, out.data_ptr(),
                                                sink.data_ptr(), stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"probe launch failed: hipError {rc}")
                    torch.cuda.synchronize(dev)
                cyc = out[0::2].double().cpu().view(blocks, 4 * wps)
                ticks = out[1::2].double().cpu().view(blocks, 4 * wps)
                per_wave = 4 * nacc * iters
                # a SIMD runs wps waves side by side: the workgroup's longest
                # wave over the MFMAs one SIMD issues
                c_simd = float(cyc.max(dim=1).values.median()) / (wps * per_wave)
                ghz = float((cyc / (ticks / 100e6)).median()) / 1e9
                print(json.dumps({"probe": "mfma_rate", "instruction": name, "waves_per_simd": wps,
                                  "accumulators": nacc, "cycles_per_mfma_per_simd": round(c_simd, 2),
                                  "flop_per_clk_per_simd": round(flop / c_simd, 1),
                                  "shader_ghz": round(ghz, 3)}), flush=True)


def lds_rate(iters: int = 4000, blocks: int = 256):
    """LDS read bandwidth per CU (the libfa_probe.so kernel: one workgroup per
    CU, 4 or 8 waves each issuing rounds of 8 independent reads) for
    ds_read_b128 and the transposing ds_read_b64_tr_b16. One JSON line per
    variant: bytes per shader cycle per CU, and the shader clock."""
    import ctypes

    import torch

    from transformer_attention_08_amd import build as _b

    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.fa_probe_lds_rate.restype = ctypes.c_int
    lib.fa_probe_lds_rate.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for mode, name, per_read in ((0, "ds_read_b128", 16 * 64), (1, "ds_read_b64_tr_b16", 8 * 64)):
        for waves in (4, 8):
            out = torch.zeros(2 * blocks * waves, dtype=torch.int64, device=dev)
            for _ in range(2):
                rc = lib.fa_probe_lds_rate(mode, waves, blocks, iters, out.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"probe launch failed: hipError {rc}")
                torch.cuda.synchronize(dev)
            cyc = out[0::2].double().cpu().view(blocks, waves)
            ticks = out[1::2].double().cpu().view(blocks, waves)
            c_block = float(cyc.max(dim=1).values.median())
            ghz = float((cyc / (ticks / 100e6)).median()) / 1e9
            print(json.dumps({"probe": "lds_rate", "instruction": name, "waves_per_cu": waves,
                              "bytes_per_clk_per_cu": round(waves * 8 * iters * per_read / c_block, 1),
                              "shader_ghz": round(ghz, 3)}), flush=True)


def coissue(iters: int = 400, blocks: int = 256):
    """MFMA / vector co-issue (the libfa_probe.so kernel): per CU, four waves
    issue 32x32x16 MFMAs (operands from registers, from 16-byte LDS reads or
    from transposing LDS reads) beside four waves running a softmax-like
    vector stream, each pair on one SIMD; each alone and both together. One
    JSON line per variant: shader cycles per MFMA of the matrix waves and per
    64-score softmax of the vector waves."""
    import ctypes

    import torch

    from transformer_attention_08_amd import build as _b

    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.fa_probe_coissue.restype = ctypes.c_int
    lib.fa_probe_coissue.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    dev = torch.device("cuda:0")
    sink = torch.zeros(512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    names = {0: "registers", 1: "ds_read_b128", 2: "2x ds_read_b64_tr_b16"}
    for opnd in (0, 1, 2):
        row = {"probe": "coissue", "mfma_operands": names[opnd]}
        for role, tag in ((1, "matrix_alone"), (2, "vector_alone"), (3, "both")):
            out = torch.zeros(8 * blocks, dtype=torch.int64, device=dev)
            for _ in range(2):
                rc = lib.fa_probe_coissue(opnd, role, blocks, iters, out.data_ptr(), sink.data_ptr(),
                                          stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"probe launch failed: hipError {rc}")
                torch.cuda.synchronize(dev)
            cyc = out.double().cpu().view(blocks, 8)
            if role & 1:
                row[tag + "_cycles_per_mfma"] = round(float(cyc[:, :4].max(dim=1).values.median()) / (32 * iters), 2)
            if role & 2:
                row[tag + "_cycles_per_softmax"] = round(float(cyc[:, 4:].max(dim=1).values.median()) / iters, 1)
        print(json.dumps(row), flush=True)


def valu_rate(iters: int = 2000, blocks: int = 256):
    """Vector ALU issue rates (the libfa_probe.so kernel): per CU, waves 0-3
    (one per SIMD) run operation A and waves 4-7 (their SIMD partners)
    operation B, 16 independent instructions per round. One JSON line per
    pair: shader cycles per instruction of each group (slowest wave of each
    workgroup, median over workgroups)."""
    import ctypes

    import torch

    from transformer_attention_08_amd import build as _b

    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.fa_probe_valu_rate.restype = ctypes.c_int
    lib.fa_probe_valu_rate.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    dev = torch.device("cuda:0")
    sink = torch.zeros(512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    names = {0: "idle", 1: "v_exp_f32", 2: "v_fma_f32", 3: "v_add_f32", 4: "v_cvt_pk_bf16_f32",
             5: "v_max3_f32", 6: "v_exp_f16", 7: "mfma_32x32x16_bf16"}
    pairs = [(1, 0), (2, 0), (3, 0), (4, 0), (5, 0), (6, 0), (7, 0), (1, 1), (2, 2), (1, 2), (1, 3), (7, 1), (7, 2)]
    for op_a, op_b in pairs:
        out = torch.zeros(8 * blocks, dtype=torch.int64, device=dev)
        for _ in range(2):
            rc = lib.fa_probe_valu_rate(op_a, op_b, blocks, iters, out.data_ptr(), sink.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"probe launch failed: hipError {rc}")
            torch.cuda.synchronize(dev)
        cyc = out.double().cpu().view(blocks, 8)
        # an MFMA round issues 8 MFMAs, a vector round 16 instructions
        per = {op: (8 if op == 7 else 16) * iters for op in (op_a, op_b)}
        row = {"probe": "valu_rate", "waves_0_3": names[op_a], "waves_4_7": names[op_b],
               "cycles_per_instr_0_3": round(float(cyc[:, :4].max(dim=1).values.median()) / per[op_a], 2)}
        if op_b:
            row["cycles_per_instr_4_7"] = round(float(cyc[:, 4:].max(dim=1).values.median()) / per[op_b], 2)
        print(json.dumps(row), flush=True)


def copy_rate(iters: int = 2000, blocks: int = 256):
    """Global -> LDS copies (the libfa_probe.so kernel): bytes per cycle per
    CU moved straight into LDS (buffer_load ... lds) or through registers,
    alone and beside a stream of 16-byte LDS reads or beside MFMAs fed by
    16-byte LDS reads, from a 2 MiB source (L2-resident) and from a 1 GiB
    one."""
    import ctypes

    import torch

    from transformer_attention_08_amd import build as _b

    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.fa_probe_copy_rate.restype = ctypes.c_int
    lib.fa_probe_copy_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    sink = torch.zeros(512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    names = {0: "lds_dma x8 waves", 1: "via registers x8 waves", 2: "lds_dma x4 + reads x4",
             3: "via registers x4 + reads x4", 4: "reads x4 alone", 5: "lds_dma x4 + MFMA x4 (LDS operands)",
             6: "MFMA x4 (LDS operands) alone", 7: "via registers x4 + MFMA x4 (LDS operands)"}
    for src_mib in (2, 1024):
        src = torch.zeros(src_mib << 20, dtype=torch.uint8, device=dev)
        for mode in range(8):
            out = torch.zeros(16 * blocks, dtype=torch.int64, device=dev)
            for _ in range(2):
                rc = lib.fa_probe_copy_rate(mode, src.data_ptr(), src.numel(), blocks, iters, out.data_ptr(),
                                            sink.data_ptr(), stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"probe launch failed: hipError {rc}")
                torch.cuda.synchronize(dev)
            v = out.view(blocks, 8, 2).double().cpu()
            cyc, rounds = v[..., 0], v[..., 1]
            row = {"probe": "copy_rate", "src_mib": src_mib, "mode": names[mode]}
            copiers = list(range(8)) if mode <= 1 else list(range(4)) if mode in (2, 3, 5, 7) else []
            readers = list(range(4, 8)) if mode in (2, 3, 4) else []
            matrix = list(range(4, 8)) if mode >= 5 else []
            if matrix:
                t = cyc[:, matrix].max(dim=1).values
                r = rounds[:, matrix].min(dim=1).values
                row["cycles_per_mfma"] = round(float((t / (r * 32)).median()), 2)
            if copiers:
                t = cyc[:, copiers].max(dim=1).values
                row["copy_bytes_per_clk_per_cu"] = round(float((len(copiers) * 4096 * iters / t).median()), 1)
            if readers:
                t = cyc[:, readers].max(dim=1).values
                b = (rounds[:, readers] * 8 * 1024).sum(dim=1)
                row["read_bytes_per_clk_per_cu"] = round(float((b / t).median()), 1)
            print(json.dumps(row), flush=True)
        del src


def wave_placement(blocks: int = 4):
    """SIMD of each wave of 512-thread workgroups (HW_ID register), per workgroup."""
    import ctypes

    import torch

    from transformer_attention_08_amd import build as _b

    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.fa_probe_hwid.restype = ctypes.c_int
    lib.fa_probe_hwid.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    out = torch.zeros(8 * blocks, dtype=torch.int32, device="cuda")
    rc = lib.fa_probe_hwid(blocks, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"probe launch failed: hipError {rc}")
    ids = [int(x) & 0xffffffff for x in out.cpu().tolist()]
    for b in range(blocks):
        w = ids[8 * b: 8 * b + 8]
        print(json.dumps({"probe": "wave_placement", "workgroup": b,
                          "simd_of_wave": [(x >> 4) & 3 for x in w], "wave_slot": [x & 15 for x in w],
                          "cu": [(x >> 8) & 15 for x in w]}), flush=True)


def backward_flops(w) -> float:
    """The five products of the gradient (S recomputed, dP, dV, dQ, dK), 2*n*n*d_k
    FLOP each per head; halved under a causal mask (2.5 x the forward count)."""
    f = 10.0 * w.batch * w.heads * w.n * w.n * w.d_k
    return f / 2 if w.causal else f


def time_steps(step, stream, steps, warmup):
    """`warmup` untimed calls, then `steps` calls timed as one block: one
    event before the first and one after the last, on the launch stream. An
    event recorded between two calls leaves the GPU idle for ~6 us (measured
    in kernel traces: back-to-back calls start with no gap), so per-call
    events stay out of the timed block. The same number of calls then runs
    again, each between two events of its own, for the per-call median and
    minimum. Returns (ms per call of the timed block, per-call ms)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({warmup} calls)", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    return total_ms / steps, per


def scrub_read(scrub, acc):
    """Read every element of scrub (a sum into acc)."""
    import torch
    torch.sum(scrub, dim=0, out=acc)


def cold_cache_pass(step, stream, flops, calls=10, scrub_bytes=512 << 20):
    """Per-call timing with scrub_bytes of device memory read before every
    call, so that no input is left in the L2s or the 256 MB Infinity Cache.
    The scrub reads (a sum) rather than writes, so that the call does not
    also pay for writing dirty scrub lines back; the events bracket the call
    alone."""
    import torch
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device="cuda")
    acc = torch.zeros((), dtype=torch.float32, device="cuda")
    per = []
    for _ in range(calls):
        scrub_read(scrub, acc)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    del scrub
    ms = statistics.median(per)
    return {"ms_median": round(ms, 5), "ms_min": round(min(per), 5),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "calls": calls, "scrub_bytes_read": scrub_bytes}


def bench_backward(args, w):
    """One step = one fa_backward call (both passes) on the workload, with the
    forward's O and LSE computed once beforehand."""
    import torch

    import transformer_attention_08_amd as fa
    import workload

    if w.dtype not in ("bf16", "f16"):
        print("the backward runs on f16 / bf16 workloads", file=sys.stderr)
        return 2
    inp, do = workload.make_inputs_with_grad(w.batch, w.heads, w.n, w.d_k, w.dtype, args.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = inp.to(dev)
    dog = do.to(dev)
    o, lse = fa.forward(d.q, d.k, d.v, causal=w.causal, scale=w.scale)
    dq, dk, dv = (torch.empty_like(d.q) for _ in range(3))
    ws = torch.empty(fa.backward_workspace_size(w.batch, w.heads, w.n), dtype=torch.uint8, device=dev)

    def step():
        fa.backward(d.q, d.k, d.v, o, lse, dog, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
                    workspace=ws)

    ms, per = time_steps(step, torch.cuda.current_stream(dev), args.steps, args.warmup)
    flops = backward_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    line = {
        "metric": f"attn bwd TFLOP/s ({w.name})",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q, K, V, dO of the workload's shape)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "n": w.n, "d_k": w.d_k,
                   "causal": w.causal, "flops_per_step": flops, "pass": "backward"},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "ms_median": round(statistics.median(per), 5),
        "ms_min": round(min(per), 5),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "kernel": "bwd_dq+bwd_dkdv2"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_backward(w, inp, do)
    print(json.dumps(line), flush=True)
    return 0


def varlen_lengths(count: int, n_max: int, seed: int):
    """Seeded log-normal sequence lengths in [16, n_max] (median about n_max / 5)."""
    import numpy as np
    rng = np.random.default_rng(seed + 7)
    mu = math.log(max(16, n_max // 5))
    return np.clip(np.exp(rng.normal(mu, 1.0, count)).astype(int), 16, n_max).tolist()


def bench_varlen(args, w):
    """One step = one fa_forward_varlen call over a packed batch of sequences
    of mixed lengths with the workload's heads, d_k, dtype and mask."""
    import numpy as np
    import torch

    import transformer_attention_08_amd as fa
    import workload

    lens = varlen_lengths(args.varlen, w.n, args.seed)
    total = int(sum(lens))
    if w.dtype == "fp8":
        print("the ragged-batch bench runs on f32 / f16 / bf16 workloads", file=sys.stderr)
        return 2
    inp = workload.make_inputs(1, w.heads, total, w.d_k, w.dtype, args.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (t[0].transpose(0, 1).contiguous().to(dev) for t in (inp.q, inp.k, inp.v))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.heads, total), dtype=torch.float32, device=dev)

    def step():
        fa.forward_varlen(q, k, v, cu, max(lens), causal=w.causal, scale=w.scale, out=o, lse=lse)

    ms, per = time_steps(step, torch.cuda.current_stream(dev), args.steps, args.warmup)
    flops = sum(4.0 * w.heads * x * x * w.d_k / (2 if w.causal else 1) for x in lens)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    line = {
        "metric": f"attn fwd TFLOP/s ({w.name}, ragged batch of {len(lens)})",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs; seeded log-normal sequence lengths)",
        "config": {"workload": w.name + "_varlen", "heads": w.heads, "d_k": w.d_k, "causal": w.causal,
                   "lengths": lens, "total_rows": total, "flops_per_step": flops},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "ms_median": round(statistics.median(per), 5),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None, "kernel": fwd_kernel(w, False, True)},
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_bf16_causal")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--splits", type=int, default=1,
                    help="cut the keys into this many blocks (fa_forward_splitkv) and merge; "
                         "0: the count fa_splitkv_splits chooses for the device")
    ap.add_argument("--backward", action="store_true",
                    help="time fa_backward (dQ, dK, dV) instead of the forward")
    ap.add_argument("--unfused", action="store_true",
                    help="time the unfused contrast (S and P written to memory) instead")
    ap.add_argument("--n", type=int, default=0, help="override the workload's sequence length")
    ap.add_argument("--layout", choices=("bhsd", "bshd"), default="bhsd",
                    help="bshd: q, k, v, o as [batch, n, heads, d_k] through fa_forward_strided")
    ap.add_argument("--varlen", type=int, default=0,
                    help="ragged batch of this many sequences (seeded log-normal lengths, "
                         "16 .. n rows) through fa_forward_varlen")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold-cache", action="store_true",
                    help="skip the second pass that reads 512 MiB of other device memory before each call")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-record", nargs=4, metavar="CSV",
                    help="write the HBM traffic record from four rocprofv3 counter files "
                         "(forward FETCH_SIZE, forward WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE)")
    ap.add_argument("--mfma-rate", action="store_true",
                    help="issue rate of the 32x32x16 and 16x16x32 MFMAs (libfa_probe.so)")
    ap.add_argument("--copy-rate", action="store_true",
                    help="global -> LDS copy rates, straight or through registers, beside LDS reads")
    ap.add_argument("--valu-rate", action="store_true",
                    help="vector ALU issue rates (exp, fma, add, pack, max3) alone and beside each other")
    ap.add_argument("--coissue", action="store_true",
                    help="MFMA / vector co-issue with register or LDS operands (libfa_probe.so)")
    ap.add_argument("--lds-rate", action="store_true",
                    help="LDS read bandwidth of ds_read_b128 and ds_read_b64_tr_b16 (libfa_probe.so)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward runs on a single MI355X "
              "here (heads would shard across GPUs with no communication); run with --gpus 1.",
              file=sys.stderr)
        return 2

    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.traffic_record:
        traffic_record(*args.traffic_record)
        return 0
    if args.mfma_rate:
        mfma_rate()
        return 0
    if args.lds_rate:
        lds_rate()
        return 0
    if args.valu_rate:
        valu_rate()
        return 0
    if args.copy_rate:
        copy_rate()
        return 0
    if args.coissue:
        coissue()
        wave_placement()
        return 0

    import torch

    import transformer_attention_08_amd as fa
    import workload

    w = workload.WORKLOADS[args.workload]
    if args.n:
        import dataclasses
        w = dataclasses.replace(w, name=f"{w.name}_n{args.n}", n=args.n)
    fa.load_library()
    if args.backward:
        return bench_backward(args, w)
    if args.varlen:
        return bench_varlen(args, w)
    inp = workload.workload_inputs(w, args.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = inp.to(dev)
    o = torch.empty(w.batch, w.heads, w.n, w.d_k, dtype=workload.torch_dtype(w.out_dtype), device=dev)
    lse = torch.empty(w.batch, w.heads, w.n, dtype=torch.float32, device=dev)
    if args.splits == 0:
        args.splits = fa.splitkv_splits(w.batch, w.heads, w.n, w.causal)
    if args.splits > 1 and w.dtype == "fp8" and (inp.q_descale, inp.k_descale, inp.v_descale) != (1, 1, 1):
        print("the split-KV entry takes e4m3 with unit descales only", file=sys.stderr)
        return 2
    ws = None
    if args.splits > 1:
        need = fa.splitkv_workspace_size(w.batch, w.heads, w.n, w.d_k, args.splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    if args.layout == "bshd":
        qs, ks, vs = (t.transpose(1, 2).contiguous() for t in (d.q, d.k, d.v))
        os_ = torch.empty((w.batch, w.n, w.heads, w.d_k), dtype=o.dtype, device=dev)
    uws = None
    if args.unfused:
        if w.dtype not in ("bf16", "f16"):
            print("the unfused contrast runs on f16 / bf16 workloads", file=sys.stderr)
            return 2
        uws = torch.empty(fa.unfused_workspace_size(w.batch, w.heads, w.n), dtype=torch.uint8, device=dev)

    def step():
        if args.layout == "bshd":
            fa.forward_strided(qs, ks, vs, layout="bshd", causal=w.causal, scale=w.scale, out=os_, lse=lse)
        elif uws is not None:
            fa.forward_unfused(d.q, d.k, d.v, causal=w.causal, scale=w.scale, out=o, lse=lse,
                               workspace=uws)
        elif ws is not None:
            fa.forward_splitkv(d.q, d.k, d.v, args.splits, causal=w.causal, scale=w.scale, out=o,
                               lse=lse, workspace=ws)
        elif w.dtype == "fp8":
            fa.forward_fp8(d.q, d.k, d.v, inp.q_descale, inp.k_descale, inp.v_descale,
                           causal=w.causal, scale=w.scale, out=o, lse=lse)
        else:
            fa.forward(d.q, d.k, d.v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    stream = torch.cuda.current_stream(dev)  # the stream fa_forward enqueues on
    ms, per = time_steps(step, stream, args.steps, args.warmup)

    flops = algorithmic_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = stored_traffic(w.name)
    split_tag = f", split-KV {args.splits}" if ws is not None else ""
    if uws is not None:
        split_tag = ", unfused: S and P in memory"
    if args.layout == "bshd":
        split_tag += ", [b, n, h, d_k] layout"
    if ws is not None or uws is not None or args.n or args.layout != "bhsd":
        traffic = None  # the stored counters cover the fused kernel at the stored shape only
    line = {
        "metric": (METRIC if w.name == "llama3_8b_bf16_causal" and ws is None and uws is None
                   and args.layout == "bhsd"
                   else f"attn fwd TFLOP/s ({w.name}{split_tag})"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "n": w.n, "d_k": w.d_k,
                   "causal": w.causal, "flops_per_step": flops, "splits": args.splits,
                   "layout": args.layout},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "ms_median": round(statistics.median(per), 5),
        "ms_min": round(min(per), 5),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic,
                     "kernel": ("unf_scores+unf_softmax+unf_pv" if uws is not None else
                                fwd_kernel(w, ws is not None) + ("+combine_splits" if ws is not None else "")),
                     "min_hbm_bytes": min_hbm_bytes(w)},
    }
    if traffic is not None:
        # not counted in this run: the committed FETCH_SIZE / WRITE_SIZE
        # record, used only while its kernel source hash matches this build
        line["roofline"]["traffic_source"] = (f"stored counter record {os.path.relpath(TRAFFIC_FILE, ROOT)} "
                                              f"(kernel source hash {kernel_source_hash()})")
    if not args.no_cold_cache:
        line["cold_cache"] = cold_cache_pass(step, stream, flops)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
