"""Build the HIP library ``libfa.so`` in place (gfx950 only).

The library holds the fused attention forward and backward kernels and the C ABI of
``include/fa.h``. It is compiled with hipcc for ``--offload-arch=gfx950``;
hipcc cross-compiles without a GPU present.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ("fa_fwd.hip", "fa_bwd.hip", "fa_unfused.hip", "fa_noalloc.hip", "fa_api.cpp")
# the matrix-core rate probe behind `bench.py --mfma-rate`; a library of its own
PROBE_LIB = os.path.join(PKG, "libfa_probe.so")
PROBE_SOURCES = ("fa_probe.hip",)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def compile_command(out: str = LIB, extra=(), sources=SOURCES) -> list:
    srcs = [os.path.join(CSRC, s) for s in sources]
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # keep the compiler from forming packed fp32 arithmetic in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        *extra, *srcs, "-o", out,
    ]


def _compile(out: str, extra, sources, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = compile_command(tmp, extra, sources)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose and r.stderr.strip():
        print(r.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra=()) -> str:
    """Compile libfa.so and the probe library; returns libfa.so's path.
    Always recompiles."""
    _compile(PROBE_LIB, (), PROBE_SOURCES, verbose)
    return _compile(LIB, extra, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
