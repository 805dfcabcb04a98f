"""The C ABI on the host: the library loads, exports what include/fa.h
declares, and rejects every invalid argument before any HIP call.

Invalid calls use fake (never dereferenced) addresses: validation runs on the
host and returns before anything is launched, so these tests are safe with or
without a GPU. The one valid call with fake addresses runs only where no GPU
is visible, where the library must report FA_ERR_HIP instead of crashing.
"""
import ctypes
import os
import re

import pytest
import torch

import transformer_attention_08_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# fake, 16-byte aligned, non-overlapping "device" addresses
BASE = 1 << 40
SPAN = 1 << 32
Q, K, V, O, L = (BASE + i * SPAN for i in range(5))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def call(lib, q=Q, k=K, v=V, o=O, lse=L, b=1, h=2, n=100, d=128, scale=0.125, causal=1, dtype=2):
    return lib.fa_forward(q, k, v, o, lse, b, h, n, d, scale, causal, dtype, None)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_and_status_strings(lib):
    assert lib.fa_abi_version() == 10000
    for code in range(10):
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_string(99).decode() == "unknown status"
    assert lib.fa_last_hip_error() in (0,) or isinstance(lib.fa_last_hip_error(), int)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(b=0), 2), (dict(h=0), 2), (dict(n=0), 2), (dict(n=-5), 2), (dict(b=-1), 2),
    (dict(dtype=4), 3), (dict(dtype=-1), 3),
    (dict(d=32), 4), (dict(d=96), 4), (dict(d=256), 4), (dict(causal=2), 4), (dict(causal=-1), 4),
    (dict(q=Q + 8), 5), (dict(o=O + 2), 5), (dict(lse=L + 4), 5),
    (dict(scale=float("nan")), 6), (dict(scale=float("inf")), 6), (dict(scale=-0.5), 6),
    (dict(scale=3e38), 6),
    (dict(o=Q), 7), (dict(o=K + 4096), 7), (dict(lse=V + 1024), 7), (dict(lse=O + 16), 7),
    (dict(b=65536, h=65536), 8), (dict(b=2 ** 20, h=2 ** 10, n=2 ** 20), 8),
])
def test_validation_errors(lib, kw, status):
    assert call(lib, **kw) == status


def test_validation_order_null_before_shape(lib):
    assert call(lib, q=None, n=0) == 1


def test_fp8_entry_validates_descales(lib):
    def c8(qd=1.0, kd=1.0, vd=1.0, **kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, b=1, h=2, n=100, d=128, scale=0.125, causal=0)
        a.update(kw)
        return lib.fa_forward_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["b"], a["h"], a["n"],
                                  a["d"], a["scale"], a["causal"], qd, kd, vd, None)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert c8(qd=bad) == 6 and c8(kd=bad) == 6 and c8(vd=bad) == 6
    assert c8(n=0) == 2
    assert c8(q=None) == 1
    assert c8(scale=1e30, qd=1e10, kd=1e10) == 6


def test_lse_may_be_null_for_validation(lib):
    # a NULL lse is allowed; with a bad shape the status is still the shape error
    assert call(lib, lse=None, n=0) == 2


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a visible GPU")
def test_valid_call_without_gpu_reports_hip_error(lib):
    assert call(lib) == 9
    assert lib.fa_last_hip_error() != 0


def test_binding_rejects_bad_tensors():
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        fa.forward(x, x, x)  # host tensors
    with pytest.raises(ValueError):
        fa.forward(x[0], x[0], x[0])  # wrong rank
