"""Work and traffic counts of the attention forward pass (oracle side).

FLOPs: the two GEMMs only, 2*n*n*d_k each per head, i.e. 4*h*n^2*d_k per
layer -- the count the "Case study: FlashAttention" slides give in "The same
computation at real size" (about 1.1 TFLOP for h=32, n=8192, d_k=128). With a
causal mask half of the score matrix is excluded, so the count is halved
(the convention used for every causal figure in this repository). Softmax
arithmetic is not counted: the same slide treats scale/mask/softmax as a
bytes-bound step, not a FLOP-bound one.

Bytes: the unavoidable HBM traffic of a fused kernel -- read Q, K, V once,
write O and the per-row log-sum-exp (fp32) once. O is written in the input
type, except for e4m3 inputs, whose O is bf16.
"""
from __future__ import annotations

ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def flops(batch: int, heads: int, n: int, d_k: int, causal: bool) -> float:
    f = 4.0 * batch * heads * n * n * d_k
    return f / 2.0 if causal else f


def exp_count(batch: int, heads: int, n: int, causal: bool) -> int:
    """Exponentials the method evaluates: one per visible (query, key) pair,
    i.e. per entry of P that the mask leaves in place -- n * n per head, or
    n (n + 1) / 2 under the causal mask (query i sees keys 0 .. i). Exact,
    not the halved FLOP convention."""
    per_head = n * (n + 1) // 2 if causal else n * n
    return int(batch) * int(heads) * per_head


def min_hbm_bytes(batch: int, heads: int, n: int, d_k: int, in_dtype: str, out_dtype: str,
                  with_lse: bool = True) -> int:
    rows = batch * heads * n
    b = rows * d_k * (3 * ELT_BYTES[in_dtype] + ELT_BYTES[out_dtype])
    if with_lse:
        b += 4 * rows
    return int(b)


def score_matrix_ratio(n: int, d_k: int) -> float:
    """Elements of one head's S (n x n) over elements of its Q (n x d_k)."""
    return (n * n) / (n * d_k)
