"""CPU oracle for exact scaled-dot-product attention, forward and gradients.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
reference that the HIP kernels are checked against. Only the test suite, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import it. It shares no code with the HIP path and the product never
routes through it.

Contents
  formats    -- decoders from stored bits (fp32, fp16, bf16, OCP fp8 e4m3fn)
                to float64, written from the format definitions.
  reference  -- the definition materialised in float64 (scores S and
                probabilities P per full row), a literal streaming version of
                the online-softmax recurrence, the associative merge of
                (m, l, o) states, and a 50-digit ``decimal`` brute force.
  backward   -- the gradients dQ, dK, dV of the definition (S, P, dP, dS
                materialised), plus row and key-column samplers for full sizes.
  accounting -- FLOP, byte and exponential counts of the method.

Parity status: every function here is pinned by ``tests/test_oracle.py`` and
``tests/test_oracle_backward.py``
against brute force, closed forms and invariants the pages fix. The numeric
tolerances that the GPU must meet are not derivable from the pages (they
announce an error analysis but never print it); those numbers are stated,
not pinned.
"""
from .formats import decode, decode_bf16, decode_e4m3fn, decode_f16, decode_f32  # noqa: F401
from .reference import (  # noqa: F401
    attention,
    attention_decimal,
    merge_states,
    empty_state,
    online_attention,
    tile_state,
    finalize_state,
)
from .backward import (  # noqa: F401
    attention_backward,
    backward_rows,
    backward_key_columns,
    head_statistics,
)
from .accounting import flops, min_hbm_bytes, exp_count, score_matrix_ratio  # noqa: F401
