"""CPU oracle for the compensated 4-bit linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
restatement of what the layer computes, written from the explanation pages of
"SPEAR: A System for Post-Quantization Error-Adaptive Recovery Enabling
Efficient Low-Bit LLM Serving" (gist.science, paper 2606.11244; English page,
Technical Summary).  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  The GPU library never calls it and shares no
code, constant or helper with it.

Every function pins to something other than itself in ``tests/test_oracle.py``
(brute force on tiny shapes, closed forms, special cases, hand-derived golden
values).  Parity status per function:

* ``unpack_int4`` / ``pack_int4``  - pinned (exhaustive, hand word, round trip)
* ``tile_words`` / ``untile_words`` - pinned (per-code byte addresses, hand
                                     tile, padding, round trip)
* ``dequant``                      - pinned (brute force, integer closed form)
* ``sigmoid`` / ``gate``           - pinned (special values, symmetry, math.exp)
* ``spear_linear_ref``             - pinned (brute force, r=0, gate off/on,
                                     rank-1 and full-rank closed forms, golden)
* ``rank_gate_linear_ref``         - pinned (brute force, reduction to the
                                     scalar gate, closed forms)
* ``select_chunk_ref``             - pinned (brute force over candidates,
                                     monotonicity in the budget)
"""

from .spear_ref import (  # noqa: F401
    ORACLE_IS_TEST_INFRASTRUCTURE,
    act_bits_to_f64,
    bf16_bits_to_f64,
    dequant,
    f16_bits_to_f64,
    gate,
    pack_int4,
    rank_gate_linear_ref,
    select_chunk_ref,
    sigmoid,
    spear_linear_ref,
    tile_words,
    unpack_int4,
    untile_words,
)
