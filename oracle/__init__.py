"""Plain CPU oracle for paged MLA decode under decode context parallelism.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
the tests, the smoke check and the benchmark's CPU-baseline leg may call it.
It shares no code with the HIP path.

Every function is pinned by CPU tests against something other than itself
(closed forms, brute force, library routines, the pages' integer formulas and
a hand-derived slot example); see tests/test_oracle_pins.py.
"""
from .mla_oracle import (  # noqa: F401
    D_QK, D_V, PAD_SLOT_ID,
    bf16_bits_to_f64, e4m3_to_f64, e4m3_encode, owns, held_positions, visible_positions, local_count,
    attend, mla_decode, mla_decode_varlen, merge_lse, cp_local_slot, kv_write, kv_write_fp8,
)
