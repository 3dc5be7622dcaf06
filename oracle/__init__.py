"""Plain CPU oracle for the QLoRA NF4 + double-quantisation + LoRA linear path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it. It shares no code, tables or constants
with the HIP library; the two meet only on the seeded inputs.

Every floating-point step is written in float64 (or in float32 where the
method itself fixes float32 rounding, as the dequantised constants do), in the
order the pages give, so that a reader can check it against them by eye.

Parity pins: every public function here is pinned by tests under
``tests/test_oracle_*.py`` against facts fixed outside this module (library
routines, closed forms, brute force, invariants). The one choice no page
fixes -- the tail probability ``DELTA`` of the level construction -- is a
reading and is flagged as such where it is defined, as are the Int4 and FP4
data types the pages compare NF4 with but do not define, and the optimizer
update rule (the pages describe paged optimizer state, not the update).
"""

from .nf4_oracle import (  # noqa: F401
    DELTA,
    NF4_BLOCK,
    DQ_BLOCK,
    phi_inv,
    nf4_levels_f64,
    nf4_levels,
    e4m3_decode,
    e4m3_encode_rne,
    bf16_round,
    quantize_nf4_dq,
    dequant,
    int4_levels,
    e2m1_decode,
    fp4_levels,
    codebook_levels,
    quantize_blockwise,
    dequant_blockwise,
    unpack_codes,
    storage_bits_per_param,
    linear_fwd,
    linear_bwd,
    grouped_linear_fwd,
    grouped_linear_bwd,
    merge_lora,
)
from .adamw import adamw_step  # noqa: F401
