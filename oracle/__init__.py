"""CPU oracle for paged decode attention, the slot-mapped KV write and the
copy-on-write block copy.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
may call it.  It shares no code with the HIP library and imports nothing from
it; it reads plain numpy arrays and returns plain numpy arrays.

Every floating-point result is computed in float64 from the exact values of
the stored bits (bfloat16 and float32 both widen to float64 without rounding).
Integer and bit results (slots, cache writes, block copies) are exact.

Every function here is pinned in ``tests/test_oracle_pins.py`` against facts
that do not come from this module (worked tables printed on the pages,
brute-force dense attention, torch's CPU SDPA in float64, closed forms).
No function is "parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    BF16,
    F32,
    to_f64,
    slot_mapping,
    write_kv,
    copy_blocks,
    decode_attention,
    pool_dims,
    ORACLE_DTYPES,
)
