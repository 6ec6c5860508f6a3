"""CPU oracle for paged decode attention and the KV-cache scatter.

This package is test infrastructure. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the library path never does,
and it shares no code with the HIP kernels (no helpers, tables or constants).

Everything is plain numpy in float64 (integer copies for the cache scatter),
written for a reader to check against the pages by eye.
"""

from .paged_attention import (  # noqa: F401
    blocks_needed,
    unused_slots,
    slot_of_token,
    upcast,
    reshape_and_cache,
    gather_sequence,
    decode,
    decode_partitions,
    lse_merge,
    decode_split,
    copy_blocks,
    swap_blocks,
    prefill,
)
