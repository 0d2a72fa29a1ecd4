"""CPU oracle for attention over a paged KV cache (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library.
"""
from .paged_attention import (  # noqa: F401
    combine,
    decode,
    decode_partials,
    extend,
    gather,
    kv_store,
    token_slots,
    widen,
)
from .rope import rope, rope_kv_store  # noqa: F401
