"""CPU oracle for the attention forward and split-KV decode (TEST INFRASTRUCTURE).

This package is test infrastructure, not part of the product path.  Only the
test suite, the smoke entry point and the benchmark's CPU-baseline leg may
import it.  It shares no code with the HIP library and imports nothing from
it.  Everything is plain numpy in float64 and materialises the full score and
probability matrices, so that a reader can check it against the pages'
definitions by eye.

Every function here is pinned by tests outside this package (brute force on
tiny inputs, a library special case, closed forms and invariants); there is no
"parity unpinned" function.
"""
from .attention import (attn_fp8qk_ref, attn_ref, decode_fp8kv_partials_ref, decode_fp8kv_ref, decode_partials_ref, decode_ref,
                        e4m3_decode, lse_merge_ref, paged_decode_partials_ref, paged_decode_ref)

__all__ = ["attn_ref", "decode_partials_ref", "lse_merge_ref", "decode_ref", "paged_decode_partials_ref",
           "paged_decode_ref", "e4m3_decode", "decode_fp8kv_partials_ref", "decode_fp8kv_ref", "attn_fp8qk_ref"]
