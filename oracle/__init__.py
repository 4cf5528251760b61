"""CPU oracle for the paged KV cache hot path (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never does, and this package imports nothing from it.
"""
from .attention import (widen, kv_cache_write, gather_kv, attention_seq_kvhead,  # noqa: F401
                        paged_attention, merge_partials, split_attention, block_bytes,
                        blocks_for_tokens)
from .fp8 import (E4M3_MAX, e4m3_decode, e4m3_encode, quantize,  # noqa: F401
                  kv_cache_write_fp8)
from .cascade import cascade_attention, check_cascade_metadata, cascade_traffic_bytes  # noqa: F401
