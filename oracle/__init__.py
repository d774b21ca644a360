"""fp64 CPU oracle (test infrastructure only; see ``oracle.core``).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.
"""
from .core import (  # noqa: F401
    attention, attention_head, attention_rows, bf16_bits_to_f64, causal_visible,
    combine_partials, decode_contiguous, decode_key_range, decode_paged, default_scale,
    kv_cache_bytes, kv_head_index, merge_softmax_states, paged_logical_rows, softmax_state,
    split_partials, tiled_forward, to_f64, window_visible,
)
from .backward import attention_backward, attention_backward_sampled, gradient_magnitudes, row_dot  # noqa: F401,E402
