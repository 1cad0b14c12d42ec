"""CPU fp64 oracle for ring attention (forward, backward) and Ulysses (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package. It does not import the HIP library and the library does not import it.
"""
from .fp64 import (  # noqa: F401
    NEG_INF, attention, contiguous_order, layout_order, merge, pairs_per_rank_step,
    permute_rows, rank_positions, ring_attention, ring_schedule, ring_source,
    striped_order, to_f64, unpermute_rows, useful_flops, useful_pairs, zigzag_order,
)
from .fp64_bwd import (  # noqa: F401
    attention_backward, attention_backward_dq_rows, backward_flops, block_backward,
    ring_attention_backward,
)
from .fp64_ulysses import (  # noqa: F401
    ulysses_all_to_all, ulysses_all_to_all_inverse, ulysses_attention, ulysses_volume,
    usp_attention, usp_token_lists,
)
