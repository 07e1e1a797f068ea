"""CPU oracle for the paged decode-attention hot path.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The library (the HIP kernels behind
the C ABI and its Python binding) never imports, links or calls it, and shares
no code with it.
"""

from .paged_attention import (  # noqa: F401
    ELEMENT_TYPES,
    bruteforce_decode,
    copy_blocks,
    decode,
    decode_blockwise,
    decode_partitioned,
    decode_probabilities,
    gather_sequence,
    prefill,
    swap_in,
    swap_out,
    to_float64,
    v_slot,
    write_kv,
)
