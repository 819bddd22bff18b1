"""CPU oracle (test infrastructure only; see irm_oracle's header)."""
from .irm_oracle import (  # noqa: F401
    TableError,
    bf16_to_f64,
    rope_inv_freq,
    rotate,
    delta_rotate,
    expand_table,
    assemble_rows,
    rotate_gather,
    mla_decode,
    mla_prefill_tail,
)
