"""fp64 CPU oracle for QSA (test infrastructure only; never used by the product path)."""
from .qsa_oracle import (  # noqa: F401
    attend,
    attend_given_selection,
    block_scores,
    compress_keys,
    default_scale,
    qsa_decode,
    qsa_prefill,
    qsa_rows,
    select_blocks,
    visible_positions,
)
