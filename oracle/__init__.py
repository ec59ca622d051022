"""float64 CPU oracle (test infrastructure only; never part of the product path)."""

from .relpos_oracle import (  # noqa: F401
    attention_dense,
    dense_bias,
    rel_tables,
    relpos_attention,
    relpos_attention_rows,
    softmax_rows,
    token_coords,
)
