"""fp64 CPU oracle (test infrastructure only; see sva_oracle's header)."""
from .sva_oracle import (  # noqa: F401
    token_coords, phi, rope_rotate, block_states, lin_attn_fwd,
    block_cache_apply, block_cache_commit, lin_attn_bwd,
)
