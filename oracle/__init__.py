"""CPU oracle (test infrastructure only): plain fp64 MLA decode written from the pages."""
from .mla_oracle import (  # noqa: F401
    absorb_q, absorbed_decode, attend_latent, cache_elems_per_token, default_scale,
    merge_splits, naive_decode, out_proj, rope_pairs, split_bounds, split_partials,
    visible_rows,
)
