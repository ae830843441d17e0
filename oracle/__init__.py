"""CPU oracle (test infrastructure only): plain fp64 MLA decode written from the pages."""
from .mla_oracle import (  # noqa: F401
    absorb_q, absorb_q_folded, absorb_q_rope, fold_o, fold_q, o_proj, out_folded, q_up, absorbed_decode, append_rows, attend_latent, cache_elems_per_token,
    default_scale, dequantize_rows, rope_frequencies, yarn_softmax_scale, e4m3_encode, e4m3_value, kv_prologue, quantize_rows, rope_frequencies, yarn_softmax_scale, merge_splits, naive_decode, out_proj, rope_pairs, split_bounds,
    split_partials, visible_rows,
)
