"""CPU oracle (test infrastructure only): plain fp64 MLA decode written from the pages."""
from .mla_oracle import (  # noqa: F401
    absorb_q, absorb_q_folded, absorb_q_rope, absorbed_decode, append_rows, attend_latent,
    cache_elems_per_token, default_scale, dequantize_rows, e4m3_encode, e4m3_value, fold_o, fold_q,
    kv_prologue, merge_splits, naive_decode, o_proj, out_folded, out_proj, q_up, quantize_rows,
    rope_frequencies, rope_pairs, split_bounds, split_partials, visible_rows, yarn_softmax_scale,
)
