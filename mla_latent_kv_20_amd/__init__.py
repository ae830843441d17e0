"""MLA absorbed decode over a latent KV cache on MI355X (gfx950).

The compute lives in the HIP library ``libmla_kv.so`` built from ``csrc/``;
``mla_latent_kv_20_amd.binding`` is the thin ctypes layer over its C ABI.
Importing the package does not load the library: the binding loads it on first
use and raises if it is missing.
"""
