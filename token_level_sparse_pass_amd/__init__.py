"""HySparse2 Hybrid Block engine for AMD MI355X (gfx950).

`hs2` is the binding of the C-ABI library libhs2.so: hs2.full_attn_select,
hs2.sparse_attn and hs2.block_forward. Build the library with
`python -m token_level_sparse_pass_amd.build`.
"""
from . import hs2  # noqa: F401
