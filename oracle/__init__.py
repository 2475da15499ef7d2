"""CPU fp64 oracle (test infrastructure; never imported by the product path)."""
from .attention import (  # noqa: F401
    CacheModel,
    PagedCacheModel,
    attend_row,
    brute,
    chunked,
    decode_cached,
    decode_paged,
    decode_recompute,
    extend,
    extend_paged,
    kv_bytes,
    kv_head_of,
    naive_causal,
    naive_windowed,
    visible,
    visible_keys,
)
from . import model  # noqa: F401,E402
