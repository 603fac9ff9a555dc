"""Tree verification for speculative decoding on MI355X (gfx950).

The verification pass -- tree-masked attention over a paged KV cache, the
token-acceptance walk, the path commit and top-k block selection for sparse
verification -- as hand-written HIP kernels behind a small C ABI
(include/sdtree.h, libsdtree.so).  This package holds the kernels' sources
(csrc/), the in-tree build (build.py) and a ctypes binding (_lib.py).
"""
from ._lib import (  # noqa: F401
    SdError, accept, accept_commit, attn_timing_events, accept_commit_noalloc, block_sums, block_sums_append, device_status, kv_commit, lib,
    topk_blocks, topk_blocks_cached, topk_blocks_shared, tree_build, tree_expand, tree_verify_attn,
    workspace_bytes,
)
