"""Committing the accepted root path into the paged KV cache.

After acceptance the accepted nodes' keys and values become ordinary
committed context, in path order, right after the old context; the context
length grows by the path length.  Reading: node j's K/V was written at
position ctx_b + j before verification, so the accepted path is compacted:

    new[ctx_b + j] = old[ctx_b + path[b, j]]   for j < path_len[b], K and V, every head
    ctx_b          += path_len[b]

Every other slot and sequence keeps its bytes.  Reads come from the old cache
(the copy is not done in place here).
"""
import numpy as np


def commit(k_pages, v_pages, block_table, ctx_lens, path, path_len, bs):
    K = k_pages.copy()
    V = v_pages.copy()
    for b in range(len(ctx_lens)):
        ctx = int(ctx_lens[b])
        for j in range(int(path_len[b])):
            src = ctx + int(path[b, j])
            dst = ctx + j
            sb, so = int(block_table[b, src // bs]), src % bs
            db, do = int(block_table[b, dst // bs]), dst % bs
            K[db, :, do, :] = k_pages[sb, :, so, :]
            V[db, :, do, :] = v_pages[sb, :, so, :]
    new_ctx = (np.asarray(ctx_lens, dtype=np.int64) + np.asarray(path_len)).astype(np.int32)
    return K, V, new_ctx
