"""Tree-masked grouped-query attention over a paged KV cache (float64).

What is computed (SpecExec page, "Approach": the whole draft tree is verified
in one target pass; EasySpec page, "+tree" baseline): for sequence b, tree
node i and query head h, with KV head g = h // (Hq / Hkv),

    S(b, i)  = { p : 0 <= p < ctx_b }  U  { ctx_b + j : j in anc*(i) }
    out[b, i, h] = sum_{p in S} softmax_p(scale * q[b, i, h] . K_g(p)) V_g(p)

where K_g(p) and V_g(p) live in the page ``block_table[b][p // bs]`` at offset
``p % bs``.  The sparse variant (sparse-verification page, "Methodology":
keep only the top-k key/value blocks per query) restricts the context part to
positions whose block index is in ``sel_blocks[b, i, h]``; the tree part is
always attended.

Readings: node i's own K/V sits at position ctx_b + i (the caller writes it
there); scale defaults to D^-1/2; no positional bias (RoPE is applied by the
caller).  K and V pages are [num_blocks, Hkv, bs, D].

Two independent formulations are given and must agree:
``attention_dense`` builds the context-plus-ancestor mask for all nodes at once;
``attention_by_path`` runs ordinary causal attention along each node's own
root path, one node at a time.
"""
import numpy as np

from .codec import decode
from .tree import ancestor_matrix, root_path


def _tree_row(tree_parent, b):
    tp = np.asarray(tree_parent)
    return tp[0] if tp.shape[0] == 1 else tp[b]


def gather_kv(k_pages, v_pages, block_table, b, g, positions, bs, dtype):
    """K and V rows [n, D] (float64) at the given logical positions of sequence b."""
    pos = np.asarray(positions, dtype=np.int64)
    blk = np.asarray(block_table)[b, pos // bs]
    off = pos % bs
    K = decode(k_pages[blk, g, off, :], dtype)
    V = decode(v_pages[blk, g, off, :], dtype)
    return K, V


def _context_positions(ctx, bs, sel):
    if sel is None:
        return np.arange(ctx)
    keep = sorted({int(n) for n in sel if n >= 0})
    pos = [p for n in keep for p in range(n * bs, min((n + 1) * bs, ctx))]
    return np.asarray(pos, dtype=np.int64)


def _softmax_attend(qv, K, V, scale):
    s = scale * (K @ qv)
    s = s - s.max()
    w = np.exp(s)
    return (w / w.sum()) @ V


def attention_dense(q, k_pages, v_pages, block_table, ctx_lens, tree_parent, bs, dtype,
                    scale=None, sel_blocks=None, rows=None):
    """All nodes at once with a [T, ctx + T] mask.  ``rows`` (optional) is a list
    of (b, i, h) triples; then an array [len(rows), D] is returned instead of
    the full [B, T, Hq, D] output."""
    B, T, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    scale = D ** -0.5 if not scale else float(scale)
    want = None
    if rows is not None:
        want = {}
        for r, (b, i, h) in enumerate(rows):
            want.setdefault((b, h // G), []).append((r, i, h))
    out = np.zeros((B, T, Hq, D)) if rows is None else np.zeros((len(rows), D))
    for b in range(B):
        ctx = int(ctx_lens[b])
        A = ancestor_matrix(_tree_row(tree_parent, b))
        for g in range(Hkv):
            if want is not None and (b, g) not in want:
                continue
            K, V = gather_kv(k_pages, v_pages, block_table, b, g, np.arange(ctx + T), bs, dtype)
            items = want[(b, g)] if want is not None else \
                [(None, i, g * G + hh) for i in range(T) for hh in range(G)]
            for r, i, h in items:
                mask = np.zeros(ctx + T, dtype=bool)
                if sel_blocks is None:
                    mask[:ctx] = True
                else:
                    mask[_context_positions(ctx, bs, sel_blocks[b, i, h])] = True
                mask[ctx:] = A[i]
                o = _softmax_attend(decode(q[b, i, h], dtype), K[mask], V[mask], scale)
                if r is None:
                    out[b, i, h] = o
                else:
                    out[r] = o
    return out


def attention_by_path(q, k_pages, v_pages, block_table, ctx_lens, tree_parent, bs, dtype,
                      scale=None, sel_blocks=None):
    """One node at a time: lay the node's root path out as an ordinary sequence
    after the context and run causal attention over it; node i is the path's
    last token, so it sees the context and every path token."""
    B, T, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    scale = D ** -0.5 if not scale else float(scale)
    out = np.zeros((B, T, Hq, D))
    for b in range(B):
        ctx = int(ctx_lens[b])
        par = _tree_row(tree_parent, b)
        for i in range(T):
            path = root_path(par, i)
            for h in range(Hq):
                g = h // G
                sel = None if sel_blocks is None else sel_blocks[b, i, h]
                cpos = _context_positions(ctx, bs, sel)
                seq = np.concatenate([cpos, ctx + np.asarray(path, dtype=np.int64)])
                K, V = gather_kv(k_pages, v_pages, block_table, b, g, seq, bs, dtype)
                n = len(seq)
                # causal mask over the laid-out sequence; the query is its last token
                causal = np.tril(np.ones((n, n), dtype=bool))
                s = scale * (K @ decode(q[b, i, h], dtype))
                s = np.where(causal[n - 1], s, -np.inf)
                s = s - s.max()
                w = np.exp(s)
                out[b, i, h] = (w / w.sum()) @ V
    return out
