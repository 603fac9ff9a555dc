"""Top-k KV-block selection for sparse verification (float32, order pinned).

The sparse-verification page ("Methodology", attention sparsity) keeps only
the top-k key/value blocks per query, chosen by a cheap relevance score.
Reading of the score: the mean-pooled key of each block, dotted with the
query (signed, unscaled).  Candidates are the blocks holding committed
context, n < ceil(ctx_b / bs); tree slots are never candidates (they are
always attended).  Selection is per query (b, node, query head).

Because the indices must match exactly, the float32 arithmetic is fixed:

* mean  = (sequential float32 sum over the block's valid tokens, in
          position order) / n_valid, one IEEE division;
* score = products q[d] * mean[d] in float32, then a halving tree:
          add element d + D/2 into d, then d + D/4, ..., then d + 1;
* order = score descending, then block index ascending; keep the first k,
          emit them in ascending block order, pad with -1.

Cached block sums (the selection read from per-block summaries kept as the
context grows): `block_sums` is the numerator of the mean above, per
physical block, and `append_block_sums` extends it by the positions a
commit appended, continuing the same sequential sum; a mean formed from the
kept sums is therefore the same float32 value as one formed from K.

Shared selection (the sparse-verification page, "Methodology", reuse across
draft tokens): one selection per (sequence, KV group), used by every tree
node and every query head of the group.  Reading of its score: the sum of the
group's per-row relevance scores, formed as the pooled query dotted with the
block mean.  The pooled query is a sequential float32 sum from +0 of the
group's query rows, node by node and, within a node, head by head; the dot
product and the order are those above.
"""
import numpy as np

from .codec import decode_f32


def _block_sum(k_pages, blk, t0, t1, dtype, start=None):
    """Sequential float32 sum of K rows t0 <= t < t1 of physical block blk
    (all heads), continuing from `start` (else from +0)."""
    Hkv, D = k_pages.shape[1], k_pages.shape[3]
    s = np.zeros((Hkv, D), dtype=np.float32) if start is None else np.array(start, dtype=np.float32)
    for t in range(t0, t1):
        s = s + decode_f32(k_pages[blk, :, t, :], dtype)
    return s


def block_sums(k_pages, block_table, ctx_lens, bs, dtype):
    """float32 [num_blocks, Hkv, D]: for every context block n < ceil(ctx_b / bs)
    of every sequence, the sequential sum of its valid K rows at its physical
    block; NaN for blocks no sequence holds as context."""
    nb_phys, Hkv, _, D = k_pages.shape
    out = np.full((nb_phys, Hkv, D), np.nan, dtype=np.float32)
    for b in range(len(ctx_lens)):
        ctx = int(ctx_lens[b])
        for n in range((ctx + bs - 1) // bs):
            blk = int(block_table[b, n])
            out[blk] = _block_sum(k_pages, blk, 0, min(bs, ctx - n * bs), dtype)
    return out


def append_block_sums(sums, k_pages, block_table, ctx_new, n_new, bs, dtype):
    """The sums after a commit appended n_new[b] positions ending at ctx_new[b]:
    positions t in [ctx_new - n_new, ctx_new), in order, are added to their
    block's sum; a block whose first position is among them starts from +0."""
    out = np.array(sums, dtype=np.float32, copy=True)
    for b in range(len(ctx_new)):
        t = int(ctx_new[b]) - int(n_new[b])
        while t < int(ctx_new[b]):
            n, off = divmod(t, bs)
            t1 = min((n + 1) * bs, int(ctx_new[b]))
            blk = int(block_table[b, n])
            out[blk] = _block_sum(k_pages, blk, off, off + (t1 - t), dtype,
                                  start=None if off == 0 else out[blk])
            t = t1
    return out


def means_from_sums(sums, block_table, ctx_lens, bs):
    """float32 [B, nmax, Hkv, D] as block_means, from kept block sums."""
    B = len(ctx_lens)
    Hkv, D = sums.shape[1], sums.shape[2]
    nb = [(int(c) + bs - 1) // bs for c in ctx_lens]
    nmax = max(nb + [0])
    out = np.full((B, nmax, Hkv, D), np.nan, dtype=np.float32)
    for b in range(B):
        ctx = int(ctx_lens[b])
        for n in range(nb[b]):
            out[b, n] = sums[int(block_table[b, n])] / np.float32(min(bs, ctx - n * bs))
    return out


def block_means(k_pages, block_table, ctx_lens, bs, dtype):
    """float32 [B, nmax, Hkv, D]; entries past a sequence's context blocks are NaN."""
    B = len(ctx_lens)
    Hkv, D = k_pages.shape[1], k_pages.shape[3]
    nb = [(int(c) + bs - 1) // bs for c in ctx_lens]
    nmax = max(nb + [0])
    out = np.full((B, nmax, Hkv, D), np.nan, dtype=np.float32)
    for b in range(B):
        ctx = int(ctx_lens[b])
        for n in range(nb[b]):
            blk = int(block_table[b, n])
            valid = min(bs, ctx - n * bs)
            s = np.zeros((Hkv, D), dtype=np.float32)
            for t in range(valid):
                s = s + decode_f32(k_pages[blk, :, t, :], dtype)
            out[b, n] = s / np.float32(valid)
    return out


def block_scores(qv, means):
    """qv: float32 [D]; means: float32 [n, D] -> float32 [n] via the halving tree."""
    p = np.asarray(qv, dtype=np.float32)[None, :] * np.asarray(means, dtype=np.float32)
    w = p.shape[1] // 2
    while w >= 1:
        p = p[:, :w] + p[:, w:2 * w]
        w //= 2
    return p[:, 0]


def select(scores, k):
    """Indices of the k best (score desc, index asc), ascending, padded with -1."""
    n = len(scores)
    order = np.lexsort((np.arange(n), -scores))
    keep = np.sort(order[:k])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(keep)] = keep
    return out


def topk_blocks(q, k_pages, block_table, ctx_lens, bs, k, dtype, means=None):
    """sel [B, T, Hq, k] int32."""
    B, T, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    if means is None:
        means = block_means(k_pages, block_table, ctx_lens, bs, dtype)
    sel = np.full((B, T, Hq, k), -1, dtype=np.int32)
    for b in range(B):
        nb = (int(ctx_lens[b]) + bs - 1) // bs
        for i in range(T):
            for h in range(Hq):
                if nb == 0:
                    continue
                sc = block_scores(decode_f32(q[b, i, h], dtype), means[b, :nb, h // G])
                sel[b, i, h] = select(sc, k)
    return sel


def pooled_query(q, b, g, G, dtype):
    """float32 [D]: the sequential sum of q[b, i, g*G + j] over i, then j."""
    D = q.shape[3]
    s = np.zeros(D, dtype=np.float32)
    for i in range(q.shape[1]):
        for j in range(G):
            s = s + decode_f32(q[b, i, g * G + j], dtype)
    return s


def topk_blocks_shared(q, k_pages, block_table, ctx_lens, bs, k, dtype, means=None):
    """sel [B, T, Hq, k] int32: one selection per (b, KV group), repeated for
    each of the group's rows."""
    B, T, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    if means is None:
        means = block_means(k_pages, block_table, ctx_lens, bs, dtype)
    sel = np.full((B, T, Hq, k), -1, dtype=np.int32)
    for b in range(B):
        nb = (int(ctx_lens[b]) + bs - 1) // bs
        if nb == 0:
            continue
        for g in range(Hkv):
            sc = block_scores(pooled_query(q, b, g, G, dtype), means[b, :nb, g])
            sel[b, :, g * G:(g + 1) * G] = select(sc, k)
    return sel
