"""Test-side helpers: building small paged caches by hand and decoding outputs."""
import itertools

import numpy as np


def paged_from_dense(Kd, Vd, bs, rng=None, spare=0):
    """Kd, Vd: [B, Hkv, n, D] float arrays (same n for all sequences).
    Returns k_pages [nb, Hkv, bs, D], v_pages [nb, Hkv, bs, D], block_table [B, per]
    with blocks optionally shuffled.  ``spare`` extra random blocks are appended."""
    B, Hkv, n, D = Kd.shape
    per = (n + bs - 1) // bs
    nb = B * per + spare
    phys = np.arange(nb)
    if rng is not None:
        phys = rng.permutation(nb)
    kp = np.zeros((nb, Hkv, bs, D), dtype=Kd.dtype)
    vp = np.zeros((nb, Hkv, bs, D), dtype=Vd.dtype)
    if rng is not None:
        kp[:] = rng.standard_normal(kp.shape)
        vp[:] = rng.standard_normal(vp.shape)
    table = np.zeros((B, per), dtype=np.int32)
    for b in range(B):
        for j in range(per):
            blk = int(phys[b * per + j])
            table[b, j] = blk
            lo, hi = j * bs, min(n, (j + 1) * bs)
            kp[blk, :, :hi - lo, :] = Kd[b, :, lo:hi, :]
            vp[blk, :, :hi - lo, :] = Vd[b, :, lo:hi, :]
    return kp, vp, table


def all_trees(T):
    """Every parent array with parent[0] = -1 and 0 <= parent[i] < i."""
    for choice in itertools.product(*[range(i) for i in range(1, T)]):
        yield np.array((-1,) + choice, dtype=np.int32)


def path_by_walk(parent, i):
    out = [i]
    while parent[out[-1]] >= 0:
        out.append(int(parent[out[-1]]))
    return out[::-1]
