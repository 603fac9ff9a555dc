"""Seeded generators for every buffer the verification pass reads.

Recipe (the same bytes feed the CPU oracle and the GPU library):

* every tensor draws from its own stream ``np.random.default_rng([seed, stream_id])``;
* normals are drawn in float32 and, for bf16 workloads, rounded once to bf16
  (round to nearest even) and kept as uint16 bit patterns;
* uniforms are ``integers(0, 2**24) * 2**-24``, exact float32 values in [0, 1);
* K and V pages are both laid out ``[num_blocks, Hkv, bs, D]``;
* tree node i's K/V sits at logical position ``ctx_b + i`` of sequence b;
* draft logits are ``rho * target + sqrt(1 - rho^2) * eps`` with ``eps`` drawn
  at the target's sigma, so the draft keeps the stated marginal and agrees
  with the target about as often as EasySpec's reported acceptance near 0.8;
* children in rejection-sampling workloads are drawn i.i.d. from the parent's
  draft distribution; greedy workloads take the draft argmax; the SpecExec
  workload builds its tree best-first from the draft's cumulative
  log-probabilities (SpecExec page, "Approach").

Nothing here performs verification arithmetic.
"""
from dataclasses import dataclass
import heapq
import math

import numpy as np

from .configs import Config

# Stream ids: one per tensor so that changing one size does not shift the others.
S_CTX, S_Q, S_K, S_V, S_TABLE, S_TREE, S_TARGET, S_NOISE, S_SAMPLE, S_UNIF, S_HOT, S_ROOT, \
    S_DRAFT = range(1, 14)


def _rng(cfg: Config, sid: int, *extra):
    return np.random.default_rng([cfg.seed, sid, *extra])


def f32_to_bf16_bits(x):
    """Round float32 values to bf16, nearest-even, returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normals(rng, shape, sigma, dtype, chunk=1 << 26):
    """float32 normals (times sigma), optionally rounded to bf16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[s:e] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return out.reshape(shape)


def as_float(a, dtype):
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


@dataclass
class Inputs:
    cfg: Config
    q: np.ndarray             # [B, T, Hq, D] float32 or bf16 bits
    k_pages: np.ndarray       # [num_blocks, Hkv, bs, D]
    v_pages: np.ndarray       # [num_blocks, Hkv, bs, D]
    block_table: np.ndarray   # int32 [B, max_blocks], -1 past each sequence's blocks
    ctx_lens: np.ndarray      # int32 [B]
    tree_parent: np.ndarray   # int32 [B, T], parent[0] = -1, parent[i] < i
    tree_token: np.ndarray    # int32 [B, T]
    target_logits: np.ndarray  # [B, T, V] float32 or bf16 bits
    draft_probs: object       # float32 [B, T, V] or None
    uniforms: np.ndarray      # float32 [B, T, 2]
    hot: np.ndarray           # int32 [B, hot_blocks] logical context blocks with scaled keys

    @property
    def num_blocks(self):
        return self.k_pages.shape[0]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]


def _random_tree(cfg: Config, rng):
    """Each new node picks its parent uniformly among earlier nodes whose depth is
    below the limit and whose child count is below the limit."""
    T = cfg.T
    parent = np.full(T, -1, dtype=np.int32)
    depth = np.zeros(T, dtype=np.int64)
    nchild = np.zeros(T, dtype=np.int64)
    for i in range(1, T):
        cand = np.nonzero((depth[:i] < cfg.max_parent_depth) & (nchild[:i] < cfg.max_children))[0]
        if cand.size == 0:
            raise ValueError("tree limits leave no parent for node %d" % i)
        p = int(cand[rng.integers(cand.size)])
        parent[i] = p
        depth[i] = depth[p] + 1
        nchild[p] += 1
    return parent


def _softmax_rows(x, tau):
    """Draft distribution (drafter side, input preparation only)."""
    z = x / tau
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _sssp_tree(cfg: Config, draft):
    """Best-first expansion of the cumulative draft log-probability (temperature 1):
    the tree holds the T most likely continuations (root included), ties broken by
    (parent, token) ascending; node ids follow insertion order."""
    T, V = draft.shape
    kmax = min(T - 1, V)

    def sorted_children(n):
        row = draft[n].astype(np.float64)
        lp = row - row.max()
        lp = lp - math.log(np.exp(lp).sum())
        if kmax < V:
            thr = np.partition(lp, V - kmax)[V - kmax]
            cand = np.nonzero(lp >= thr)[0]
        else:
            cand = np.arange(V)
        order = np.lexsort((cand, -lp[cand]))
        c = cand[order][:kmax]
        return c, lp[c]

    parent = np.full(T, -1, dtype=np.int32)
    token = np.zeros(T, dtype=np.int32)
    cum = np.zeros(T, dtype=np.float64)
    kids = {}
    ptr = {}
    heap = []

    def push_next(n):
        c, lp = kids[n]
        k = ptr[n]
        if k < len(c):
            heapq.heappush(heap, (-(cum[n] + lp[k]), n, int(c[k])))
            ptr[n] = k + 1

    kids[0] = sorted_children(0)
    ptr[0] = 0
    push_next(0)
    for n in range(1, T):
        negc, p, tok = heapq.heappop(heap)
        parent[n], token[n], cum[n] = p, tok, -negc
        push_next(p)
        kids[n] = sorted_children(n)
        ptr[n] = 0
        push_next(n)
    return parent, token


def make_inputs(cfg: Config) -> Inputs:
    B, T, Hq, Hkv, D, bs, V = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D, cfg.bs, cfg.V
    ctx = _rng(cfg, S_CTX).integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=B).astype(np.int32)

    # Paged cache: sequence b needs ceil((ctx_b + T) / bs) blocks.
    nblk = [(int(c) + T + bs - 1) // bs for c in ctx]
    num_blocks = int(sum(nblk))
    max_blocks = max(nblk)
    order = np.arange(num_blocks, dtype=np.int32)
    if cfg.shuffle_table:
        order = _rng(cfg, S_TABLE).permutation(num_blocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = order[off:off + nblk[b]]
        off += nblk[b]

    q = _normals(_rng(cfg, S_Q), (B, T, Hq, D), 1.0, cfg.dtype)
    if cfg.hot_blocks:
        hot = np.zeros((B, cfg.hot_blocks), dtype=np.int32)
        r = _rng(cfg, S_HOT)
        for b in range(B):
            nctx = (int(ctx[b]) + bs - 1) // bs
            hot[b] = np.sort(r.choice(nctx, size=cfg.hot_blocks, replace=False))
        kf = _normals(_rng(cfg, S_K), (num_blocks, Hkv, bs, D), 1.0, "f32")
        for b in range(B):
            kf[table[b, hot[b]]] *= np.float32(cfg.hot_scale)
        k_pages = f32_to_bf16_bits(kf) if cfg.dtype == "bf16" else kf
        del kf
    else:
        hot = np.zeros((B, 0), dtype=np.int32)
        k_pages = _normals(_rng(cfg, S_K), (num_blocks, Hkv, bs, D), 1.0, cfg.dtype)
    v_pages = _normals(_rng(cfg, S_V), (num_blocks, Hkv, bs, D), 1.0, cfg.dtype)

    parent = np.full((B, T), -1, dtype=np.int32)
    token = np.zeros((B, T), dtype=np.int32)
    draft_probs = None
    root_tok = _rng(cfg, S_ROOT).integers(0, V, size=B)
    a = math.sqrt(1.0 - cfg.rho * cfg.rho)
    if cfg.tree == "sssp":
        if B != 1:
            raise ValueError("best-first trees are built for one sequence")
        draft = _normals(_rng(cfg, S_DRAFT), (T, V), cfg.logit_sigma, "f32")
        p, tk = _sssp_tree(cfg, draft)
        parent[0], token[0] = p, tk
        token[0, 0] = root_tok[0]
        noise = _normals(_rng(cfg, S_NOISE), (T, V), cfg.logit_sigma, "f32")
        tgt = (cfg.rho * draft.astype(np.float64) + a * noise).astype(np.float32)
        target = (f32_to_bf16_bits(tgt) if cfg.logit_dtype == "bf16" else tgt)[None]
    else:
        target = _normals(_rng(cfg, S_TARGET), (B, T, V), cfg.logit_sigma, cfg.logit_dtype)
        tree_rng = _rng(cfg, S_TREE)
        noise_rng = _rng(cfg, S_NOISE)
        samp_rng = _rng(cfg, S_SAMPLE)
        if cfg.mode == "mss":
            draft_probs = np.empty((B, T, V), dtype=np.float32)
        for b in range(B):
            if cfg.tree == "chain":
                parent[b] = np.arange(-1, T - 1, dtype=np.int32)
            else:
                parent[b] = _random_tree(cfg, tree_rng)
            token[b, 0] = root_tok[b]
            tf = as_float(target[b], cfg.logit_dtype).astype(np.float64)
            eps = noise_rng.standard_normal((T, V), dtype=np.float32).astype(np.float64)
            dl = cfg.rho * tf + a * cfg.logit_sigma * eps
            if cfg.mode == "mss":
                qd = _softmax_rows(dl, cfg.temperature).astype(np.float32)
                draft_probs[b] = qd
                cdf = np.cumsum(qd.astype(np.float64), axis=-1)
                for i in range(1, T):
                    u = samp_rng.random() * cdf[parent[b, i], -1]
                    token[b, i] = min(int(np.searchsorted(cdf[parent[b, i]], u, side="right")), V - 1)
            else:
                am = np.argmax(dl, axis=-1)
                for i in range(1, T):
                    token[b, i] = am[parent[b, i]]
    unif = (_rng(cfg, S_UNIF).integers(0, 1 << 24, size=(B, T, 2)).astype(np.float64)
            * 2.0 ** -24).astype(np.float32)
    return Inputs(cfg=cfg, q=q, k_pages=k_pages, v_pages=v_pages, block_table=table,
                  ctx_lens=ctx, tree_parent=parent, tree_token=token, target_logits=target,
                  draft_probs=draft_probs, uniforms=unif, hot=hot)
