"""The five verification workloads, with every unstated field made explicit.

Shapes follow the speculative-decoding pages: SpecExec's budget-2048 draft
trees built by best-first expansion (SpecExec page, "Approach" and "Key
results"), EasySpec's temperature 0.8 and acceptance near 0.8 (EasySpec page,
"Key results"), and long inputs for sparse verification (sparse-verification
page, "Practical Implications").  Head shapes are those of Llama-3-8B
(32 query / 8 KV heads) and Llama-2-70B (64 / 8), head dim 128.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    B: int                 # sequences
    Hq: int                # query heads
    Hkv: int               # KV heads
    D: int                 # head dim
    dtype: str             # 'f32' or 'bf16' for q / K / V / out
    ctx_lo: int            # committed context length: uniform integer in [ctx_lo, ctx_hi]
    ctx_hi: int
    bs: int                # tokens per KV block (page)
    tree: str              # 'chain' | 'random' | 'sssp'
    T: int                 # tree nodes including the root (node 0)
    max_parent_depth: int  # random trees: a parent must have depth < this
    max_children: int      # random trees: a parent must have fewer children than this
    V: int                 # vocabulary
    logit_dtype: str       # 'f32' or 'bf16'
    logit_sigma: float     # target logits ~ N(0, sigma^2)
    mode: str              # 'greedy' | 'mss' | 'exec'
    temperature: float
    shuffle_table: bool
    topk: int = 0          # > 0: sparse verification keeps this many blocks per query
    hot_blocks: int = 0    # blocks per sequence whose keys are scaled by hot_scale
    hot_scale: float = 5.0
    rho: float = 0.99      # correlation of draft logits with target logits
    seed: int = 0

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def M(self):
        return self.T * self.G


CONFIGS = {
    # Tiny chain verify.
    "tiny_chain": Config(
        name="tiny_chain", B=1, Hq=2, Hkv=2, D=64, dtype="f32", ctx_lo=256, ctx_hi=256,
        bs=256, tree="chain", T=5, max_parent_depth=0, max_children=0, V=1024,
        logit_dtype="f32", logit_sigma=2.0, mode="greedy", temperature=0.0,
        shuffle_table=False),
    # Llama-3-8B-shaped layer, 64-node random tree, rejection sampling at 0.8.
    "llama3_8b_tree64": Config(
        name="llama3_8b_tree64", B=16, Hq=32, Hkv=8, D=128, dtype="bf16", ctx_lo=4096,
        ctx_hi=4096, bs=16, tree="random", T=64, max_parent_depth=8, max_children=4,
        V=128256, logit_dtype="bf16", logit_sigma=3.0, mode="mss", temperature=0.8,
        shuffle_table=False),
    # SpecExec-scale tree on a Llama-2-70B-shaped layer.
    "specexec_70b_tree2048": Config(
        name="specexec_70b_tree2048", B=1, Hq=64, Hkv=8, D=128, dtype="bf16", ctx_lo=2048,
        ctx_hi=2048, bs=16, tree="sssp", T=2048, max_parent_depth=0, max_children=0,
        V=32000, logit_dtype="bf16", logit_sigma=3.0, mode="exec", temperature=0.6,
        shuffle_table=False),
    # Long-context paged verify with a shuffled block table.
    "longctx_paged_tree16": Config(
        name="longctx_paged_tree16", B=8, Hq=64, Hkv=8, D=128, dtype="bf16", ctx_lo=16384,
        ctx_hi=32768, bs=16, tree="random", T=16, max_parent_depth=6, max_children=2,
        V=128256, logit_dtype="bf16", logit_sigma=3.0, mode="mss", temperature=1.0,
        shuffle_table=True),
    # Sparse verification: top-32 blocks of 64 tokens out of a 65536 context.
    "sparse_topk32_ctx64k": Config(
        name="sparse_topk32_ctx64k", B=4, Hq=32, Hkv=8, D=128, dtype="bf16", ctx_lo=65536,
        ctx_hi=65536, bs=64, tree="chain", T=8, max_parent_depth=0, max_children=0,
        V=128256, logit_dtype="bf16", logit_sigma=3.0, mode="greedy", temperature=0.0,
        shuffle_table=False, topk=32, hot_blocks=16),
}

CONFIG_ORDER = ["tiny_chain", "llama3_8b_tree64", "specexec_70b_tree2048",
                "longctx_paged_tree16", "sparse_topk32_ctx64k"]


def small_variant(name, **over):
    """Same structure as a named workload, at a size the oracle finishes in
    seconds, with ragged context lengths so that tiles end part-way."""
    c = CONFIGS[name]
    small = {
        "tiny_chain": dict(),
        "llama3_8b_tree64": dict(B=3, ctx_lo=130, ctx_hi=301, V=4099),
        "specexec_70b_tree2048": dict(T=160, ctx_lo=200, ctx_hi=200, V=700),
        "longctx_paged_tree16": dict(B=3, ctx_lo=500, ctx_hi=900, V=3001),
        "sparse_topk32_ctx64k": dict(B=2, ctx_lo=1000, ctx_hi=1500, topk=6, hot_blocks=3,
                                     V=2053),
    }[name]
    small.update(over)
    return replace(c, name=c.name + "_small", **small)
