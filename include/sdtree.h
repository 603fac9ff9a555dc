/*
 * sdtree.h -- tree verification for speculative decoding on MI355X (gfx950).
 *
 * The verification pass of speculative decoding (SpecExec page, "Approach":
 * the whole draft tree is verified in one target pass; EasySpec page, "+tree"
 * baseline; sparse-verification page, "Methodology") as four calls:
 *
 *   sd_tree_verify_attn  every draft-tree node attends to the committed context
 *                        plus its own ancestors, grouped-query heads, paged KV;
 *   sd_accept            the acceptance walk (greedy, rejection sampling, or
 *                        sampling from the target at each node);
 *   sd_kv_commit         the accepted root path becomes committed context;
 *   sd_accept_commit     sd_accept then sd_kv_commit, in one launch;
 *   sd_accept_commit_noalloc  the same without a workspace argument, for
 *                        callers that cannot allocate;
 *   sd_topk_blocks       top-k KV blocks per query for sparse verification;
 *   sd_block_sums, sd_block_sums_append, sd_topk_blocks_cached
 *                        the same selection from per-block key sums kept as
 *                        the context grows;
 *   sd_tree_expand       one batched expansion step of the draft-tree search;
 *   sd_tree_build        the whole best-first draft-tree search to a budget.
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory.  Scratch comes from a caller
 *     workspace `ws` of at least sd_workspace_bytes(...) bytes, zero-filled
 *     once by the caller before its first use (the library leaves it reusable);
 *     the one exception, sd_accept_commit_noalloc, uses a fixed device array
 *     of the library instead.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream)
 *     and return an sd_status.  Argument and shape errors are detected on the
 *     host before anything is launched; then nothing is launched.
 *   - Data-dependent errors (a bad parent index, a block id out of range, a
 *     context that does not fit the block table) set a sticky bit in the
 *     workspace status word and the affected unit is skipped;
 *     sd_device_status reads (and clears) it.
 *   - No exceptions, aborts or printing.  One workspace must not be used by two
 *     calls that may run concurrently, and a workspace serves one call kind:
 *     sd_accept keeps barrier counters in its workspace that must read zero
 *     when a call starts (every call leaves them at zero).
 *
 * Layouts (row-major, innermost last)
 *   q, out        [B, T, Hq, D]                 element type `dtype`
 *   k_pages       [num_blocks, Hkv, bs, D]      element type `dtype`
 *   v_pages       [num_blocks, Hkv, bs, D]      element type `dtype` (as k_pages)
 *   block_table   int32 [B, max_blocks]         logical block -> physical block
 *   ctx_lens      int32 [B]                     committed context length
 *   tree_parent   int32 [B or 1, T]             parent[0] = -1, 0 <= parent[i] < i
 *   tree_token    int32 [B or 1, T]
 *   Logical position p of sequence b lives in block block_table[b][p / bs] at
 *   offset p % bs.  Tree node i's K/V must already sit at position ctx_b + i
 *   (the caller writes it there), so the table must cover ctx_b + T positions.
 *   Query head h reads KV head h / (Hq / Hkv).
 */
#ifndef SDTREE_H
#define SDTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sd_status {
  SD_OK = 0,
  SD_INVALID_ARG = 1,        /* null pointer, bad scalar (k <= 0, temperature < 0, ...) */
  SD_BAD_SHAPE = 2,          /* inconsistent sizes (Hq % Hkv != 0, T < 1, ...) */
  SD_BAD_DTYPE = 3,          /* element type code not supported by the call */
  SD_UNSUPPORTED = 4,        /* valid but outside what the kernels handle (D not 64/128, T > 4096) */
  SD_CAPACITY = 5,           /* workspace smaller than sd_workspace_bytes() */
  SD_HIP_ERROR = 6,          /* a HIP runtime call failed */
  SD_DEVICE_DATA_ERROR = 7   /* returned by sd_device_status when a sticky bit is set */
} sd_status;

typedef enum sd_dtype { SD_F32 = 0, SD_BF16 = 1 } sd_dtype;

/* Sticky bits of the workspace status word. */
#define SD_ERR_PARENT     0x1u   /* parent[i] not in [-1, i) (attention) or not in [0, i) (accept) */
#define SD_ERR_BLOCK      0x2u   /* block_table entry outside [0, num_blocks) */
#define SD_ERR_CAPACITY   0x4u   /* ctx_b + T exceeds max_blocks * bs, or ctx_b < 0 */
#define SD_ERR_TOKEN      0x8u   /* tree token outside [0, V) */
#define SD_ERR_SELECTION  0x10u  /* sel_blocks entry not a context block / not ascending */
#define SD_ERR_BUILD      0x40u  /* sd_tree_build: a round's float32 pre-selection missed a candidate
                                    (more than its margin within float32 rounding of the cut) */
#define SD_ERR_TIMEOUT    0x20u  /* a cross-workgroup wait gave up; results of the call are invalid
                                    and the workspace must be zero-filled again */
#define SD_ERR_DEBUG      0x80u  /* debug build (libsdtree_debug.so) only: a device-side
                                    consistency check between a launch's plan and its kernel
                                    failed; the call's results are invalid */

typedef struct sd_shape {
  int32_t B;            /* sequences */
  int32_t T;            /* tree nodes including the root (node 0) */
  int32_t Hq;           /* query heads */
  int32_t Hkv;          /* KV heads; Hq % Hkv == 0 */
  int32_t D;            /* head dim: 64 or 128 */
  int32_t bs;           /* tokens per KV block: a power of two >= 8 */
  int32_t max_blocks;   /* columns of block_table */
  int32_t num_blocks;   /* blocks in k_pages / v_pages */
  int32_t dtype;        /* sd_dtype of q, k_pages, v_pages, out */
  int32_t tree_stride;  /* 0: one tree shared by all sequences, T: one tree per sequence */
  float scale;          /* softmax scale; 0 means 1/sqrt(D) */
} sd_shape;

typedef struct sd_accept_shape {
  int32_t B;            /* sequences */
  int32_t T;            /* tree nodes including the root */
  int32_t V;            /* vocabulary */
  int32_t logit_dtype;  /* sd_dtype of target_logits */
  int32_t tree_stride;  /* 0 or T, as in sd_shape */
} sd_accept_shape;

typedef struct sd_expand_shape {
  int32_t E;            /* expanded nodes (rows of draft logits) */
  int32_t V;            /* vocabulary */
  int32_t logit_dtype;  /* sd_dtype of draft_logits */
} sd_expand_shape;

/* Shape of a draft-tree build: T nodes (the budget, root included), a drafter
   logits table of T rows of V. */
typedef struct sd_build_shape {
  int32_t T;
  int32_t V;
  int32_t logit_dtype;  /* SD_F32 or SD_BF16 */
} sd_build_shape;

enum { SD_CALL_ATTN = 1, SD_CALL_ACCEPT = 2, SD_CALL_TOPK = 3, SD_CALL_COMMIT = 4, SD_CALL_BLOCK_SUMS = 5,
       SD_CALL_EXPAND = 6, SD_CALL_BUILD = 7 };

/*
 * Tree-masked grouped-query attention over the paged cache.
 * For every (b, i, h): out = softmax(scale * q . K^T) V over the keys at
 * positions {p < ctx_b} U {ctx_b + j : j is i or an ancestor of i}
 * (SpecExec page, "Approach"; EasySpec page, "+tree").
 *   sel_blocks  NULL for dense attention, else int32 [B, T, Hq, k_sel]: the
 *               context blocks each query keeps, ascending, -1 padded at the
 *               end (sparse-verification page, "Methodology": top-k blocks per
 *               query); tree ancestors are always attended.
 *   k_sel       0 for dense attention, else 1 .. 65536 (SD_UNSUPPORTED above:
 *               a wider list is padding, since it cannot hold more distinct
 *               blocks than the context has).
 *   out         written in `dtype`.
 *   ws          >= sd_workspace_bytes(SD_CALL_ATTN, shape, k_sel).
 */
sd_status sd_tree_verify_attn(const sd_shape* shape, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* block_table,
                              const int32_t* ctx_lens, const int32_t* tree_parent,
                              const int32_t* sel_blocks, int32_t k_sel, void* out, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Acceptance walk from the root (SpecExec page, "Approach" and "Builds on";
 * EasySpec page, "Approach").  The rule follows the arguments:
 *   temperature == 0                    greedy: follow the target argmax
 *                                       (lowest id on ties) while a child
 *                                       carries it (lowest node index first);
 *   temperature > 0, draft_probs given  rejection sampling: siblings in
 *                                       ascending index, child c with token x
 *                                       accepted when u[c][0]*q(x) < r(x); on
 *                                       rejection r <- normalise(max(r-q, 0));
 *   temperature > 0, draft_probs NULL   sample x from softmax(l / temperature)
 *                                       with u[cur][1]; descend into the child
 *                                       carrying x, else stop.
 *   target_logits  [B, T, V] in logit_dtype; draft_probs float32 [B, T, V].
 *   uniforms       float32 [B, T, 2] in [0, 1); may be NULL when temperature == 0.
 *   path           int32 [B, T]: accepted nodes from the root, -1 padded.
 *   path_len       int32 [B]: accepted drafts + 1.   bonus  int32 [B]: next root token.
 *   ws             >= sd_workspace_bytes(SD_CALL_ACCEPT, shape, 0).
 */
sd_status sd_accept(const sd_accept_shape* shape, const void* target_logits,
                    const float* draft_probs, const int32_t* tree_parent,
                    const int32_t* tree_token, const float* uniforms, float temperature,
                    int32_t* path, int32_t* path_len, int32_t* bonus, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * Commit the accepted path (SpecExec page, "Approach": the tokens the walk
 * accepts become committed context for the next verification pass; the
 * accepted root path is compacted into the slots right after the context):
 * for j < path_len[b], position ctx_b + j takes the
 * K/V of position ctx_b + path[b][j] (every KV head), then ctx_lens[b] +=
 * path_len[b].  In place; path must be increasing with path[b][0] == 0 (as
 * sd_accept produces), which makes the in-place copy safe.  k_pages, v_pages
 * and ctx_lens are modified.
 *   block_sums  float32 [num_blocks, Hkv, D] or NULL: kept block key sums
 *               (sd_block_sums), current for the old lengths; the commit then
 *               extends them over the committed positions exactly as
 *               sd_block_sums_append would (sparse-verification page,
 *               "Methodology": the blocks' summaries are maintained as the
 *               context grows, so selection never reads K).  A sequence whose path or table fails validation
 * is left untouched and a sticky bit is set in ws (>= sd_workspace_bytes(
 * SD_CALL_COMMIT, shape, 0) bytes: the status word and one completion counter
 * per sequence, which every call leaves at zero).
 *   path      int32 [B, T] as produced by sd_accept; path_len int32 [B].
 */
sd_status sd_kv_commit(const sd_shape* shape, void* k_pages, void* v_pages,
                       const int32_t* block_table, int32_t* ctx_lens, float* block_sums,
                       const int32_t* path, const int32_t* path_len, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * sd_accept followed by sd_kv_commit of the accepted paths, in one launch:
 * the acceptance kernel commits each sequence's path once its walk has ended,
 * so the path never leaves the device between the two steps.  Results are
 * those of the two calls in sequence: path, path_len and bonus as sd_accept;
 * k_pages, v_pages and ctx_lens as sd_kv_commit given that path.  Arguments
 * are those of the two calls; `kv_shape` describes the paged cache and is
 * checked as for sd_kv_commit, and its B and T must equal `shape`'s.  Data
 * errors of either half set their sticky bits in `ws`
 * (>= sd_workspace_bytes(SD_CALL_ACCEPT, shape, 0)); a sequence whose tree
 * fails validation gets path_len 0 and commits nothing, and one whose slots
 * [ctx, ctx + T) fail the commit's checks keeps its cache and length.
 * block_sums (may be NULL) as for sd_kv_commit: extended in the same launch.
 */
sd_status sd_accept_commit(const sd_accept_shape* shape, const sd_shape* kv_shape,
                           const void* target_logits, const float* draft_probs,
                           const int32_t* tree_parent, const int32_t* tree_token,
                           const float* uniforms, float temperature, int32_t* path,
                           int32_t* path_len, int32_t* bonus, void* k_pages, void* v_pages,
                           const int32_t* block_table, int32_t* ctx_lens, float* block_sums,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * sd_accept_commit for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as sd_accept_commit,
 * except that there is no workspace: the acceptance walk's cross-workgroup
 * exchange slots live in a device array of the library (1 MiB, one copy per
 * GPU, held until the process ends), and the sticky error bits go to
 * `status`, a caller-owned device word (OR-ed into; read and clear it with
 * sd_device_status(status, stream, &bits)).
 *   Limit: when a sequence is walked by several workgroups (up to 16, while
 *   B * 16 <= 256 and V > 2048), at most 128 sequences per call; a larger
 *   call returns SD_CAPACITY before launching anything.
 *   The call allocates nothing (no hipMalloc, no library allocation); it
 *   clears the slots it uses with a small kernel before the walk.
 *   Concurrency: every call on one GPU shares that GPU's slots, so two calls
 *   that may overlap on one GPU (different streams, no ordering) race and
 *   must not be issued; calls ordered on one stream are fine.
 */
sd_status sd_accept_commit_noalloc(const sd_accept_shape* shape, const sd_shape* kv_shape,
                                   const void* target_logits, const float* draft_probs,
                                   const int32_t* tree_parent, const int32_t* tree_token,
                                   const float* uniforms, float temperature, int32_t* path,
                                   int32_t* path_len, int32_t* bonus, void* k_pages,
                                   void* v_pages, const int32_t* block_table, int32_t* ctx_lens,
                                   float* block_sums, uint32_t* status, void* stream);

/*
 * Top-k context blocks per query (sparse-verification page, "Methodology":
 * keep the top-k key/value blocks per query by a cheap relevance score).
 * Score of block n for query (b, i, h) = q . mean of the block's valid keys,
 * computed in float32 in a fixed order (sequential token sum, one division,
 * products, halving-tree sum over D).  Candidates: n < ceil(ctx_b / bs).
 * Keeps the k best (score descending, lower index first on ties).
 *   sel_blocks  int32 [B, T, Hq, k]: ascending, -1 padded.
 *   ws          >= sd_workspace_bytes(SD_CALL_TOPK, shape, k).
 */
sd_status sd_topk_blocks(const sd_shape* shape, const void* q, const void* k_pages,
                         const int32_t* block_table, const int32_t* ctx_lens, int32_t k,
                         int32_t* sel_blocks, void* ws, size_t ws_bytes, void* stream);

/*
 * Kept block key sums, so that top-k need not read K on every call (the
 * sparse-verification page, "Methodology": the relevance score uses the
 * mean-pooled key of each block; keeping the per-block sums as the context
 * grows gives the same means without a scan of K).
 *   block_sums  float32 [num_blocks, Hkv, D], indexed by PHYSICAL block; owned
 *               by the caller.  A physical block shared by several sequences
 *               must be a whole block in each.
 * sd_block_sums: for every context block n < ceil(ctx_b / bs) of every
 *   sequence, block_sums[block_table[b][n]][g][:] = the float32 sum of its valid
 *   K rows, sequential in position order from +0.  Other entries are not
 *   written.  ws >= sd_workspace_bytes(SD_CALL_BLOCK_SUMS, shape, 0).
 * sd_block_sums_append: after a commit (ctx_lens already advanced), adds the
 *   K rows of positions [ctx_b - n_new[b], ctx_b) to their blocks' sums in
 *   position order; a block whose first position is among them starts from
 *   +0.  With n_new = the commit's path_len, the sums stay equal to
 *   sd_block_sums at the new lengths, bit for bit.  n_new[b] must lie in
 *   [0, ctx_b]; a sequence with a bad count or a touched block out of range
 *   is left unchanged and a sticky bit is set.
 * sd_topk_blocks_cached: sd_topk_blocks with each mean formed as the kept sum
 *   divided by the valid count (one IEEE division), so the selection is that
 *   of sd_topk_blocks bit for bit while the sums are current.  K is not read.
 *   ws >= sd_workspace_bytes(SD_CALL_TOPK, shape, k).
 */
sd_status sd_block_sums(const sd_shape* shape, const void* k_pages, const int32_t* block_table,
                        const int32_t* ctx_lens, float* block_sums, void* ws, size_t ws_bytes,
                        void* stream);
sd_status sd_block_sums_append(const sd_shape* shape, const void* k_pages,
                               const int32_t* block_table, const int32_t* ctx_lens,
                               const int32_t* n_new, float* block_sums, void* ws, size_t ws_bytes,
                               void* stream);
sd_status sd_topk_blocks_cached(const sd_shape* shape, const void* q, const float* block_sums,
                                const int32_t* block_table, const int32_t* ctx_lens, int32_t k,
                                int32_t* sel_blocks, void* ws, size_t ws_bytes, void* stream);

/*
 * One selection per (sequence, KV group), reused by every tree node and every
 * query head of the group (sparse-verification page, "Methodology": reuse
 * across draft tokens).  The group's score of block n is the sum of its rows'
 * scores, formed as (pooled query) . mean: the pooled query is the float32
 * sum from +0 of q[b, i, g*G + j] over i, then j, sequentially; the mean,
 * the dot product and the order are those of sd_topk_blocks.  Means come
 * from block_sums when it is not NULL (as sd_topk_blocks_cached; k_pages is
 * then not read), else from K.
 *   sel_blocks  int32 [B, T, Hq, k]: each group's list in all its rows, so
 *               sparse attention reads k blocks per (sequence, KV head).
 *   ws          >= sd_workspace_bytes(SD_CALL_TOPK, shape, k).
 */
sd_status sd_topk_blocks_shared(const sd_shape* shape, const void* q, const void* k_pages,
                                const float* block_sums, const int32_t* block_table,
                                const int32_t* ctx_lens, int32_t k, int32_t* sel_blocks, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * One batched expansion step of the draft-tree search (SpecExec page,
 * "Approach": the draft tree is grown from the continuations of highest
 * cumulative probability by a batched shortest-path search with the draft
 * model).  Every token x after expanded node e is a candidate child scored
 *   s(e, x) = cum_logp[e] + log_softmax(draft_logits[e] / temperature)[x]
 * in float32; the k best are written best first (ties to the smaller
 * e * V + x):
 *   draft_logits  [E, V] in logit_dtype;  cum_logp  float32 [E];
 *   out_row int32 [k] (index of e), out_token int32 [k], out_score float32 [k].
 * 1 <= k <= min(4096, E * V); temperature > 0; E * V < 2^32 - 1.
 * ws >= sd_workspace_bytes(SD_CALL_EXPAND, shape, k), zero-filled before
 * its first use (every call leaves it reusable, also for calls of another
 * shape that fit in it).  The draft model, and which
 * kept children are inserted or expanded next, stay with the caller.
 */
sd_status sd_tree_expand(const sd_expand_shape* shape, const void* draft_logits,
                         const float* cum_logp, float temperature, int32_t k, int32_t* out_row,
                         int32_t* out_token, float* out_score, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * The draft-tree search to a budget (SpecExec page, "Approach": the tree is
 * built deterministically from the continuations of highest cumulative
 * probability by a parallel shortest-path search with the drafter).  Node
 * ids follow the order a sequential best-first search would take the nodes:
 * after ids 0 .. n - 1 the next node is the best child of those nodes not
 * yet taken, by (cumulative log-probability descending, parent id, token),
 * where the log-probability of token x after node e is
 * log_softmax(draft_logits[e] / temperature)[x] in float64 and the root has
 * cumulative log-probability 0.  Row n of draft_logits is the drafter's
 * output at the node that receives id n (the caller's drafter fills rows in
 * that order).
 *   The search runs in rounds that each take the longest prefix of the next
 *   candidates that the sequential search would take in a row (see
 *   csrc/build.hip); a round selects candidates in float32 with a margin of
 *   256 and orders them in float64.  The call waits on `stream` once per
 *   round (it reads the node count back) and returns when the tree is full.
 *   draft_logits  [T, V] in logit_dtype (finite values).
 *   parent, token int32 [T]: parent[0] = -1, token[0] = root_token;
 *                 0 <= parent[i] < i.   cum_logp  float64 [T].
 *   rounds        host pointer, may be NULL: the number of rounds run.
 *   Limits: 1 <= T <= 3841 (T - 1 + 256 candidates per round at most 4096),
 *   T * V < 2^32, temperature > 0, 0 <= root_token < V.  A round whose
 *   pre-selection missed a candidate stops the build and sets SD_ERR_BUILD.
 *   ws >= sd_workspace_bytes(SD_CALL_BUILD, shape, 0), zero-filled before its
 *   first use.
 */
sd_status sd_tree_build(const sd_build_shape* shape, const void* draft_logits, float temperature,
                        int32_t root_token, int32_t* parent, int32_t* token, double* cum_logp,
                        int32_t* rounds, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes a call needs; `shape` points to an sd_shape (ATTN, TOPK,
 * COMMIT, BLOCK_SUMS), an sd_accept_shape (ACCEPT, also for
 * sd_accept_commit), an sd_expand_shape (EXPAND) or an sd_build_shape
 * (BUILD); `extra` is k_sel (ATTN, 0 = dense) or k (TOPK, EXPAND).  0 on bad
 * input. */
size_t sd_workspace_bytes(int32_t call_id, const void* shape, int32_t extra);

/* Synchronises `stream`, reads the sticky bits into *bits (may be NULL), clears
 * them, and returns SD_DEVICE_DATA_ERROR if any was set. */
sd_status sd_device_status(void* ws, void* stream, uint32_t* bits);

/* Kernel timing for profilers and benchmarks (not part of the method): the
 * next sd_tree_verify_attn call made on this host thread launches its first
 * kernel so that it records `start_event` when that kernel begins, and its
 * last kernel so that it records `stop_event` when that kernel ends
 * (hipExtLaunchKernelGGL).  hipEventElapsedTime(start, stop) is then the
 * call's own device time, without the idle gap that an event recorded on the
 * stream around the call adds.  Both are hipEvent_t handles created with
 * timing enabled (either may be NULL: not recorded).  The setting is used by
 * that one call, also when it fails, and then cleared; NULL, NULL clears it.
 * Returns SD_OK. */
sd_status sd_attn_timing_events(void* start_event, void* stop_event);

/* Static description of a status code. */
const char* sd_status_str(int32_t code);

#ifdef __cplusplus
}
#endif
#endif /* SDTREE_H */
