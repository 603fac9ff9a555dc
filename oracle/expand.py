"""One batched expansion step of the draft-tree search (TEST INFRASTRUCTURE).

The SpecExec page ("Approach") builds the draft tree deterministically from
the continuations of highest cumulative probability, by a parallel (batched)
shortest-path search with the draft model: each step runs the draft model on
a batch of tree nodes, and every token x after an expanded node e becomes a
candidate child whose cumulative log-probability is the node's plus the
draft's log-probability of x there.  The step keeps the best candidates.

Reading (the page gives no formula): the draft's log-probability at node e is
log_softmax(l_e / tau)[x] of the node's draft logits at temperature tau > 0;
the step keeps the k candidates of largest cumulative log-probability,
ordered by it, descending, with ties going to the smaller (e, x).  Everything
around the step (the draft model, where the kept children are inserted,
which nodes the next step expands) is outside this function.
"""
import numpy as np

from .codec import decode


def expand(draft_logits, logit_dtype, cum_logp, tau, k):
    """draft_logits [E, V] (stored dtype), cum_logp [E] -> (row int32 [k],
    token int32 [k], score float64 [k]), best first."""
    l = decode(draft_logits, logit_dtype) / float(tau)
    E, V = l.shape
    m = l.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(l - m).sum(axis=1))
    score = np.asarray(cum_logp, np.float64)[:, None] + l - lse[:, None]
    flat = score.ravel()
    # descending score, then ascending flat index (e * V + x): a stable sort of -score
    order = np.argsort(-flat, kind="stable")[:k]
    return (order // V).astype(np.int32), (order % V).astype(np.int32), flat[order]
