"""The draft-tree search to a budget (TEST INFRASTRUCTURE).

The SpecExec page ("Approach") builds the draft tree deterministically from
the continuations of highest cumulative probability: a shortest-path search
over the tree of continuations, where a node's cost is minus its cumulative
draft log-probability.  Written here as the plain sequential best-first
search:

* the root (id 0) has cumulative log-probability 0;
* the log-probability of token x after node e is log_softmax(l_e / tau)[x] in
  float64, where l_e is the drafter's logits row for node e;
* after ids 0 .. n - 1 are taken, id n goes to the best child of those nodes
  not taken yet, by (cumulative log-probability descending, parent id
  ascending, token ascending);
* this repeats until the tree holds T nodes.

Reading (the page gives no formula): the drafter's row for a node is row n of
a table, n being the id the node receives, so the table is filled in the
order the search takes nodes (a drafter run on each new node as it is taken);
temperature divides the logits; ties as above.

Pins (tests/test_oracle_build.py): the result is characterised by properties
checked there independently of this code -- parents precede children,
cumulative log-probabilities add up along each edge (scipy's log_softmax),
ids are in strictly increasing (score, parent, token) order, and every child
of a taken node that was not taken scores below the last node taken -- which
together leave exactly one tree; plus a two-token closed form.
"""
import numpy as np

from .codec import decode


def log_softmax_rows(draft_logits, logit_dtype, tau):
    """float64 log_softmax(l / tau) of every row: (z - max) - log(sum exp(z - max))."""
    z = decode(draft_logits, logit_dtype) / float(tau)
    m = z.max(axis=1, keepdims=True)
    d = z - m
    return d - np.log(np.exp(d).sum(axis=1, keepdims=True))


def build_tree(draft_logits, logit_dtype, tau, T, root_token=0):
    """Returns (parent int32 [T], token int32 [T], cum float64 [T])."""
    lp = log_softmax_rows(np.asarray(draft_logits)[:T], logit_dtype, tau)
    V = lp.shape[1]
    keep = min(max(T - 1, 1), V)     # no node can have more children than T - 1
    parent = np.full(T, -1, np.int32)
    token = np.zeros(T, np.int32)
    cum = np.zeros(T)
    token[0] = root_token
    kids = []          # per taken node: its children, best first
    nxt = []           # per taken node: index of its best child not yet taken

    def children(e):
        row = lp[e]
        if keep < V:
            idx = np.argpartition(-row, keep - 1)[:keep]
            cut = row[idx].min()
            idx = np.nonzero(row >= cut)[0]      # every token tied with the cut too
        else:
            idx = np.arange(V)
        return idx[np.lexsort((idx, -row[idx]))][:keep]

    kids.append(children(0))
    nxt.append(0)
    for n in range(1, T):
        best = None
        for e in range(n):
            if nxt[e] >= len(kids[e]):
                continue
            x = int(kids[e][nxt[e]])
            key = (-(cum[e] + lp[e, x]), e, x)
            if best is None or key < best:
                best = key
        negc, e, x = best
        parent[n], token[n], cum[n] = e, x, -negc
        nxt[e] += 1
        kids.append(children(n))
        nxt.append(0)
    return parent, token, cum
