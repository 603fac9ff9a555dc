"""Token acceptance walk over a verified draft tree (float64).

Three rules, chosen by the arguments (reading: temperature 0 means greedy;
temperature > 0 with draft probabilities means rejection sampling; temperature
> 0 without them means sampling from the target at each node):

* greedy -- at the current node take the target argmax (lowest token id on
  ties); descend into the lowest-index child carrying that token, else stop.
  At temperature 0 this reproduces target-argmax decoding exactly, which is
  what keeps verification lossless (EasySpec page, "Approach").
* rejection sampling ("mss") -- standard speculative sampling (SpecExec page,
  "Builds on": speculative sampling, SpecInfer), applied to siblings in
  ascending index: child c with token x is accepted when u_c * q(x) < r(x);
  on rejection the target residual becomes normalise(max(r - q, 0)) and the
  next sibling is tried against it.  If every child is rejected (or there is
  none) the bonus token is drawn from the current residual.
* "exec" -- draw x from the target softmax at the current node; descend into
  the lowest-index child with token x, else x is the bonus.  This stays
  equivalent to sequential sampling from the target and works for
  deterministic trees (SpecExec page, "Approach").

Uniforms: u[b, i, 0] is the acceptance test of node i, u[b, i, 1] the sample
drawn at node i.  Temperature divides the target logits only.  When the
residual mass is exactly zero the residual is left as it was.

The output ``path`` starts with the root (node 0) and lists accepted nodes;
``path_len`` counts them (accepted drafts + 1); ``bonus`` is the token the
target emits after the path, the next step's root.
"""
import numpy as np

from .codec import decode
from .tree import children_of


def softmax(logits, temperature):
    z = logits / temperature
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def invcdf(w, u):
    """Smallest x with sum_{y <= x} w_y > u * sum(w); if rounding leaves no such
    x, the last x with w_x > 0."""
    c = np.cumsum(w)
    thr = u * c[-1]
    x = int(np.searchsorted(c, thr, side="right"))
    if x >= len(w):
        x = int(np.nonzero(w > 0)[0][-1])
    return x, c, thr


def accept(target_logits, logit_dtype, draft_probs, tree_parent, tree_token, uniforms,
           temperature, trace=False):
    """Returns (path [B, T] int32 padded with -1, path_len [B], bonus [B]) and,
    with trace=True, a per-sequence list of decision events for the
    comparison protocol."""
    B, T, V = target_logits.shape
    path = np.full((B, T), -1, dtype=np.int32)
    plen = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    events = []
    tp = np.asarray(tree_parent)
    for b in range(B):
        par = tp[0] if tp.shape[0] == 1 else tp[b]
        tok = np.asarray(tree_token)[0] if np.asarray(tree_token).shape[0] == 1 else tree_token[b]
        ev = []
        cur = 0
        walk = [0]
        while True:
            logits = decode(target_logits[b, cur], logit_dtype)
            kids = children_of(par, cur)
            if temperature == 0:
                a = int(np.argmax(logits))
                ev.append(("argmax", cur, a))
                nxt = next((c for c in kids if int(tok[c]) == a), None)
                if nxt is None:
                    bonus[b] = a
                    break
            elif draft_probs is None:
                p = softmax(logits, temperature)
                u = float(uniforms[b, cur, 1])
                x, c, thr = invcdf(p, u)
                ev.append(("sample", cur, x, c, thr))
                nxt = next((k for k in kids if int(tok[k]) == x), None)
                if nxt is None:
                    bonus[b] = x
                    break
            else:
                r = softmax(logits, temperature)
                qd = np.asarray(draft_probs[b, cur], dtype=np.float32).astype(np.float64)
                nxt = None
                for k in kids:
                    x = int(tok[k])
                    u = float(uniforms[b, k, 0])
                    ok = u * qd[x] < r[x]
                    ev.append(("test", cur, k, r[x], qd[x], u, ok))
                    if ok:
                        nxt = k
                        break
                    rn = np.maximum(r - qd, 0.0)
                    z = rn.sum()
                    if z > 0:
                        r = rn / z
                if nxt is None:
                    x, c, thr = invcdf(r, float(uniforms[b, cur, 1]))
                    ev.append(("sample", cur, x, c, thr))
                    bonus[b] = x
                    break
            walk.append(nxt)
            cur = nxt
        path[b, :len(walk)] = walk
        plen[b] = len(walk)
        events.append(ev)
    if trace:
        return path, plen, bonus, events
    return path, plen, bonus
