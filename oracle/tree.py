"""Draft-tree structure.

A tree of T nodes is given by ``parent[T]``: node 0 is the root (the token the
target emitted last step, not yet in the committed cache), ``parent[0] = -1``
and ``0 <= parent[i] < i`` for every other node, so nodes are in topological
order (SpecExec page, "Approach": the draft tree of most likely continuations).
A node's inclusive ancestor set anc*(i) = {i, parent(i), ..., root}.
"""
import numpy as np


def root_path(parent, i):
    """Nodes from the root down to i, inclusive: [0, ..., parent(i), i]."""
    path = []
    n = int(i)
    while n >= 0:
        path.append(n)
        n = int(parent[n])
    return path[::-1]


def ancestor_matrix(parent):
    """Boolean [T, T] matrix A with A[i, j] = (j in anc*(i)).

    For attention, a negative parent on a non-root node just ends the chain
    (the node sees itself and whatever it does reach)."""
    T = len(parent)
    A = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in root_path(parent, i):
            A[i, j] = True
    return A


def children_of(parent, node):
    """Children of ``node`` in ascending index order."""
    return [c for c in range(len(parent)) if int(parent[c]) == node]
