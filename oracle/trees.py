"""Tree-structure helpers of the oracle (TEST INFRASTRUCTURE ONLY).

From "7.6 Speculative Decoding: Draft Models, Medusa, EAGLE & Lookahead",
section "Tree Attention: Verifying Many Candidates at Once" (build_tree_attn:
a node sees itself and its ancestors; its position id is its depth), and
"Medusa, EAGLE and self-speculation", "Verifying a tree instead of a line"
(the same ancestor-or-self mask over a parent array).
"""
from __future__ import annotations

import numpy as np


def ancestor_mask(parents) -> np.ndarray:
    """mask[i, j] = 1 iff node j is node i or one of its ancestors."""
    n = len(parents)
    mask = np.zeros((n, n), dtype=np.int64)
    for i in range(n):
        j = i
        while j is not None and j != -1:
            mask[i, j] = 1
            j = parents[j]
    return mask


def depths(parents) -> list[int]:
    """Number of ancestors of each node."""
    out = []
    for i in range(len(parents)):
        d, j = 0, parents[i]
        while j is not None and j != -1:
            d += 1
            j = parents[j]
        out.append(d)
    return out


def longest_valid_path(parents, tokens, argmax_of):
    """Brute force over every root-to-node path: a path survives iff each of
    its nodes carries the argmax of its parent's row. Returns the longest
    surviving path, ties broken by the smallest final node index."""
    n = len(parents)
    best = [0]
    for end in range(n):
        path = []
        j = end
        while j != -1:
            path.append(j)
            j = parents[j]
        path.reverse()
        if all(tokens[c] == argmax_of[parents[c]] for c in path[1:]):
            if len(path) > len(best) or (len(path) == len(best) and end < best[-1]):
                best = path
    return best
