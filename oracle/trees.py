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


def tree_is_valid(parents) -> bool:
    """The order build_tree_attn asks for: the root first (parent -1), and
    every other node's parent an earlier node."""
    return len(parents) >= 1 and parents[0] == -1 and all(0 <= parents[i] < i for i in range(1, len(parents)))


def tree_attn_batch(parents: np.ndarray, offsets=None, packed: bool = False):
    """Batched build_tree_attn. parents: [B, N] (one tree per sequence) or [N]
    (with offsets giving B). Returns (mask [B, N, N] uint8, or [B, N, ceil(N/32)]
    uint32 words with bit j % 32 of word j // 32 for column j; position ids
    [B, N] int32 = offset + depth). A sequence whose tree is not in that order
    gets an all-zero mask and position ids -1."""
    parents = np.asarray(parents)
    if parents.ndim == 1:
        B = 1 if offsets is None else len(offsets)
        parents = np.broadcast_to(parents, (B, parents.shape[0]))
    B, N = parents.shape
    offsets = np.zeros(B, np.int64) if offsets is None else np.asarray(offsets, np.int64)
    mask = np.zeros((B, N, N), np.uint8)
    pos = np.full((B, N), -1, np.int32)
    for b in range(B):
        par = [int(x) for x in parents[b]]
        if not tree_is_valid(par):
            continue
        mask[b] = ancestor_mask(par)
        pos[b] = np.asarray(depths(par), np.int64) + offsets[b]
    if not packed:
        return mask, pos
    W = (N + 31) // 32
    words = np.zeros((B, N, W), np.uint32)
    for j in range(N):
        words[:, :, j // 32] |= mask[:, :, j].astype(np.uint32) << np.uint32(j % 32)
    return words, pos
