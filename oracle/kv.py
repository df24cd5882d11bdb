"""KV-cache rollback after verification (TEST INFRASTRUCTURE ONLY).

From "7.6 Speculative Decoding: Draft Models, Medusa, EAGLE & Lookahead",
section "KV-Cache Reuse and Rollback": after a chain step every layer's cache is
cropped to keep = T + n positions; after a tree step the cache keeps exactly the
accepted root-to-leaf path, gathered along the sequence dimension with
index_select over the flattened node positions.

Layout here: one tensor per K or V, [layers, batch, heads, positions, head_dim].
Node i of sequence b's tree sits at position root[b] + i (node 0, the root, is
the last committed token, whose cache entry the verify pass wrote). The path is
the verify step's: root first, path_len nodes. Written as the page's gather,
with numpy.take along the sequence axis as index_select.
"""
from __future__ import annotations

import numpy as np


def kv_rollback(cache: np.ndarray, root: np.ndarray, path: np.ndarray, path_len: np.ndarray):
    """Returns (new cache, new lengths). keep_idx = [0 .. root) + root + path[:len];
    positions from len(keep_idx) on are left as they were. A sequence with a
    path that is not a valid gather (len < 1 or beyond the path array, a node
    before its predecessor, a position past the end) is left unchanged and gets
    length -1."""
    L, B, H, S, D = cache.shape
    out = cache.copy()
    new_len = np.empty(B, np.int32)
    for b in range(B):
        n = int(path_len[b])
        p = [int(x) for x in path[b, :max(n, 0)]]
        r = int(root[b])
        ok = 1 <= n <= path.shape[1] and p[0] == 0 and all(p[k] > p[k - 1] for k in range(1, n)) and 0 <= r and r + p[-1] < S
        if not ok:
            new_len[b] = -1
            continue
        keep = np.concatenate([np.arange(r), r + np.asarray(p)])
        out[:, b, :, :len(keep), :] = np.take(cache[:, b], keep, axis=2)  # index_select(seq, keep_idx)
        new_len[b] = len(keep)
    return out, new_len
