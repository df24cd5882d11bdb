"""Pins of the oracle's KV-cache rollback ([SB] "KV-Cache Reuse and Rollback")."""
import numpy as np

from oracle import kv


def test_chain_path_is_the_crop():
    """A chain step's path is the identity: nothing moves, and the new length
    is the page's keep = T + n (root at T - 1, path of n + 1 nodes)."""
    rng = np.random.default_rng(0)
    c = rng.standard_normal((2, 3, 2, 20, 4)).astype(np.float32)
    T = np.array([5, 9, 1], np.int32)
    n = np.array([0, 3, 4], np.int32)
    path = np.full((3, 5), -1, np.int32)
    for b in range(3):
        path[b, :n[b] + 1] = np.arange(n[b] + 1)
    out, new_len = kv.kv_rollback(c, T - 1, path, n + 1)
    assert np.array_equal(out, c)
    assert list(new_len) == list(T + n)


def test_tree_path_gathers_the_accepted_nodes():
    """Path [0, 2, 5] under a root at position 3: positions 3, 4, 5 take the
    entries of positions 3, 5, 8; everything before the root and after the new
    length is left as it was."""
    L, B, H, S, D = 2, 1, 2, 12, 3
    c = np.arange(L * B * H * S * D, dtype=np.float32).reshape(L, B, H, S, D)
    out, new_len = kv.kv_rollback(c, np.array([3]), np.array([[0, 2, 5, -1]], np.int32), np.array([3]))
    assert new_len[0] == 6
    assert np.array_equal(out[:, :, :, :3], c[:, :, :, :3])
    assert np.array_equal(out[:, :, :, 3], c[:, :, :, 3])
    assert np.array_equal(out[:, :, :, 4], c[:, :, :, 5])
    assert np.array_equal(out[:, :, :, 5], c[:, :, :, 8])
    assert np.array_equal(out[:, :, :, 6:], c[:, :, :, 6:])


def test_invalid_paths_are_left_alone():
    c = np.zeros((1, 3, 1, 8, 2), np.float32)
    path = np.array([[0, 1, -1], [1, 2, -1], [0, 7, -1]], np.int32)
    out, new_len = kv.kv_rollback(c, np.array([0, 0, 3]), path, np.array([0, 2, 2]))
    assert list(new_len) == [-1, -1, -1]  # empty path; root not first; past the end
    assert np.array_equal(out, c)
    out, new_len = kv.kv_rollback(c, np.array([0, 0, 0]), path, np.array([4, 3, 1]))
    assert list(new_len) == [-1, -1, 1]  # a length beyond the path array; a path with a -1 node
    assert np.array_equal(out, c)
