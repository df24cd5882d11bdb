"""Pins of the oracle's batched tree attention mask and position ids ([SB]
"Tree Attention", build_tree_attn; [SS] "Verifying a tree instead of a line").
The printed mask and depths themselves are pinned in test_oracle_pins.py;
these pin the batched form, its packed layout, the offsets and the validity
rule. No GPU."""
import json
import os

import numpy as np

from oracle import trees

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_batch_reproduces_the_printed_mask_and_depths_with_offsets():
    g = _load("tree_mask_ss.json")
    mask, pos = trees.tree_attn_batch(np.array(g["parents"]), offsets=[0, 100])
    assert mask[0].tolist() == g["printed_mask"] and mask[1].tolist() == g["printed_mask"]
    d = _load("tree_depths_sb.json")
    _, pos = trees.tree_attn_batch(np.array([d["parents"]] * 2), offsets=[0, 7])
    assert pos[0].tolist() == d["printed_depths"]
    assert pos[1].tolist() == [x + 7 for x in d["printed_depths"]]


def test_mask_invariants_on_random_trees():
    """Lower triangular with a unit diagonal (parents precede children); row i
    has depth(i) + 1 ones; row i = row parent(i) plus the diagonal; two nodes
    see each other only along one line of descent."""
    rng = np.random.default_rng(1)
    for _ in range(50):
        N = int(rng.integers(1, 60))
        par = [-1] + [int(rng.integers(0, i)) for i in range(1, N)]
        mask, pos = trees.tree_attn_batch(np.array([par]))
        m = mask[0].astype(int)
        assert np.all(np.triu(m, 1) == 0) and np.all(np.diag(m) == 1)
        assert m.sum(1).tolist() == [p + 1 for p in pos[0]]
        for i in range(1, N):
            row = m[par[i]].copy()
            row[i] = 1
            assert np.array_equal(m[i], row)
        anc = m @ m.T  # shared ancestors count
        for i in range(N):
            for j in range(N):
                if m[i, j] and i != j:
                    assert anc[i, j] == pos[0][j] + 1


def test_packed_words_hold_the_same_bits():
    rng = np.random.default_rng(2)
    B, N = 3, 70
    par = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, N)] for _ in range(B)], np.int32)
    mask, pos = trees.tree_attn_batch(par)
    words, pos2 = trees.tree_attn_batch(par, packed=True)
    assert words.shape == (B, N, 3) and np.array_equal(pos, pos2)
    for j in range(N):
        assert np.array_equal((words[:, :, j // 32] >> np.uint32(j % 32)) & 1, mask[:, :, j])


def test_invalid_trees_are_marked():
    par = np.array([[-1, 0, 1], [0, 0, 1], [-1, 2, 1], [-1, 0, 0]], np.int32)
    mask, pos = trees.tree_attn_batch(par)
    assert pos[1].tolist() == [-1] * 3 and pos[2].tolist() == [-1] * 3
    assert not mask[1].any() and not mask[2].any()
    assert pos[0].tolist() == [0, 1, 2] and pos[3].tolist() == [0, 1, 1]
