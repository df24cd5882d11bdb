"""The input generators keep their stated contracts (no GPU)."""
import numpy as np

import oracle
import workloads


def test_tree_sample_without_replacement_draws_distinct_siblings():
    parents, depth = workloads.tree_c5_structure()
    inp = workloads.make_tree_sample("t", 4, 500, parents, depth, bf16=False, seed=1, without_replacement=True)
    for b in range(4):
        for v in set(int(p) for p in parents[1:]):
            kids = [c for c in range(1, len(parents)) if parents[c] == v]
            toks = inp.node_tokens[b, kids]
            assert len(set(toks.tolist())) == len(kids)
    assert inp.meta["without_replacement"]


def test_kv_and_tree_mask_generators_make_valid_inputs():
    parents, _ = workloads.tree_c5_structure()
    kv = workloads.make_kv_rollback("k", 1, 16, 1, 300, 8, elem_bytes=4, seed=2, kind="tree", parents=parents)
    from oracle import kv as okv
    _, n = okv.kv_rollback(np.zeros((1, 16, 1, 300, 1), np.float32), kv.root, kv.path, kv.path_len)
    assert np.all(n >= 1)  # every generated path is a valid gather
    tm = workloads.make_tree_mask("m", 8, 40, seed=3)
    from oracle import trees
    assert all(trees.tree_is_valid(list(p)) for p in tm.parents)
