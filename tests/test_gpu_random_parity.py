"""Randomized GPU parity against the CPU oracle, through the C ABI.

Each case draws its own shape and settings from a fixed seed: batch, draft
length, vocabulary (small ones of a few hundred entries or fewer, sizes that
are not multiples of the 8-element vector, and the full 128256), bf16 or
fp32 logits, dense or one-hot drafts, a mix of greedy and sampled
temperatures, the Philox seed and offset, and, for chains, both the
library's tiling and a forced one. Greedy trees get random shapes and
match rates; sampled trees get random shapes and both sibling rules. Tokens,
accepted lengths and paths must match the oracle bit for bit ([SB] "The rule", "Extending to a chain of γ draft tokens" and "Tree
Attention"); at these seeds nothing is excused.
"""
import numpy as np
import pytest

import oracle
import workloads
from workloads import make_chain, make_tree, make_tree_sample

from gpu_util import compare_chain, oracle_sample, run_sample, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _vocab(rng):
    pick = rng.random()
    if pick < 0.3:
        return int(rng.integers(9, 200))
    if pick < 0.55:
        return 128256
    return int(rng.integers(300, 70000))


@pytest.mark.parametrize("block", range(4))
def test_random_chains(dev, block):
    rng = np.random.default_rng(9100 + block)
    for it in range(12):
        B, G, V = int(rng.integers(1, 48)), int(rng.integers(1, 9)), _vocab(rng)
        bf16 = bool(rng.random() < 0.7)
        one_hot = bool(rng.random() < 0.3)
        temps = tuple(float(x) for x in rng.choice([0.0, 0.3, 0.7, 1.0, 1.5, 2.5], size=int(rng.integers(1, 4))))
        kw = dict(bf16=bf16, seed=int(rng.integers(1 << 30)), target_sigma=float(rng.choice([0.5, 1.0, 2.0, 3.0])),
                  temperatures=temps)
        if one_hot:
            kw["one_hot"] = True
        else:
            kw["draft_sigma"] = (float(rng.uniform(0.05, 0.5)), float(rng.uniform(0.6, 2.5)))
        inp = make_chain("random_%d_%d" % (block, it), B, G, V, **kw)
        seed, offset = int(rng.integers(0, 1 << 40)), int(rng.integers(0, 1 << 20))
        ref = oracle_sample(inp, seed=seed, offset=offset)
        label = "block %d case %d: B=%d G=%d V=%d bf16=%s one-hot=%s T=%s" % (block, it, B, G, V, bf16, one_hot, temps)
        for tiling in (None, (int(rng.choice([1, 2, 4, 8])), int(rng.integers(0, 12)))):
            got = run_sample(inp, torch, dev, seed=seed, offset=offset, tiling=tiling, diag=bool(rng.random() < 0.5))
            compare_chain(got, ref, check_diag=False, label="%s tiling %s" % (label, tiling))


@pytest.mark.parametrize("block", range(2))
def test_random_sampled_trees(dev, block):
    import rejection_sampling_verify_amd as rsv
    rng = np.random.default_rng(9200 + block)
    for it in range(10):
        N, B, V = int(rng.integers(2, 60)), int(rng.integers(1, 24)), _vocab(rng) if rng.random() < 0.5 else 128256
        bf16 = bool(rng.random() < 0.7)
        wor = bool(rng.random() < 0.5)
        parents = workloads.random_tree(rng, N, (1, 4))
        depth = np.array(oracle.tree_depths(parents), np.int32)
        inp = make_tree_sample("random_tree_%d_%d" % (block, it), B, V, parents, depth, bf16=bf16,
                               seed=int(rng.integers(1 << 30)), temperatures=(0.6, 1.0, 1.7),
                               target_sigma=float(rng.choice([1.0, 2.0, 3.0])), zipf=float(rng.choice([0.0, 1.1])),
                               draft_sigma=(0.1, 2.0), without_replacement=wor)
        seed, offset = int(rng.integers(0, 1 << 40)), int(rng.integers(0, 1 << 20))
        path, plen, token = rsv.spec_verify_tree_sample(
            to_dev(inp.target, torch, dev), to_dev(inp.draft, torch, dev), torch.from_numpy(inp.parents).to(dev),
            torch.from_numpy(inp.depth).to(dev), torch.from_numpy(inp.node_tokens).to(dev),
            torch.from_numpy(inp.temperature).to(dev), inp.max_depth, seed=seed, offset=offset,
            without_replacement=wor)
        torch.cuda.synchronize()
        ref = oracle.verify_tree_sample(inp.target, inp.draft, inp.parents, inp.depth, inp.node_tokens,
                                        inp.temperature, inp.max_depth, seed=seed, offset=offset,
                                        without_replacement=wor)
        label = "block %d case %d: N=%d B=%d V=%d bf16=%s wor=%s" % (block, it, N, B, V, bf16, wor)
        assert np.array_equal(plen.cpu().numpy(), ref["path_len"]), label
        assert np.array_equal(path.cpu().numpy(), ref["path"]), label
        assert np.array_equal(token.cpu().numpy(), ref["token"]), label


@pytest.mark.parametrize("block", range(2))
def test_random_greedy_trees(dev, block):
    import rejection_sampling_verify_amd as rsv
    rng = np.random.default_rng(9300 + block)
    for it in range(10):
        N, B, V = int(rng.integers(1, 300)), int(rng.integers(1, 40)), _vocab(rng)
        bf16 = bool(rng.random() < 0.7)
        parents = workloads.random_tree(rng, N, (1, int(rng.integers(1, 7))))
        depth = np.array(oracle.tree_depths(parents), np.int32)
        inp = make_tree("random_greedy_%d_%d" % (block, it), B, V, parents, depth, bf16=bf16,
                        seed=int(rng.integers(1 << 30)), target_sigma=float(rng.choice([1.0, 3.0])),
                        hit=float(rng.choice([0.3, 0.7, 0.95])))
        path, plen, bonus = rsv.spec_verify_tree(
            to_dev(inp.target, torch, dev), torch.from_numpy(inp.parents).to(dev),
            torch.from_numpy(inp.depth).to(dev), torch.from_numpy(inp.node_tokens).to(dev), inp.max_depth)
        torch.cuda.synchronize()
        ref = oracle.verify_tree(inp.target, inp.parents, inp.depth, inp.node_tokens, inp.max_depth)
        label = "block %d case %d: N=%d B=%d V=%d bf16=%s" % (block, it, N, B, V, bf16)
        assert np.array_equal(plen.cpu().numpy(), ref["path_len"]), label
        assert np.array_equal(path.cpu().numpy(), ref["path"]), label
        assert np.array_equal(bonus.cpu().numpy(), ref["bonus"]), label
