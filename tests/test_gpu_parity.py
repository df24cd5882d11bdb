"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs. Ids, lengths and tree paths bit-exact (sequences the
oracle marks as Gumbel near-ties or accept knife-edges excused and counted);
accept probabilities, log-normalizers and residual mass within 1e-5."""
import os
import sys

import numpy as np
import pytest

import oracle
import workloads
from workloads import make_chain, make_tree

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


def _report(label, s):
    print("[parity] %s B=%d excused=%d %s" % (label, s["B"], len(s["excused"]),
          {k: "%.2g" % v for k, v in s.items() if k.endswith("maxerr")}), flush=True)


# -------------------------------------------------------------------------
# Chains: small and scaled workloads (several chunks and a ragged tail)
# -------------------------------------------------------------------------

CHAIN_CASES = {
    # name: kwargs of make_chain
    "f32_small": dict(B=1, gamma=4, V=1000, bf16=False, seed=1000, target_sigma=2.0, draft_sigma=0.5),
    "f32_ragged": dict(B=6, gamma=3, V=5003, bf16=False, seed=5, target_sigma=2.0, draft_sigma=0.8,
                       temperatures=(0.0, 0.6, 1.3), row_stride=5004),
    "bf16_peaked": dict(B=16, gamma=5, V=32000, bf16=True, seed=6, target_sigma=3.0, boost="peaks", n_boost=5,
                        boost_value=8.0, draft_scale=0.8, draft_sigma=1.0, temperatures=(0.8,)),
    "bf16_mixed_ragged": dict(B=24, gamma=8, V=40003, bf16=True, seed=7, target_sigma=3.0, boost="zipf",
                              draft_sigma=(0.2, 2.0), temperatures=(0.0, 0.7, 1.0), row_stride=40008),
    "bf16_onehot": dict(B=32, gamma=6, V=50000, bf16=True, seed=8, target_sigma=3.0, one_hot=True,
                        temperatures=(1.0,)),
    "bf16_onehot_mixed": dict(B=20, gamma=3, V=9001, bf16=True, seed=9, target_sigma=3.0, one_hot=True,
                              temperatures=(0.0, 1.0, 0.5)),
    "bf16_padded_rows": dict(B=8, gamma=4, V=20000, bf16=True, seed=10, target_sigma=3.0, draft_sigma=1.0,
                             temperatures=(0.0, 1.0), row_stride=20040),
    "bf16_misaligned_rows": dict(B=6, gamma=2, V=7001, bf16=True, seed=11, target_sigma=3.0, draft_sigma=1.0,
                                 temperatures=(0.9,), row_stride=7001),
    "bf16_gamma1": dict(B=40, gamma=1, V=3000, bf16=True, seed=12, target_sigma=1.0, draft_sigma=0.3,
                        temperatures=(1.0,)),
    "bf16_gamma16": dict(B=4, gamma=16, V=4096, bf16=True, seed=13, target_sigma=1.0, draft_sigma=0.2,
                         temperatures=(1.0, 0.0)),
}


@pytest.mark.parametrize("name", sorted(CHAIN_CASES))
def test_chain_parity(dev, name):
    kw = dict(CHAIN_CASES[name])
    inp = make_chain(name, kw.pop("B"), kw.pop("gamma"), kw.pop("V"), **kw)
    got = run_sample(inp, torch, dev)
    ref = oracle_sample(inp)
    _report(name, compare_chain(got, ref, label=name))


def test_chain_seeds_and_offsets(dev):
    """Different seeds/offsets change the draws, and every one matches."""
    inp = make_chain("offsets", 16, 4, 6000, bf16=True, seed=21, target_sigma=2.0, draft_sigma=1.5,
                     temperatures=(1.0,))
    outs = []
    for seed, off in ((0, 0), (0, 1), (123456789012345, 7), (2**64 - 1, 2**31 - 1)):
        got = run_sample(inp, torch, dev, seed=seed, offset=off)
        ref = oracle_sample(inp, seed=seed, offset=off)
        compare_chain(got, ref, label="seed %d off %d" % (seed, off))
        outs.append(got["tokens"])
    assert not all(np.array_equal(outs[0], o) for o in outs[1:])


def test_greedy_entry_point(dev):
    import rejection_sampling_verify_amd as rsv
    inp = make_chain("greedy", 64, 5, 30011, bf16=True, seed=22, target_sigma=1.0, draft_sigma=0.05,
                     temperatures=(0.0,))
    t = to_dev(inp.target, torch, dev)
    ids = torch.from_numpy(inp.draft_ids).to(dev)
    tok, n = rsv.spec_verify_greedy(t, ids)
    torch.cuda.synchronize()
    ref = oracle.verify_greedy(inp.target, inp.draft_ids)
    assert np.array_equal(n.cpu().numpy(), ref["n"])
    assert np.array_equal(tok.cpu().numpy(), ref["tokens"])
    # the sampled entry point at temperature 0 gives the same answer
    got = run_sample(inp, torch, dev)
    assert np.array_equal(got["tokens"], ref["tokens"]) and np.array_equal(got["n"], ref["n"])


def test_greedy_ties_lowest_index(dev):
    import rejection_sampling_verify_amd as rsv
    B, G, V = 4, 2, 20000
    tgt = np.zeros((B, G + 1, V), np.float32)
    for b in range(B):
        tgt[b, :, [17 + b, 9000 + b, 19999 - b]] = 3.0  # three-way tie in every row
    ids = np.array([[17 + b, 9000 + b] for b in range(B)], np.int32)
    ids[1] = [17 + 1, 17 + 1]
    t = torch.from_numpy(tgt).to(dev)
    tok, n = rsv.spec_verify_greedy(t, torch.from_numpy(ids).to(dev))
    ref = oracle.verify_greedy(tgt, ids)
    assert np.array_equal(tok.cpu().numpy(), ref["tokens"]) and np.array_equal(n.cpu().numpy(), ref["n"])
    assert ref["tokens"][0].tolist() == [17, 17, -1]


def test_bad_inputs_per_sequence(dev):
    inp = make_chain("bad", 6, 3, 2000, bf16=True, seed=23, target_sigma=1.0, draft_sigma=0.5,
                     temperatures=(1.0,))
    inp.draft_ids[1, 2] = 2000
    inp.draft_ids[2, 0] = -5
    inp.temperature[3] = -1.0
    inp.temperature[4] = np.nan
    got = run_sample(inp, torch, dev)
    ref = oracle_sample(inp)
    assert got["n"].tolist()[1:5] == [-1, -1, -2, -2]
    assert np.all(got["tokens"][1:5] == -1)
    compare_chain(got, ref, label="bad")


def test_deterministic_and_grid_invariant(dev):
    """Bitwise identical outputs across runs and tilings (pass-2 chunks per
    row forced through the debug entry point), and oracle-exact at any pass-1
    chunk length."""
    inp = make_chain("grid", 40, 6, 70001, bf16=True, seed=24, target_sigma=3.0, draft_sigma=(0.3, 1.5),
                     temperatures=(0.0, 0.7, 1.0))
    base = run_sample(inp, torch, dev)
    ref = oracle_sample(inp)
    compare_chain(base, ref, label="grid base")
    for tiling in ((0, 1), (0, 3), (0, 7), (0, 1000), (0, 5), None):
        got = run_sample(inp, torch, dev, tiling=tiling)
        for key in ("tokens", "n", "accept_prob", "logz_target", "logz_draft"):
            assert np.array_equal(got[key], base[key], equal_nan=True), (tiling, key)
        # the residual mass is summed over pass-2 chunks: their count changes rounding only
        np.testing.assert_allclose(got["residual_mass"], base["residual_mass"], rtol=0, atol=1e-6)
    # a different chunk length changes only rounding: still oracle-exact
    for kv in (1, 2, 8):
        compare_chain(run_sample(inp, torch, dev, tiling=(kv, 0)), ref, label="kv %d" % kv)


def test_onehot_tilings(dev):
    """One-hot drafts at mixed accept lengths: every tiling gives identical,
    oracle-exact outputs and leaves the workspace zero."""
    import rejection_sampling_verify_amd as rsv
    inp = make_chain("onehot_layouts", 48, 5, 30011, bf16=True, seed=25, target_sigma=6.0,
                     temperatures=(0.6, 1.0), one_hot=True, onehot_hit=0.85)
    ref = oracle_sample(inp)
    ws = rsv.Workspace(dev).get(48, 6, 30011)
    base = None
    for tiling in (None, (0, 1), (0, 2), (0, 3), (0, 100), (4, 0), (1, 7)):
        got = run_sample(inp, torch, dev, workspace=ws, tiling=tiling)
        compare_chain(got, ref, label="onehot %s" % (tiling,))
        if base is None:
            base = got
        # Pass-2 chunking changes nothing; a pass-1 chunk length changes only
        # the rounding of the row statistics (oracle-exact above).
        keys = ("tokens", "n", "accept_prob", "logz_target", "residual_mass") if tiling is None or tiling[0] == 0 \
            else ("tokens", "n")
        for key in keys:
            assert np.array_equal(got[key], base[key], equal_nan=True), (tiling, key)
        assert int(ws.count_nonzero().item()) == 0
    assert set(np.unique(base["n"])) >= {0, 1, 2, 5}


def test_workspace_reuse_across_shapes(dev):
    """One workspace serves calls of different shapes; each call leaves it zero."""
    import rejection_sampling_verify_amd as rsv
    ws = rsv.Workspace(dev).get(64, 17, 131072)
    shapes = [(32, 8, 100000), (3, 2, 500), (64, 16, 131072), (1, 1, 7), (17, 5, 33333), (40, 7, 60000)]
    for k, (B, G, V) in enumerate(shapes):
        inp = make_chain("ws%d" % k, B, G, V, bf16=True, seed=30 + k, target_sigma=2.0, draft_sigma=1.0,
                         temperatures=(0.0, 1.0), one_hot=(k % 2 == 1))
        got = run_sample(inp, torch, dev, workspace=ws)
        compare_chain(got, oracle_sample(inp), label="ws %s" % (shapes[k],))
    assert int(ws.count_nonzero().item()) == 0


@pytest.mark.parametrize("name", ["chain_bf16_peaked", "chain_bf16_llama", "onehot_bf16_qwen"])
def test_without_diagnostics(dev, name):
    """The call without diagnostic outputs (the kernels that skip the residual
    mass, as the benchmark runs them) gives the same ids and lengths as the
    call with them, at the default and at forced pass-2 chunk counts, and
    matches the oracle."""
    inp = workloads.make(name)
    ref = oracle_sample(inp)
    with_diag = run_sample(inp, torch, dev)
    for chunks in (None, 1, 5):
        got = run_sample(inp, torch, dev, diag=False, tiling=None if chunks is None else (0, chunks))
        assert np.array_equal(got["n"], with_diag["n"]), (name, chunks)
        assert np.array_equal(got["tokens"], with_diag["tokens"]), (name, chunks)
        compare_chain(got, ref, check_diag=False, label="%s no diagnostics" % name)


def test_more_sequences_than_resident_workgroups(dev):
    """More sequences with a pending draw than pass-2 workgroups fit on the
    GPU at once: one chunk per row, every sequence still drawn, oracle-exact,
    workspace left zero."""
    import rejection_sampling_verify_amd as rsv
    B, G, V = 2600, 3, 900
    inp = make_chain("many", B, G, V, bf16=True, seed=41, target_sigma=2.0, draft_sigma=1.0,
                     temperatures=(0.0, 0.8, 1.0))
    ws = rsv.Workspace(dev).get(B, G + 1, V)
    got = run_sample(inp, torch, dev, workspace=ws)
    compare_chain(got, oracle_sample(inp), label="many sequences")
    assert int(ws.count_nonzero().item()) == 0


# -------------------------------------------------------------------------
# Trees
# -------------------------------------------------------------------------

def _run_tree(inp, dev):
    import rejection_sampling_verify_amd as rsv
    t = to_dev(inp.target, torch, dev)
    par = torch.from_numpy(inp.parents).to(dev)
    dep = torch.from_numpy(inp.depth).to(dev)
    tok = torch.from_numpy(inp.node_tokens).to(dev)
    path, plen, bonus = rsv.spec_verify_tree(t, par, dep, tok, inp.max_depth)
    torch.cuda.synchronize()
    return path.cpu().numpy(), plen.cpu().numpy(), bonus.cpu().numpy()


def _check_tree(inp, dev):
    path, plen, bonus = _run_tree(inp, dev)
    ref = oracle.verify_tree(inp.target, inp.parents, inp.depth, inp.node_tokens, inp.max_depth)
    assert np.array_equal(plen, ref["path_len"])
    assert np.array_equal(path, ref["path"])
    assert np.array_equal(bonus, ref["bonus"])
    return ref


def test_tree_small(dev):
    parents = np.array([-1, 0, 0, 0, 1, 1, 2, 3, 4, 4, 6], np.int32)
    depth = np.array(oracle.tree_depths(parents), np.int32)
    for V, hit in ((50, 0.9), (3001, 0.6), (20000, 0.5)):
        inp = make_tree("t", 50, V, parents, depth, bf16=True, seed=40 + V, hit=hit)
        _check_tree(inp, dev)


def test_tree_chain_shaped_equals_greedy(dev):
    import rejection_sampling_verify_amd as rsv
    inp = make_chain("tchain", 30, 6, 12000, bf16=True, seed=41, target_sigma=1.0, draft_sigma=0.02,
                     temperatures=(0.0,))
    parents = np.array([-1] + list(range(6)), np.int32)
    depth = np.arange(7, dtype=np.int32)
    tok = np.concatenate([np.zeros((30, 1), np.int32), inp.draft_ids], axis=1)
    t = to_dev(inp.target, torch, dev)
    path, plen, bonus = rsv.spec_verify_tree(t, torch.from_numpy(parents).to(dev), torch.from_numpy(depth).to(dev),
                                             torch.from_numpy(tok).to(dev), 6)
    gtok, gn = rsv.spec_verify_greedy(t, torch.from_numpy(inp.draft_ids).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(plen.cpu().numpy() - 1, gn.cpu().numpy())
    gtok = gtok.cpu().numpy()
    for b in range(30):
        n = int(gn[b])
        assert bonus[b].item() == gtok[b, n]


def test_tree_fp32_repeatable(dev):
    """fp32 trees; repeated calls on one workspace give identical results and
    each returns the workspace to zero."""
    import rejection_sampling_verify_amd as rsv
    parents, depth = workloads.tree_c5_structure()
    inp = make_tree("tl", 24, 20011, parents, depth, bf16=False, seed=43, hit=0.6)
    base = _check_tree(inp, dev)
    ws = rsv.Workspace(dev).get(24, len(parents), 20011)
    t = to_dev(inp.target, torch, dev)
    args = (t, torch.from_numpy(inp.parents).to(dev), torch.from_numpy(inp.depth).to(dev),
            torch.from_numpy(inp.node_tokens).to(dev), inp.max_depth)
    for rep in range(3):
        path, plen, bonus = rsv.spec_verify_tree(*args, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(plen.cpu().numpy(), base["path_len"]), rep
        assert np.array_equal(path.cpu().numpy(), base["path"]), rep
        assert np.array_equal(bonus.cpu().numpy(), base["bonus"]), rep
        assert int(ws.count_nonzero().item()) == 0, rep


def test_tree_malformed(dev):
    parents = np.array([-1, 0, 2, 1], np.int32)  # node 2 is its own parent
    depth = np.array([0, 1, 2, 2], np.int32)
    inp = make_tree("bad", 3, 100, parents, depth, bf16=True, seed=42)
    path, plen, bonus = _run_tree(inp, dev)
    assert np.all(plen == -3) and np.all(bonus == -1) and np.all(path == -1)


# -------------------------------------------------------------------------
# The five named workloads at full size
# -------------------------------------------------------------------------

@pytest.mark.parametrize("name", workloads.CONFIGS)
def test_named_workload_full_size(dev, name):
    inp = workloads.make(name)
    if name.startswith("tree"):
        ref = _check_tree(inp, dev)
        print("[parity] %s B=%d exact; first-match walk differs on %d sequences" %
              (name, inp.B, int(np.sum(ref["first_match_node"] != ref["path"][np.arange(inp.B), ref["path_len"] - 1]))),
              flush=True)
        return
    got = run_sample(inp, torch, dev)
    ref = oracle_sample(inp)
    s = compare_chain(got, ref, label=name)
    _report(name, s)
    n = got["n"]
    print("[parity] %s mean accepted %.3f, emitted/step %.3f" % (name, n.mean(), n.mean() + 1), flush=True)


@pytest.mark.parametrize("name", [n for n in workloads.CONFIGS if not n.startswith("tree")])
def test_named_chains_more_seeds(dev, name):
    """The chain workloads at full size under four more (seed, offset) pairs:
    the same logits with other accept uniforms and Gumbel noise, hence other
    first rejections and other residual, one-hot and bonus draws. Launched as
    the bench launches them (no diagnostics); nothing is excused."""
    inp = workloads.make(name)
    for seed, offset in ((11, 0), (12, 5), ((1 << 40) + 3, 17), (977, 1 << 20)):
        got = run_sample(inp, torch, dev, seed=seed, offset=offset, diag=False)
        ref = oracle_sample(inp, seed=seed, offset=offset)
        compare_chain(got, ref, check_diag=False, label="%s seed %d offset %d" % (name, seed, offset))


def test_tree_deepest_paths(dev):
    """1024-node trees at full depth: a chain-shaped tree (depth 1023) whose
    every child carries its parent's argmax, so the accepted path runs to the
    last node, and a deep, narrow random tree (1 or 2 children per node)."""
    N = 1024
    chain = np.arange(-1, N - 1, dtype=np.int32)
    depth = np.array(oracle.tree_depths(chain), np.int32)
    inp = make_tree("chain1024", 3, 2000, chain, depth, bf16=True, seed=46, hit=1.0)
    ref = _check_tree(inp, dev)
    assert np.all(ref["path_len"] == N)
    rng = np.random.default_rng(47)
    narrow = workloads.random_tree(rng, N, (1, 2))
    depth = np.array(oracle.tree_depths(narrow), np.int32)
    assert depth.max() >= 9
    inp = make_tree("narrow1024", 4, 3001, narrow, depth, bf16=False, seed=48, hit=0.97)
    ref = _check_tree(inp, dev)
    assert ref["path_len"].max() >= 6


def test_tree_largest(dev):
    """The greedy tree walk at the largest tree (1024 nodes): deep paths
    (children carry their parent's argmax often), bit-exact."""
    rng = np.random.default_rng(44)
    parents = workloads.random_tree(rng, 1024, (2, 6))
    depth = np.array(oracle.tree_depths(parents), np.int32)
    inp = make_tree("t1024", 6, 2000, parents, depth, bf16=True, seed=45, hit=0.9)
    ref = _check_tree(inp, dev)
    assert ref["path_len"].max() >= 4
