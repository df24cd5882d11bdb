"""GPU parity of sampled tree verification (multi-round rejection sampling)
against the CPU oracle, through the C ABI.

Paths, path lengths and tokens are bit-exact, except sequences the oracle
marks as a Gumbel near-tie of its final draw (relative top-two gap < 1e-6) or
as an accept knife-edge. For trees the knife-edge margin is 1e-4 rather than
the chains' 1e-5: after k rejections the kernels read the target distribution
as (p - A q)_+ / B in fp32, and the error of an accept probability computed that
way grows like (A + B) / B times the rounding of p and q (B, the residual mass
left, can be small). Excused sequences are counted and printed."""
import numpy as np
import pytest

import oracle
import workloads
from workloads import make_tree_sample

from gpu_util import NEAR_TIE, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TREE_KNIFE = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_amd as rsv
    rsv.lib()
    return torch.device("cuda:0")


def _run(inp, dev, seed=0, offset=0, workspace=None, temperature=None, parents=None, tokens=None, wor=False):
    import rejection_sampling_verify_amd as rsv
    t = to_dev(inp.target, torch, dev)
    d = to_dev(inp.draft, torch, dev)
    par = torch.from_numpy(inp.parents if parents is None else parents).to(dev)
    dep = torch.from_numpy(inp.depth).to(dev)
    tok = torch.from_numpy(inp.node_tokens if tokens is None else tokens).to(dev)
    temp = torch.from_numpy(inp.temperature if temperature is None else temperature).to(dev)
    path, plen, token = rsv.spec_verify_tree_sample(t, d, par, dep, tok, temp, inp.max_depth, seed=seed,
                                                    offset=offset, workspace=workspace, without_replacement=wor)
    torch.cuda.synchronize()
    return {"path": path.cpu().numpy(), "path_len": plen.cpu().numpy(), "token": token.cpu().numpy()}


def _compare(got, ref, label, allow_excused=0):
    B = ref["path_len"].shape[0]
    excused = []
    for b in range(B):
        if (got["path_len"][b] == ref["path_len"][b] and np.array_equal(got["path"][b], ref["path"][b])
                and got["token"][b] == ref["token"][b]):
            continue
        ok = ref["top_gap"][b] < NEAR_TIE or ref["margin"][b] < TREE_KNIFE
        assert ok, ("%s sequence %d differs: gpu len %d path %s token %d, oracle len %d path %s token %d "
                    "(gap %.3g, margin %.3g)" % (label, b, got["path_len"][b], got["path"][b].tolist(),
                                                 got["token"][b], ref["path_len"][b], ref["path"][b].tolist(),
                                                 ref["token"][b], ref["top_gap"][b], ref["margin"][b]))
        excused.append(b)
    print("[tree-sample parity] %s B=%d excused=%d rejections=%s" % (label, B, len(excused),
          np.bincount(np.maximum(ref["rejections"], 0)).tolist()), flush=True)
    # At the fixed seeds of the tests nothing is excused.
    assert len(excused) == allow_excused, "%s: excused %s, expected %d" % (label, excused, allow_excused)
    return excused


def _oracle(inp, seed=0, offset=0, temperature=None, parents=None, tokens=None, wor=False):
    return oracle.verify_tree_sample(inp.target, inp.draft, inp.parents if parents is None else parents, inp.depth,
                                     inp.node_tokens if tokens is None else tokens,
                                     inp.temperature if temperature is None else temperature, inp.max_depth,
                                     seed=seed, offset=offset, without_replacement=wor)


def _random_tree(rng, N, branching=(1, 4)):
    parents = [-1]
    frontier = [0]
    while len(parents) < N:
        nxt = []
        for p in frontier:
            for _ in range(int(rng.integers(branching[0], branching[1] + 1))):
                if len(parents) < N:
                    parents.append(p)
                    nxt.append(len(parents) - 1)
        frontier = nxt or [len(parents) - 1]
    par = np.array(parents, np.int32)
    return par, oracle.tree_depths(par)


CASES = {
    # name: (B, N, V, bf16, temperatures, seed)
    "f32_small": (24, 9, 1000, False, (0.6, 1.0, 1.8), 1),
    "f32_ragged": (16, 17, 5003, False, (1.0,), 2),
    "bf16_deep": (12, 13, 20000, True, (0.7, 1.0), 3),
    "bf16_wide": (16, 21, 40003, True, (1.0, 0.5), 4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_tree_sample_parity(dev, name):
    B, N, V, bf16, temps, seed = CASES[name]
    rng = np.random.default_rng(seed)
    parents, depth = _random_tree(rng, N)
    inp = make_tree_sample(name, B, V, parents, depth, bf16=bf16, seed=seed, temperatures=temps,
                           target_sigma=2.0, zipf=0.0 if not bf16 else 1.1, draft_sigma=(0.3, 1.5))
    for s, off in ((0, 0), (7, 3)):
        got = _run(inp, dev, seed=s, offset=off)
        _compare(got, _oracle(inp, seed=s, offset=off), "%s seed %d" % (name, s))


def test_chain_shaped_tree_matches_the_chain_oracle(dev):
    """A tree in which every node has one child verifies as the chain
    (the same keying of the random words)."""
    B, G, V = 32, 6, 3000
    inp = make_tree_sample("chain", B, V, np.arange(-1, G, dtype=np.int32), np.arange(0, G + 1, dtype=np.int32),
                           bf16=True, seed=21, temperatures=(0.7, 1.0, 1.5), draft_sigma=(0.5, 2.0))
    got = _run(inp, dev, seed=5, offset=1)
    ch = oracle.verify_sample(inp.target, np.ascontiguousarray(inp.draft[:, :G]), inp.node_tokens[:, 1:],
                              inp.temperature, seed=5, offset=1)
    ref = _oracle(inp, seed=5, offset=1)
    assert np.array_equal(ref["path_len"] - 1, ch["n"])
    _compare(got, ref, "chain-shaped")
    assert len(set((got["path_len"] - 1).tolist())) > 2


def test_draft_equal_to_target_follows_first_children(dev):
    B, V = 8, 4096
    parents = np.array([-1, 0, 0, 1, 1, 2, 3], np.int32)
    depth = oracle.tree_depths(parents)
    inp = make_tree_sample("q_eq_p", B, V, parents, depth, bf16=True, seed=22, temperatures=(1.0,))
    inp.draft[:] = inp.target
    got = _run(inp, dev, seed=2)
    assert np.all(got["path"] == np.array([0, 1, 3, 6], np.int32))
    _compare(got, _oracle(inp, seed=2), "q = p")


def test_bad_inputs_and_workspace(dev):
    """Per-sequence codes (bad temperature -2, bad token -1, invalid tree -3)
    match the oracle, and every call returns its workspace to zero."""
    import rejection_sampling_verify_amd as rsv
    B, V = 6, 2000
    parents = np.array([-1, 0, 0, 1, 2], np.int32)
    depth = oracle.tree_depths(parents)
    inp = make_tree_sample("bad", B, V, parents, depth, bf16=False, seed=23, temperatures=(1.0,))
    ws = rsv.Workspace(dev).get(B, len(parents), V)
    temp = inp.temperature.copy()
    temp[1] = 0.0
    temp[2] = -1.0
    tok = inp.node_tokens.copy()
    tok[3, 2] = V
    got = _run(inp, dev, temperature=temp, tokens=tok, workspace=ws)
    ref = _oracle(inp, temperature=temp, tokens=tok)
    assert list(got["path_len"][1:4]) == [-2, -2, -1]
    _compare(got, ref, "bad inputs")
    assert int(ws.count_nonzero().item()) == 0
    bad_parents = parents.copy()
    bad_parents[3] = 4  # a child before its parent
    got = _run(inp, dev, parents=bad_parents, workspace=ws)
    assert np.all(got["path_len"] == -3) and np.all(got["token"] == -1)
    assert int(ws.count_nonzero().item()) == 0


def test_more_sequences_than_one_walk_launch(dev):
    """Enough sequences that the walk runs in several launches (every
    workgroup of a launch must be resident at once)."""
    import rejection_sampling_verify_amd as rsv
    B, V = 3000, 1000
    parents = np.array([-1, 0, 0, 0, 1], np.int32)
    depth = oracle.tree_depths(parents)
    inp = make_tree_sample("many", B, V, parents, depth, bf16=True, seed=24, temperatures=(0.8, 1.2),
                           zipf=0.0, target_sigma=1.5)
    ws = rsv.Workspace(dev).get(B, len(parents), V)
    got = _run(inp, dev, seed=3, workspace=ws)
    _compare(got, _oracle(inp, seed=3), "many sequences")
    assert int(ws.count_nonzero().item()) == 0


def test_named_workload_full_size(dev):
    inp = workloads.make_extra("tree_sample_bf16_llama")
    got = _run(inp, dev, seed=inp.seed, offset=inp.offset)
    ref = _oracle(inp, seed=inp.seed, offset=inp.offset)
    _compare(got, ref, "tree_sample_bf16_llama")
    assert np.all(ref["path_len"] >= 1)
    # Other accept uniforms and noise over the same logits, both sibling rules.
    for seed, offset, wor in ((21, 0, False), (22, 9, True), ((1 << 36) + 5, 123, False), (23, 1 << 18, True)):
        got = _run(inp, dev, seed=seed, offset=offset, wor=wor)
        _compare(got, _oracle(inp, seed=seed, offset=offset, wor=wor),
                 "tree_sample_bf16_llama seed %d offset %d wor=%s" % (seed, offset, wor))


@pytest.mark.parametrize("N,V", [(1, 1000), (2, 1000), (2, 700), (3, 2048)])
def test_smallest_trees_and_vocabularies(dev, N, V):
    """A root alone (a bonus draw, one action) and the smallest trees with a
    child, at vocabularies of one workgroup part: the walk's second slot
    buffer sits in the greedy tree's slot area, which holds it exactly from
    N = 2 on and is never used by a one-node tree."""
    import rejection_sampling_verify_amd as rsv
    B = 40
    parents = np.arange(-1, N - 1, dtype=np.int32)
    depth = np.arange(N, dtype=np.int32)
    inp = make_tree_sample("small_%d_%d" % (N, V), B, V, parents, depth, bf16=True, seed=30 + N, temperatures=(0.8, 1.2),
                           zipf=0.0, target_sigma=1.5, draft_sigma=(0.2, 1.0))
    ws = rsv.Workspace(dev).get(B, N, V)
    for s in (0, 5):
        got = _run(inp, dev, seed=s, workspace=ws)
        ref = _oracle(inp, seed=s)
        _compare(got, ref, "N=%d V=%d seed %d" % (N, V, s))
        assert int(ws.count_nonzero().item()) == 0
    if N == 1:
        assert np.all(got["path_len"] == 1)


# Siblings drawn without replacement: each round's q is q over the tokens not
# drawn yet, renormalized; drawn siblings keep their residual values.

@pytest.mark.parametrize("name", sorted(CASES))
def test_tree_sample_without_replacement_parity(dev, name):
    B, N, V, bf16, temps, seed = CASES[name]
    rng = np.random.default_rng(seed + 100)
    parents, depth = _random_tree(rng, N)
    inp = make_tree_sample(name + "_wor", B, V, parents, depth, bf16=bf16, seed=seed + 100, temperatures=temps,
                           target_sigma=2.0, zipf=0.0 if not bf16 else 1.1, draft_sigma=(0.3, 1.5),
                           without_replacement=True)
    for s_, off in ((0, 0), (9, 4)):
        got = _run(inp, dev, seed=s_, offset=off, wor=True)
        ref = _oracle(inp, seed=s_, offset=off, wor=True)
        _compare(got, ref, "%s without replacement seed %d" % (name, s_))
    assert np.any(ref["rejections"] >= 2)  # drawn siblings kept apart in passes and draws


def test_without_replacement_full_size_and_rules(dev):
    """The 65-node workload's shape with siblings drawn without replacement;
    duplicate siblings are a bad token only in this mode; one child per node
    verifies as with replacement."""
    import rejection_sampling_verify_amd as rsv
    parents, depth = workloads.tree_c5_structure()
    inp = make_tree_sample("c5_wor", 32, 128256, parents, depth, bf16=True, seed=2100, without_replacement=True)
    ws = rsv.Workspace(dev).get(32, len(parents), 128256)
    got = _run(inp, dev, seed=1, workspace=ws, wor=True)
    _compare(got, _oracle(inp, seed=1, wor=True), "c5 without replacement")
    assert int(ws.count_nonzero().item()) == 0
    tok = inp.node_tokens.copy()
    tok[3, 2] = tok[3, 1]  # two children of the root with one token
    got = _run(inp, dev, seed=1, tokens=tok, wor=True)
    assert got["path_len"][3] == -1
    _compare(got, _oracle(inp, seed=1, tokens=tok, wor=True), "duplicate siblings")
    got_iid = _run(inp, dev, seed=1, tokens=tok)
    assert got_iid["path_len"][3] >= 1
    chain = make_tree_sample("chain_wor", 16, 3000, np.arange(-1, 5, dtype=np.int32), np.arange(6, dtype=np.int32),
                             bf16=True, seed=2101, temperatures=(0.8, 1.2), without_replacement=True)
    a = _run(chain, dev, seed=3)
    b = _run(chain, dev, seed=3, wor=True)
    assert all(np.array_equal(a[k], b[k]) for k in ("path", "path_len", "token"))


@pytest.mark.parametrize("wor", [False, True])
def test_largest_tree(dev, wor):
    """A tree of the largest size (1024 nodes), in both sibling modes: the
    walk's LDS arrays, child lists and duplicate check at their limit."""
    B, N, V = 4, 1024, 3000
    rng = np.random.default_rng(40)
    parents, depth = _random_tree(rng, N, branching=(2, 6))
    inp = make_tree_sample("n1024", B, V, parents, depth, bf16=True, seed=41, temperatures=(0.9,), zipf=0.0,
                           target_sigma=1.5, draft_sigma=(0.3, 1.0), without_replacement=wor)
    got = _run(inp, dev, seed=2, wor=wor)
    _compare(got, _oracle(inp, seed=2, wor=wor), "N=1024 wor=%d" % wor)
    assert np.all(got["path_len"] >= 1)


@pytest.mark.parametrize("wor", [False, True])
def test_deepest_paths(dev, wor):
    """1024-node trees at full depth, both sibling rules: a chain-shaped tree
    (depth 1023) with q = p at every node, so every child is accepted and the
    walk takes 1023 steps to the last node (the walk's step bound and path
    writes at their limit), and a deep, narrow random tree (1 or 2 children
    per node)."""
    N = 1024
    chain = np.arange(-1, N - 1, dtype=np.int32)
    depth = np.array(oracle.tree_depths(chain), np.int32)
    inp = make_tree_sample("chain1024", 2, 1500, chain, depth, bf16=True, seed=49, temperatures=(1.0,), zipf=0.0,
                           target_sigma=1.5, draft_sigma=(0.0, 0.0), without_replacement=wor)
    got = _run(inp, dev, seed=3, wor=wor)
    _compare(got, _oracle(inp, seed=3, wor=wor), "chain N=1024 wor=%d" % wor)
    assert np.all(got["path_len"] == N)
    rng = np.random.default_rng(50)
    parents, depth = _random_tree(rng, N, branching=(1, 2))
    inp = make_tree_sample("narrow1024", 3, 2000, parents, depth, bf16=False, seed=51, temperatures=(0.8, 1.0),
                           zipf=0.0, target_sigma=1.0, draft_sigma=(0.1, 0.4), without_replacement=wor)
    got = _run(inp, dev, seed=4, wor=wor)
    _compare(got, _oracle(inp, seed=4, wor=wor), "narrow N=1024 wor=%d" % wor)
    assert got["path_len"].max() >= 4


@pytest.mark.parametrize("wor", [False, True])
@pytest.mark.parametrize("bf16", [True, False])
def test_residual_without_mass(dev, bf16, wor):
    """Siblings whose residual has no mass. The root's draft row equals its
    target row (its one child is accepted); at that child the draft row equals
    the target row except at the first k of its three children's tokens,
    where the draft logit is -30 (too small to move any normalizer sum) and
    the target logit -60 (a about e^-30, never accepted at these seeds). Each
    such rejection leaves (p - q)_+ with no mass, so the target distribution
    stays p; a later sibling then has p(x) = q(x) and is accepted. With all
    three rejected the walk ends in a draw from p itself (i.i.d. siblings).
    Without replacement, a drawn sibling leaves q, so the second rejection's
    residual holds the first sibling's own p(x) alone: the target becomes that
    token, every later sibling is rejected and the walk emits it."""
    B, V = 12, 20000 if bf16 else 5003
    parents = np.array([-1, 0, 1, 1, 1, 2, 3], np.int32)
    depth = oracle.tree_depths(parents)
    inp = make_tree_sample("no_mass", B, V, parents, depth, bf16=bf16, seed=31, temperatures=(1.0, 0.8),
                           target_sigma=1.0, zipf=0.0)
    rng = np.random.default_rng(32)
    put = (lambda v: workloads.round_bf16(np.float32([v]))[0]) if bf16 else np.float32
    kk = np.zeros(B, np.int32)
    for b in range(B):
        inp.draft[b, 0] = inp.target[b, 0]
        inp.draft[b, 1] = inp.target[b, 1]
        xs = rng.choice(V, size=3, replace=False)
        inp.node_tokens[b, 2:5] = xs
        kk[b] = b % 3 + 1
        for x in xs[:kk[b]]:
            inp.target[b, 1, x] = put(-60.0)
            inp.draft[b, 1, x] = put(-30.0)
    ref = _oracle(inp, seed=3, wor=wor)
    got = _run(inp, dev, seed=3, wor=wor)
    _compare(got, ref, "no mass bf16=%s wor=%s" % (bf16, wor))
    assert np.all(got["path"][:, :2] == [0, 1])
    for b in range(B):
        k = kk[b]
        assert ref["rejections"][b] >= k
        assert ref["flags"][b] & oracle.FLAG_FALLBACK
        if wor and k >= 2:
            assert got["path_len"][b] == 2 and got["token"][b] == inp.node_tokens[b, 2]
        elif k < 3:
            assert got["path"][b, 2] == 2 + k  # the first sibling with p(x) = q(x)
        else:
            assert got["path_len"][b] == 2
