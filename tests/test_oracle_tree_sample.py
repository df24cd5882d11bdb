"""Pins of the oracle's sampled tree verification against what the pages and
the mathematics fix ([SB] "Tree Attention": multi-round rejection sampling).

No GPU. The pages' rule: test the children of a node one by one against the
current target distribution p, replacing p by the normalized residual
(p - q)_+ after each rejection, and draw the replacement from the final
residual when every child is rejected; each round is the single-candidate rule,
so the emitted token is distributed exactly as p. By default siblings are
read as i.i.d. draws from the draft distribution q at their parent (the
plainest reading). The pages also mention siblings drawn without
replacement, where q is renormalized over the candidates left; the oracle
and the library implement that variant too (without_replacement=True), and
it is pinned below by its own exact enumeration.
"""
import itertools
from fractions import Fraction

import numpy as np
from scipy import stats

import oracle


def _rule_law(p, q, k):
    """Exact law of (round of acceptance or None, emitted token) for one node
    with k children drawn i.i.d. from q, by enumerating every draw tuple and
    following the rule with rational arithmetic. Written from the rule's
    statement, independently of the C oracle."""
    V = len(p)
    # The target distribution before each round does not depend on which
    # tokens were drawn: p_1 = p, p_{j+1} = (p_j - q)_+ / ||.||_1.
    ps = [list(p)]
    for _ in range(k):
        r = [max(a - b, Fraction(0)) for a, b in zip(ps[-1], q)]
        z = sum(r)
        ps.append([x / z for x in r] if z > 0 else list(ps[-1]))
    law = {}
    for xs in itertools.product(range(V), repeat=k):
        w = Fraction(1)
        for x in xs:
            w *= q[x]
        if w == 0:
            continue
        still = Fraction(1)  # probability that rounds 1..j-1 all rejected
        for j, x in enumerate(xs):
            a = min(Fraction(1), ps[j][x] / q[x])
            key = (j, x)
            law[key] = law.get(key, Fraction(0)) + w * still * a
            still *= 1 - a
        for t in range(V):
            key = (None, t)
            law[key] = law.get(key, Fraction(0)) + w * still * ps[k][t]
    return law


def test_rule_is_lossless_by_exact_enumeration():
    """The emitted token's law equals p exactly, for 1 to 3 siblings (the
    pages: the proof for one candidate carries over to every round)."""
    cases = [
        ([Fraction(3, 10), Fraction(5, 10), Fraction(2, 10)], [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]),
        ([Fraction(1, 8), Fraction(1, 8), Fraction(3, 4)], [Fraction(6, 10), Fraction(3, 10), Fraction(1, 10)]),
        ([Fraction(1, 3), Fraction(1, 3), Fraction(1, 3)], [Fraction(1, 3), Fraction(1, 3), Fraction(1, 3)]),
    ]
    for p, q in cases:
        for k in (1, 2, 3):
            law = _rule_law(p, q, k)
            assert sum(law.values()) == 1
            emitted = [sum(v for (j, t), v in law.items() if t == s) for s in range(len(p))]
            assert emitted == p, (p, q, k, emitted)


def test_more_siblings_accept_more_often():
    """The chance that some child is accepted grows with the number of
    siblings (the pages: the point of branching)."""
    p = [Fraction(3, 10), Fraction(5, 10), Fraction(2, 10)]
    q = [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]
    acc = [sum(v for (j, t), v in _rule_law(p, q, k).items() if j is not None) for k in (1, 2, 3)]
    # one sibling: sum_v min(p, q) = 1 - TV(p, q)
    assert acc[0] == sum(min(a, b) for a, b in zip(p, q))
    assert acc[0] < acc[1] < acc[2] < 1


def _one_node_batch(rng, p_row_logits, q_row_logits, k, B, V):
    """B independent trials of a root with k leaf children drawn from q."""
    N = k + 1
    target = np.broadcast_to(np.asarray(p_row_logits, np.float32), (B, N, V)).copy()
    draft = np.broadcast_to(np.asarray(q_row_logits, np.float32), (B, N, V)).copy()
    q = np.exp(np.asarray(q_row_logits, np.float64))
    q /= q.sum()
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = rng.choice(V, size=(B, k), p=q)
    parents = np.array([-1] + [0] * k, np.int32)
    depth = np.array([0] + [1] * k, np.int32)
    return target, draft, parents, depth, tok


def test_oracle_emits_p_and_the_rule_rounds_chi_square():
    """The oracle's emitted first token follows p, and the round at which a
    child is accepted (or none) follows the exactly enumerated law."""
    rng = np.random.default_rng(11)
    V, k, B = 4, 3, 60000
    lp = np.log(np.array([0.1, 0.2, 0.3, 0.4]))
    lq = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    target, draft, parents, depth, tok = _one_node_batch(rng, lp, lq, k, B, V)
    o = oracle.verify_tree_sample(target, draft, parents, depth, tok, np.ones(B, np.float32), 1, seed=5)
    # p and q exactly as the oracle sees them (fp64 softmax of the stored fp32 logits)
    p64 = np.exp(np.float64(target[0, 0])) / np.exp(np.float64(target[0, 0])).sum()
    q64 = np.exp(np.float64(draft[0, 0])) / np.exp(np.float64(draft[0, 0])).sum()
    first = np.where(o["path_len"] >= 2, tok[np.arange(B), np.maximum(o["path"][:, 1], 0)], o["token"])
    counts = np.bincount(first, minlength=V)
    assert stats.chisquare(counts, p64 * B).pvalue > 1e-3
    # round of acceptance: path[1] - 1 (children are nodes 1..k in index order), k for none
    rounds = np.where(o["path_len"] >= 2, o["path"][:, 1] - 1, k)
    law = _rule_law([Fraction(float(x)) for x in p64], [Fraction(float(x)) for x in q64], k)
    exp_r = np.array([float(sum(v for (j, t), v in law.items() if j == r)) for r in range(k)] +
                     [float(sum(v for (j, t), v in law.items() if j is None))])
    assert stats.chisquare(np.bincount(rounds, minlength=k + 1), exp_r * B).pvalue > 1e-3
    # rejections counted: one per rejected sibling before the accepted one
    assert np.array_equal(o["rejections"], rounds)


def test_chain_shaped_tree_verifies_as_the_chain():
    """A tree in which every node has one child is the chain: same accepted
    count, same token, bit for bit (the accept uniform of the first sibling
    under node i is the chain's u_i; the noise of a draw at node i is the
    chain's noise at position i)."""
    rng = np.random.default_rng(3)
    B, G, V = 24, 5, 300
    N = G + 1
    target = rng.normal(0, 2.5, (B, N, V)).astype(np.float32)
    draft = np.zeros((B, N, V), np.float32)
    draft[:, :G] = target[:, :G] + rng.normal(0, 1.0, (B, G, V)).astype(np.float32)
    draft[:, G] = rng.normal(0, 1.0, (B, V)).astype(np.float32)  # a leaf row: never read
    T = np.array([0.6, 1.0, 1.7] * (B // 3), np.float32)
    ids = np.zeros((B, G), np.int32)
    for b in range(B):
        for i in range(G):
            y = np.float64(draft[b, i]) / T[b]
            q = np.exp(y - y.max())
            ids[b, i] = rng.choice(V, p=q / q.sum())
    ch = oracle.verify_sample(target, np.ascontiguousarray(draft[:, :G]), ids, T, seed=9, offset=2)
    parents = np.arange(-1, G, dtype=np.int32)
    depth = np.arange(0, N, dtype=np.int32)
    tok = np.concatenate([np.zeros((B, 1), np.int32), ids], axis=1)
    tr = oracle.verify_tree_sample(target, draft, parents, depth, tok, T, G, seed=9, offset=2)
    assert np.array_equal(tr["path_len"] - 1, ch["n"])
    assert np.array_equal(tr["token"], ch["tokens"][np.arange(B), ch["n"]])
    for b in range(B):
        assert list(tr["path"][b, :tr["path_len"][b]]) == list(range(tr["path_len"][b]))
    assert len(set(ch["n"].tolist())) > 2  # the case mixes early, late and no rejections


def test_draft_equal_to_target_accepts_the_first_child_everywhere():
    """q = p: every first child is accepted (a = 1), so the path follows first
    children down to a leaf, and the token is the bonus drawn there."""
    rng = np.random.default_rng(4)
    B, V = 6, 50
    parents = np.array([-1, 0, 0, 1, 1, 2, 3], np.int32)
    depth = oracle.tree_depths(parents)
    N = len(parents)
    target = rng.normal(0, 2, (B, N, V)).astype(np.float32)
    tok = rng.integers(0, V, (B, N)).astype(np.int32)
    o = oracle.verify_tree_sample(target, target.copy(), parents, depth, tok, np.ones(B, np.float32), 3, seed=1)
    for b in range(B):
        assert list(o["path"][b]) == [0, 1, 3, 6]
    assert np.all(o["rejections"] == 0)


def test_bad_inputs_are_marked():
    rng = np.random.default_rng(5)
    B, V = 3, 10
    parents = np.array([-1, 0, 0], np.int32)
    depth = oracle.tree_depths(parents)
    t = rng.normal(0, 1, (B, 3, V)).astype(np.float32)
    tok = np.array([[0, 1, 2], [0, 1, V], [0, 3, 4]], np.int32)
    o = oracle.verify_tree_sample(t, t.copy(), parents, depth, tok, np.array([1.0, 1.0, 0.0], np.float32), 1)
    assert list(o["path_len"]) == [o["path_len"][0], -1, -2] and o["path_len"][0] >= 1
    bad_tree = oracle.verify_tree_sample(t, t.copy(), np.array([-1, 0, 0], np.int32), np.array([0, 1, 2], np.int32),
                                         tok, np.ones(B, np.float32), 2)
    assert np.all(bad_tree["path_len"] == -3)


# ---------------------------------------------------------------------------
# Siblings drawn without replacement: each round's q is q over the tokens not
# drawn yet, renormalized (the page's variant).
# ---------------------------------------------------------------------------

def _rule_law_wor(p, q, k):
    """Exact law of (round of acceptance or None, emitted token) for k
    siblings drawn from q without replacement, enumerating every ordered draw
    of distinct tokens with rational arithmetic. Written from the rule's
    statement, independently of the C oracle."""
    V = len(p)

    def renorm_without(qj, x):
        left = 1 - qj[x]
        return [Fraction(0) if t == x else (v / left if left > 0 else v) for t, v in enumerate(qj)]

    law = {}
    for xs in itertools.permutations(range(V), k):
        # probability of this ordered draw
        w = Fraction(1)
        qj = list(q)
        for x in xs:
            w *= qj[x]
            qj = renorm_without(qj, x)
        if w == 0:
            continue
        # the rule along it
        pj, qj = list(p), list(q)
        still = Fraction(1)
        for j, x in enumerate(xs):
            a = min(Fraction(1), pj[x] / qj[x])
            law[(j, x)] = law.get((j, x), Fraction(0)) + w * still * a
            still *= 1 - a
            r = [max(u - v, Fraction(0)) for u, v in zip(pj, qj)]
            z = sum(r)
            if z > 0:
                pj = [u / z for u in r]
            qj = renorm_without(qj, x)
        for t in range(V):
            law[(None, t)] = law.get((None, t), Fraction(0)) + w * still * pj[t]
    return law


def test_without_replacement_rule_is_lossless_by_exact_enumeration():
    cases = [
        ([Fraction(3, 10), Fraction(5, 10), Fraction(2, 10)], [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]),
        ([Fraction(1, 8), Fraction(1, 8), Fraction(1, 4), Fraction(1, 2)],
         [Fraction(4, 10), Fraction(3, 10), Fraction(2, 10), Fraction(1, 10)]),
    ]
    for p, q in cases:
        for k in range(1, len(p) + 1):
            law = _rule_law_wor(p, q, k)
            assert sum(law.values()) == 1
            emitted = [sum(v for (j, t), v in law.items() if t == s) for s in range(len(p))]
            assert emitted == p, (p, q, k, emitted)
    # with one sibling the two rules coincide
    p, q = cases[0]
    assert _rule_law_wor(p, q, 1) == _rule_law(p, q, 1)


def _one_node_batch_wor(rng, lp, lq, k, B, V):
    N = k + 1
    target = np.broadcast_to(np.asarray(lp, np.float32), (B, N, V)).copy()
    draft = np.broadcast_to(np.asarray(lq, np.float32), (B, N, V)).copy()
    q = np.exp(np.asarray(lq, np.float64))
    q /= q.sum()
    tok = np.zeros((B, N), np.int32)
    for b in range(B):
        tok[b, 1:] = rng.choice(V, size=k, replace=False, p=q)
    parents = np.array([-1] + [0] * k, np.int32)
    depth = np.array([0] + [1] * k, np.int32)
    return target, draft, parents, depth, tok


def test_oracle_without_replacement_emits_p_and_the_rule_rounds_chi_square():
    rng = np.random.default_rng(12)
    V, k, B = 4, 3, 60000
    lp = np.log(np.array([0.1, 0.2, 0.3, 0.4]))
    lq = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    target, draft, parents, depth, tok = _one_node_batch_wor(rng, lp, lq, k, B, V)
    o = oracle.verify_tree_sample(target, draft, parents, depth, tok, np.ones(B, np.float32), 1, seed=6,
                                  without_replacement=True)
    p64 = np.exp(np.float64(target[0, 0])) / np.exp(np.float64(target[0, 0])).sum()
    q64 = np.exp(np.float64(draft[0, 0])) / np.exp(np.float64(draft[0, 0])).sum()
    first = np.where(o["path_len"] >= 2, tok[np.arange(B), np.maximum(o["path"][:, 1], 0)], o["token"])
    assert stats.chisquare(np.bincount(first, minlength=V), p64 * B).pvalue > 1e-3
    rounds = np.where(o["path_len"] >= 2, o["path"][:, 1] - 1, k)
    law = _rule_law_wor([Fraction(float(x)) for x in p64], [Fraction(float(x)) for x in q64], k)
    exp_r = np.array([float(sum(v for (j, t), v in law.items() if j == r)) for r in range(k)] +
                     [float(sum(v for (j, t), v in law.items() if j is None))])
    assert stats.chisquare(np.bincount(rounds, minlength=k + 1), exp_r * B).pvalue > 1e-3
    # the i.i.d. rule's round law differs here, so the test tells the two apart
    law_iid = _rule_law([Fraction(float(x)) for x in p64], [Fraction(float(x)) for x in q64], k)
    assert abs(float(law_iid.get((None, 0), 0)) - float(law.get((None, 0), 0))) > 1e-3 or \
        abs(sum(float(v) for (j, t), v in law_iid.items() if j == 1) -
            sum(float(v) for (j, t), v in law.items() if j == 1)) > 1e-3


def test_without_replacement_single_children_and_duplicates():
    """One child per node: the same outputs as the i.i.d. rule. Duplicate
    sibling tokens are a bad input without replacement."""
    rng = np.random.default_rng(13)
    B, V = 16, 50
    parents = np.array([-1, 0, 1, 2], np.int32)
    depth = oracle.tree_depths(parents)
    t = rng.normal(0, 2, (B, 4, V)).astype(np.float32)
    d = (t + rng.normal(0, 1, (B, 4, V))).astype(np.float32)
    tok = rng.integers(0, V, (B, 4)).astype(np.int32)
    a = oracle.verify_tree_sample(t, d, parents, depth, tok, np.ones(B, np.float32), 3, seed=2)
    b = oracle.verify_tree_sample(t, d, parents, depth, tok, np.ones(B, np.float32), 3, seed=2,
                                  without_replacement=True)
    assert all(np.array_equal(a[key], b[key]) for key in ("path", "path_len", "token"))
    par2 = np.array([-1, 0, 0], np.int32)
    tok2 = np.array([[0, 5, 5], [0, 5, 6]], np.int32)
    t2 = rng.normal(0, 1, (2, 3, V)).astype(np.float32)
    r = oracle.verify_tree_sample(t2, t2.copy(), par2, oracle.tree_depths(par2), tok2, np.ones(2, np.float32), 1,
                                  without_replacement=True)
    assert r["path_len"][0] == -1 and r["path_len"][1] >= 1
    r = oracle.verify_tree_sample(t2, t2.copy(), par2, oracle.tree_depths(par2), tok2, np.ones(2, np.float32), 1)
    assert r["path_len"][0] >= 1  # with replacement, repeats are fine
