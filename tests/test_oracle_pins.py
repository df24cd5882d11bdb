"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU. Each test names the passage or fact it rests on; together they are
chosen so that a dropped term, a wrong sign, a swapped p/q, an off-by-one row
or a wrong sampler fails at least one of them.
"""
import json
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import brute, trees

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _logits_from_probs(rows, T=1.0):
    """fp32 logits whose softmax(l / T) is the given distribution."""
    return (T * np.log(np.asarray(rows, np.float64))).astype(np.float32)


def _softmax64(l, T):
    y = np.asarray(l, np.float64) / T
    y -= y.max()
    e = np.exp(y)
    return e / e.sum()


def _draw_ids(rng, q_rows, B):
    """x_i ~ q_i for B independent trials (the emulated drafter)."""
    gamma = len(q_rows)
    ids = np.empty((B, gamma), np.int32)
    for i, q in enumerate(q_rows):
        q = np.asarray(q, np.float64)
        ids[:, i] = rng.choice(len(q), size=B, p=q / q.sum())
    return ids


def _chi2_pvalue(observed: dict, expected_prob: dict, total: int, min_expected=5.0):
    """Chi-square goodness of fit; bins with small expectation are pooled."""
    keys = list(expected_prob)
    extra = sum(v for k, v in observed.items() if k not in expected_prob)
    assert extra == 0, "outcome outside the support of the exact law"
    exp_counts = np.array([float(expected_prob[k]) * total for k in keys])
    obs_counts = np.array([observed.get(k, 0) for k in keys], np.float64)
    small = exp_counts < min_expected
    if small.any():
        exp_counts = np.append(exp_counts[~small], exp_counts[small].sum())
        obs_counts = np.append(obs_counts[~small], obs_counts[small].sum())
    return stats.chisquare(obs_counts, exp_counts * obs_counts.sum() / exp_counts.sum()).pvalue


# --------------------------------------------------------------------------
# Philox4x32-10
# --------------------------------------------------------------------------

def test_philox_known_answers():
    """Random123's published known-answer vectors for Philox4x32-10."""
    for vec in _load("philox_kat.json")["vectors"]:
        ctr = [int(w, 16) for w in vec["ctr"]]
        key = [int(w, 16) for w in vec["key"]]
        out = [int(w, 16) for w in vec["out"]]
        assert list(oracle.philox4x32_10(ctr, key)) == out


ATEN_PROBE = r"""
#include <cstdio>
#include <cstdint>
#include <ATen/core/PhiloxRNGEngine.h>
int main() {
  // Draw the same blocks through ATen's engine: key = seed, counter = (offset
  // lo, offset hi, subsequence lo, subsequence hi), four words per block.
  for (uint64_t seed : {0ull, 0x0123456789abcdefull}) {
    for (uint64_t sub : {0ull, 7ull, 0xfffffffe00000003ull}) {
      for (uint64_t off : {0ull, 1ull, 41ull}) {
        at::Philox4_32 eng(seed, sub, off);
        unsigned w[4];
        for (int k = 0; k < 4; ++k) w[k] = eng();
        std::printf("%llu %llu %llu %u %u %u %u\n", (unsigned long long)seed,
                    (unsigned long long)sub, (unsigned long long)off, w[0], w[1], w[2], w[3]);
      }
    }
  }
  return 0;
}
"""


def test_philox_matches_an_independent_implementation(tmp_path):
    """Cross-check against the Philox engine shipped (as source) with PyTorch."""
    torch = pytest.importorskip("torch")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if shutil.which("g++") is None or not os.path.exists(os.path.join(inc, "ATen/core/PhiloxRNGEngine.h")):
        pytest.skip("no compiler or header")
    src = tmp_path / "aten_philox.cpp"
    exe = tmp_path / "aten_philox"
    src.write_text(ATEN_PROBE)
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("ATen header did not compile standalone: " + r.stderr[-300:])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    lines = out.strip().splitlines()
    assert len(lines) == 18
    for line in lines:
        seed, sub, off, *w = (int(t) for t in line.split())
        ctr = [off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        assert list(oracle.philox4x32_10(ctr, key)) == w


def test_uniform_maps_and_counter_layout():
    """u = (w >> 8) 2^-24 from word 0 of counter (0, i, b, 2*offset); Gumbel
    noise from word v%4 of counter (v/4, pos, b, 2*offset+1)."""
    seed, off = 0x1234_5678_9ABC_DEF0, 5
    key = [seed & 0xFFFFFFFF, seed >> 32]
    w = oracle.philox4x32_10([0, 3, 11, 2 * off], key)
    assert oracle.accept_uniform(seed, off, 11, 3) == (int(w[0]) >> 8) / 2.0 ** 24
    for v in (0, 1, 2, 3, 4, 1001):
        w = oracle.philox4x32_10([v // 4, 2, 9, 2 * off + 1], key)
        U = ((int(w[v % 4]) >> 8) + 0.5) / 2.0 ** 24
        assert oracle.gumbel(seed, off, 9, 2, v) == pytest.approx(-np.log(-np.log(U)), rel=1e-15)


def test_accept_uniforms_are_uniform():
    us = np.array([oracle.accept_uniform(0, 0, b, i) for b in range(4000) for i in range(4)])
    assert us.min() >= 0.0 and us.max() < 1.0
    assert stats.kstest(us, "uniform").pvalue > 1e-4


# --------------------------------------------------------------------------
# The accept rule: worked example, closed forms, exact law
# --------------------------------------------------------------------------

def _worked_example_rows():
    ex = _load("worked_example_dm.json")
    p_draft, q_draft = ex["p_of_draft"], ex["q_of_draft"]
    # Tokens A, B, C, D are ids 0..3; the other three of them get 0.01 each
    # and the rest of each row's mass goes to ids 4..5.
    ps, qs = [], []
    for i in range(4):
        p = np.full(6, 0.01)
        q = np.full(6, 0.01)
        p_x = p_draft[i] if p_draft[i] is not None else 0.3
        p[i], q[i] = p_x, q_draft[i]
        p[4], p[5] = (1 - p_x - 0.03) * 0.5, (1 - p_x - 0.03) * 0.5
        q[4], q[5] = (1 - q_draft[i] - 0.03) * 0.25, (1 - q_draft[i] - 0.03) * 0.75
        ps.append(p)
        qs.append(q)
    ps.append(np.full(6, 1 / 6))  # bonus row
    return ex, np.array(ps), np.array(qs)


def test_worked_example_accept_probabilities():
    """'The Algorithm' worked round: 0.68/0.72 -> 0.94, 0.70/0.65 -> 1.00,
    0.60/0.81 -> 0.74."""
    ex, ps, qs = _worked_example_rows()
    T = 1.0
    tgt = _logits_from_probs(ps, T)[None]
    dft = _logits_from_probs(qs, T)[None]
    ids = np.array([[0, 1, 2, 3]], np.int32)
    r = oracle.verify_sample(tgt, dft, ids, np.array([T], np.float32))
    a = r["accept_prob"][0]
    for i in range(3):
        assert round(a[i], 2) == pytest.approx(ex["printed_accept_prob"][i])
        assert a[i] == pytest.approx(min(1.0, ex["p_of_draft"][i] / ex["q_of_draft"][i]), abs=1e-6)


def test_worked_example_walk():
    """With uniforms that accept A and B and reject C, the step emits A, B and
    a replacement C' drawn from (p - q)_+ at C's position: three tokens."""
    ex, ps, qs = _worked_example_rows()
    tgt = _logits_from_probs(ps)[None]
    dft = _logits_from_probs(qs)[None]
    ids = np.array([[0, 1, 2, 3]], np.int32)
    u = np.array([[0.5, 0.99, 0.9, 0.0]])
    r = oracle.verify_sample(tgt, dft, ids, np.array([1.0], np.float32), u_override=u)
    n = int(r["n"][0])
    toks = r["tokens"][0]
    assert n == len(ex["printed_outcome"]["accepted"]) == 2
    assert n + 1 == ex["printed_outcome"]["emitted_count"]
    assert list(toks[:2]) == [0, 1] and list(toks[3:]) == [-1, -1]
    c_prime = int(toks[2])
    assert ps[2][c_prime] > qs[2][c_prime]  # only where p exceeds q
    assert c_prime != 2


def _random_rational_dist(rng, V, denom=12):
    w = rng.integers(0, 4, size=V)
    w[rng.integers(V)] += 1
    return [Fraction(int(x), int(w.sum())) for x in w]


@pytest.mark.parametrize("V,gamma", [(2, 1), (3, 2), (4, 2), (3, 3)])
def test_exact_law_emits_target_distribution(V, gamma):
    """Exhaustive exact enumeration ('The proof that this is exact'): at every
    position the emitted token is distributed as p_i given the step reached i,
    and the step moves on with probability sum_x min(p_i(x), q_i(x))."""
    rng = np.random.default_rng(V * 10 + gamma)
    for _ in range(4):
        ps = [_random_rational_dist(rng, V) for _ in range(gamma + 1)]
        qs = [_random_rational_dist(rng, V) for _ in range(gamma)]
        law = brute.step_law(ps, qs)
        assert sum(law.values()) == 1
        reach, cond = brute.position_marginals(law, gamma, V)
        assert reach[0] == 1
        for i in range(gamma + 1):
            if reach[i]:
                assert cond[i] == ps[i]
            if i < gamma:
                assert reach[i + 1] == reach[i] * brute.acceptance_rate(ps[i], qs[i])
                assert brute.acceptance_rate(ps[i], qs[i]) == 1 - brute.total_variation(ps[i], qs[i])


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_oracle_matches_exact_law(T):
    """The oracle's outcomes over many independent sequences (distinct b, so
    distinct Philox counters) fit the exact law of the enumeration."""
    rng = np.random.default_rng(7)
    V, gamma, B = 3, 2, 60000
    ps = [[Fraction(1, 2), Fraction(1, 3), Fraction(1, 6)], [Fraction(1, 5), Fraction(3, 5), Fraction(1, 5)],
          [Fraction(1, 4), Fraction(1, 4), Fraction(1, 2)]]
    qs = [[Fraction(1, 6), Fraction(1, 2), Fraction(1, 3)], [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]]
    law = brute.step_law(ps, qs)
    tgt = np.broadcast_to(_logits_from_probs([[float(x) for x in p] for p in ps], T), (B, gamma + 1, V)).copy()
    dft = np.broadcast_to(_logits_from_probs([[float(x) for x in q] for q in qs], T), (B, gamma, V)).copy()
    ids = _draw_ids(rng, [[float(x) for x in q] for q in qs], B)
    r = oracle.verify_sample(tgt, dft, ids, np.full(B, T, np.float32), seed=99, offset=3)
    obs = {}
    for b in range(B):
        n = int(r["n"][b])
        key = (n, tuple(int(t) for t in r["tokens"][b, :n + 1]))
        obs[key] = obs.get(key, 0) + 1
    assert _chi2_pvalue(obs, law, B) > 1e-4


def test_acceptance_equals_one_minus_tv():
    """Exercise 2(c) identity: E_{x~q}[min(1, p(x)/q(x))] = sum_x min(p, q) =
    1 - TV(p, q); fails if p and q are swapped in the ratio."""
    rng = np.random.default_rng(3)
    V = 6
    for T in (1.0, 0.8):
        l_p = rng.normal(0, 1.5, V).astype(np.float32)
        l_q = rng.normal(0, 1.5, V).astype(np.float32)
        tgt = np.broadcast_to(np.stack([l_p, l_p]), (V, 2, V)).copy()
        dft = np.broadcast_to(l_q[None], (V, 1, V)).copy()
        ids = np.arange(V, dtype=np.int32)[:, None]
        r = oracle.verify_sample(tgt, dft, ids, np.full(V, T, np.float32))
        p, q = _softmax64(l_p, float(np.float32(T))), _softmax64(l_q, float(np.float32(T)))
        alpha = float(np.sum(q * r["accept_prob"][:, 0]))
        assert alpha == pytest.approx(1 - 0.5 * np.abs(p - q).sum(), abs=1e-12)
        assert alpha == pytest.approx(np.minimum(p, q).sum(), abs=1e-12)


def test_expected_tokens_closed_form():
    """'The Algorithm': E[tokens per round] = (1 - alpha^(k+1)) / (1 - alpha);
    alpha = 0.8, k = 4 gives 3.36 as printed."""
    ex = _load("worked_example_dm.json")["expected_tokens_per_round"]
    alpha, k = ex["alpha"], ex["k"]
    E = (1 - alpha ** (k + 1)) / (1 - alpha)
    assert round(E, 2) == ex["printed"]
    # p = (0.9, 0.1), q = (0.7, 0.3): sum min = 0.8 at every position.
    B = 200000
    rng = np.random.default_rng(11)
    p, q = [0.9, 0.1], [0.7, 0.3]
    tgt = np.broadcast_to(_logits_from_probs([p] * (k + 1)), (B, k + 1, 2)).copy()
    dft = np.broadcast_to(_logits_from_probs([q] * k), (B, k, 2)).copy()
    ids = _draw_ids(rng, [q] * k, B)
    r = oracle.verify_sample(tgt, dft, ids, np.ones(B, np.float32), seed=5)
    emitted = r["n"].astype(np.float64) + 1
    sem = emitted.std() / np.sqrt(B)
    assert abs(emitted.mean() - E) < 4 * sem
    # per-position acceptance given the position was reached
    for i in range(k):
        reached = r["n"] >= i
        acc = (r["n"][reached] > i).mean()
        assert abs(acc - 0.8) < 4 * np.sqrt(0.16 / reached.sum())


def test_one_hot_draft():
    """Exercise 4's one-hot q: a = p(x), and the replacement is p without x."""
    rng = np.random.default_rng(5)
    V, B = 5, 40000
    l = rng.normal(0, 1.0, V).astype(np.float32)
    l[2] += 1.5
    x = 2
    tgt = np.broadcast_to(np.stack([l, l]), (B, 2, V)).copy()
    ids = np.full((B, 1), x, np.int32)
    r = oracle.verify_sample(tgt, None, ids, np.ones(B, np.float32), seed=8)
    p = _softmax64(l, 1.0)
    assert np.allclose(r["accept_prob"][:, 0], p[x], rtol=0, atol=1e-12)
    assert np.all(np.isnan(r["logz_draft"]))
    rej = r["n"] == 0
    assert abs(rej.mean() - (1 - p[x])) < 4 * np.sqrt(p[x] * (1 - p[x]) / B)
    repl = r["tokens"][rej, 0]
    assert not np.any(repl == x)
    assert np.allclose(r["residual_mass"][rej], 1 - p[x], atol=1e-12)
    expect = {(int(v),): p[v] / (1 - p[x]) for v in range(V) if v != x}
    obs = {}
    for v in repl:
        obs[(int(v),)] = obs.get((int(v),), 0) + 1
    assert _chi2_pvalue(obs, expect, int(rej.sum())) > 1e-4


def test_one_hot_residual_on_a_long_row():
    """Exercise 4's replacement p without x on a row of 37768 entries, heavy
    tokens spread along it (x among them): every token other than x comes out
    with p(v) / (1 - p(x)), counted per heavy token and per stretch of the
    rest."""
    rng = np.random.default_rng(41)
    K = 16384
    V, B = 2 * K + 5000, 12000
    l = (rng.normal(0, 1.0, V) - 6.0).astype(np.float32)
    heavy = {100: 2.0, 101: 3.0, K + 7: 1.5, K + 9000: 2.2, 2 * K + 4999: 1.8}
    for v, val in heavy.items():
        l[v] = val
    x = 101
    tgt = np.broadcast_to(np.stack([l, l]), (B, 2, V)).copy()
    ids = np.full((B, 1), x, np.int32)
    u = np.full((B, 1), 1.0 - 2.0 ** -24)  # every sequence rejects x
    r = oracle.verify_sample(tgt, None, ids, np.ones(B, np.float32), seed=17, u_override=u)
    assert np.all(r["n"] == 0)
    p = _softmax64(l, 1.0)
    res = p.copy()
    res[x] = 0.0
    res /= res.sum()
    tok = r["tokens"][:, 0]
    assert not np.any(tok == x)
    cats = {}
    for v in heavy:
        if v != x:
            cats[("tok", v)] = res[v]
    for j in range(3):
        lo, hi = j * K, min(V, (j + 1) * K)
        rest = res[lo:hi].sum() - sum(res[v] for v in heavy if lo <= v < hi)
        cats[("rest", j)] = rest
    obs = {}
    for v in tok:
        key = ("tok", int(v)) if int(v) in heavy else ("rest", int(v) // K)
        obs[key] = obs.get(key, 0) + 1
    assert _chi2_pvalue(obs, cats, B) > 1e-4
    assert np.allclose(r["residual_mass"], 1.0 - p[x], atol=1e-12)


def test_one_hot_residual_with_masked_stretch():
    """With every entry of the first 16384 but x at -inf, no replacement comes
    from there, and both later stretches are reached."""
    K = 16384
    V, B = 2 * K + 8000, 400
    l = np.full(V, -np.inf, np.float32)
    l[5] = 4.0  # x
    l[K:] = np.random.default_rng(3).normal(0, 1.0, V - K).astype(np.float32)
    tgt = np.broadcast_to(np.stack([l, l]), (B, 2, V)).copy()
    ids = np.full((B, 1), 5, np.int32)
    u = np.full((B, 1), 1.0 - 2.0 ** -24)
    r = oracle.verify_sample(tgt, None, ids, np.ones(B, np.float32), seed=2, u_override=u)
    assert np.all(r["n"] == 0)
    assert np.all(r["tokens"][:, 0] >= K)
    assert (r["tokens"][:, 0] >= 2 * K).any() and (r["tokens"][:, 0] < 2 * K).any()


def test_bonus_draw_follows_p_of_last_row():
    """With q = p every draft is accepted; the bonus token is then a draw from
    p of row gamma (not of any other row)."""
    rng = np.random.default_rng(12)
    V, B, T = 16, 100000, 0.9
    l0 = rng.normal(0, 1.0, V).astype(np.float32)
    l1 = rng.normal(0, 1.0, V).astype(np.float32)
    tgt = np.broadcast_to(np.stack([l0, l1]), (B, 2, V)).copy()
    dft = np.broadcast_to(l0[None], (B, 1, V)).copy()
    ids = rng.integers(0, V, size=(B, 1)).astype(np.int32)
    r = oracle.verify_sample(tgt, dft, ids, np.full(B, T, np.float32), seed=21)
    assert np.all(r["n"] == 1)
    p1 = _softmax64(l1, T)
    obs = {}
    for v in r["tokens"][:, 1]:
        obs[(int(v),)] = obs.get((int(v),), 0) + 1
    assert _chi2_pvalue(obs, {(v,): p1[v] for v in range(V)}, B) > 1e-4


def test_residual_draw_follows_positive_part():
    """Forced rejections: the replacement follows (p - q)_+ / beta, and beta is
    the residual mass."""
    rng = np.random.default_rng(13)
    V, B, T = 12, 100000, 1.0
    lp = rng.normal(0, 1.0, V).astype(np.float32)
    lq = rng.normal(0, 1.0, V).astype(np.float32)
    p, q = _softmax64(lp, T), _softmax64(lq, T)
    x = int(np.argmax(q - p))  # p(x) < q(x): a < 1
    tgt = np.broadcast_to(np.stack([lp, lp]), (B, 2, V)).copy()
    dft = np.broadcast_to(lq[None], (B, 1, V)).copy()
    ids = np.full((B, 1), x, np.int32)
    u = np.full((B, 1), 1.0 - 2.0 ** -24)
    r = oracle.verify_sample(tgt, dft, ids, np.full(B, T, np.float32), seed=4, u_override=u)
    assert np.all(r["n"] == 0)
    res = np.maximum(p - q, 0.0)
    assert np.allclose(r["residual_mass"], res.sum(), atol=1e-12)
    obs = {}
    for v in r["tokens"][:, 0]:
        obs[(int(v),)] = obs.get((int(v),), 0) + 1
    expect = {(v,): res[v] / res.sum() for v in range(V) if res[v] > 0}
    assert _chi2_pvalue(obs, expect, B) > 1e-4


def test_temperature_divides_logits():
    """softmax(l / T): scaling logits and temperature together changes nothing
    (bitwise, since both scalings are by a power of two)."""
    inp_rng = np.random.default_rng(9)
    B, gamma, V = 64, 3, 50
    tgt = inp_rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    dft = (tgt[:, :gamma] + inp_rng.normal(0, 1, (B, gamma, V))).astype(np.float32)
    ids = inp_rng.integers(0, V, (B, gamma)).astype(np.int32)
    T = np.full(B, 0.7, np.float32)
    a = oracle.verify_sample(tgt, dft, ids, T, seed=1)
    b = oracle.verify_sample(tgt * 2, dft * 2, ids, T * 2, seed=1)
    assert np.array_equal(a["tokens"], b["tokens"]) and np.array_equal(a["n"], b["n"])
    assert np.array_equal(a["accept_prob"], b["accept_prob"])
    c = oracle.verify_sample(tgt, dft, ids, np.full(B, 1.4, np.float32), seed=1)
    assert not np.array_equal(a["accept_prob"], c["accept_prob"])


def test_bf16_decode_is_exact():
    """bf16 bit patterns decode to the fp32 values they stand for."""
    from workloads import bf16_to_f32, round_bf16
    pats = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], np.uint16)
    vals = bf16_to_f32(pats)
    assert list(vals[:4]) == [1.0, -2.0, 0.0, -0.0]
    assert vals[4] == np.float32(3.3895314e38) and vals[6] == np.float32(3.140625)
    rng = np.random.default_rng(2)
    B, gamma, V = 32, 3, 300
    t16 = round_bf16(rng.normal(0, 3, (B, gamma + 1, V)).astype(np.float32))
    d16 = round_bf16(rng.normal(0, 3, (B, gamma, V)).astype(np.float32))
    ids = rng.integers(0, V, (B, gamma)).astype(np.int32)
    T = np.where(np.arange(B) % 3 == 0, 0.0, 0.8).astype(np.float32)
    a = oracle.verify_sample(t16, d16, ids, T, seed=3)
    b = oracle.verify_sample(bf16_to_f32(t16), bf16_to_f32(d16), ids, T, seed=3)
    for k in ("tokens", "n", "accept_prob", "logz_target"):
        assert np.array_equal(a[k], b[k], equal_nan=True)


# --------------------------------------------------------------------------
# Greedy
# --------------------------------------------------------------------------

def test_greedy_ties_and_alignment():
    """Row i verifies draft i; row gamma gives the bonus; ties go to the lowest
    index ('Copying, verified against plain greedy': row j predicts token j+1)."""
    V, gamma = 8, 3
    tgt = np.zeros((1, gamma + 1, V), np.float32)
    for i in range(gamma + 1):
        tgt[0, i, i + 1] = 5.0
    ids = np.array([[1, 2, 3]], np.int32)
    r = oracle.verify_greedy(tgt, ids)
    assert r["n"][0] == 3 and list(r["tokens"][0]) == [1, 2, 3, 4]
    shifted = np.array([[2, 3, 4]], np.int32)  # aligned to the wrong rows
    r = oracle.verify_greedy(tgt, shifted)
    assert r["n"][0] == 0 and list(r["tokens"][0]) == [1, -1, -1, -1]
    tie = np.zeros((1, 2, V), np.float32)
    tie[0, 0, [3, 5]] = 2.0
    tie[0, 1, [6, 7]] = 1.0
    assert list(oracle.verify_greedy(tie, np.array([[5]], np.int32))["tokens"][0]) == [3, -1]
    assert list(oracle.verify_greedy(tie, np.array([[3]], np.int32))["tokens"][0]) == [3, 6]


def test_greedy_equals_plain_argmax_chain():
    """At temperature 0 the emitted tokens are the plain argmax chain up to and
    including the first disagreement (byte-identical to greedy decoding)."""
    rng = np.random.default_rng(4)
    B, gamma, V = 200, 5, 40
    tgt = rng.normal(0, 1, (B, gamma + 1, V)).astype(np.float32)
    g = tgt.argmax(axis=2)
    ids = np.where(rng.random((B, gamma)) < 0.7, g[:, :gamma], rng.integers(0, V, (B, gamma))).astype(np.int32)
    r = oracle.verify_greedy(tgt, ids)
    for b in range(B):
        n = int(r["n"][b])
        assert list(r["tokens"][b, :n + 1]) == list(g[b, :n + 1])
        assert n == gamma or ids[b, n] != g[b, n]
        assert all(ids[b, :n] == g[b, :n])
    s = oracle.verify_sample(tgt, tgt[:, :gamma].copy(), ids, np.zeros(B, np.float32))
    assert np.array_equal(s["tokens"], r["tokens"]) and np.array_equal(s["n"], r["n"])


def test_sampled_rule_tends_to_greedy_as_temperature_vanishes():
    """With well separated logits, T -> 0 makes p and q point masses and the
    sampled rule reduces to argmax matching."""
    rng = np.random.default_rng(6)
    B, gamma, V = 100, 4, 20
    tgt = (rng.permutation(V * (gamma + 1) * B).reshape(B, gamma + 1, V) % V).astype(np.float32)
    dft = (rng.permutation(V * gamma * B).reshape(B, gamma, V) % V).astype(np.float32)
    for b in range(B):
        for i in range(gamma + 1):
            tgt[b, i] = rng.permutation(V)
        for i in range(gamma):
            dft[b, i] = rng.permutation(V)
    g = tgt.argmax(2)
    ids = np.where(rng.random((B, gamma)) < 0.6, g[:, :gamma], dft.argmax(2)).astype(np.int32)
    dft2 = dft.copy()
    for b in range(B):
        for i in range(gamma):  # the drafter's own argmax is the drafted id
            dft2[b, i, ids[b, i]] = V + 1
    cold = oracle.verify_sample(tgt, dft2, ids, np.full(B, 0.01, np.float32), seed=2)
    greedy = oracle.verify_greedy(tgt, ids)
    assert np.array_equal(cold["n"], greedy["n"])
    assert np.array_equal(cold["tokens"], greedy["tokens"])


# --------------------------------------------------------------------------
# Per-sequence errors
# --------------------------------------------------------------------------

def test_bad_inputs_are_reported_per_sequence():
    rng = np.random.default_rng(1)
    B, gamma, V = 4, 2, 10
    tgt = rng.normal(0, 1, (B, gamma + 1, V)).astype(np.float32)
    dft = rng.normal(0, 1, (B, gamma, V)).astype(np.float32)
    ids = rng.integers(0, V, (B, gamma)).astype(np.int32)
    ids[1, 1] = V
    T = np.array([1.0, 1.0, -0.5, np.nan], np.float32)
    r = oracle.verify_sample(tgt, dft, ids, T)
    assert r["n"][0] >= 0
    assert r["n"][1] == oracle.SEQ_BAD_TOKEN and np.all(r["tokens"][1] == -1)
    assert r["n"][2] == oracle.SEQ_BAD_TEMPERATURE and r["n"][3] == oracle.SEQ_BAD_TEMPERATURE


# --------------------------------------------------------------------------
# Trees
# --------------------------------------------------------------------------

def test_tree_depths_printed():
    """build_tree_attn's printed position ids for [root, A, B, A1, A2, B1, B2]."""
    g = _load("tree_depths_sb.json")
    assert list(oracle.tree_depths(g["parents"])) == g["printed_depths"]
    assert trees.depths(g["parents"]) == g["printed_depths"]


def test_tree_mask_printed():
    """tree_mask.py's printed ancestor mask and its 4 / 9 / 20 counts."""
    g = _load("tree_mask_ss.json")
    assert trees.ancestor_mask(g["parents"]).tolist() == g["printed_mask"]
    par = g["parents"]
    leaves = [i for i in range(len(par)) if i not in par]
    assert len(leaves) == g["printed_counts"]["candidate_paths"]
    assert len(par) == g["printed_counts"]["tree_positions"]
    assert sum(trees.depths(par)[l] + 1 for l in leaves) == g["printed_counts"]["separate_positions"]


def _tree_logits_with_argmax(argmax_of, V):
    rows = np.zeros((len(argmax_of), V), np.float32)
    for i, g in enumerate(argmax_of):
        rows[i, g] = 1.0
    return rows


@pytest.mark.parametrize("parents", [[-1, 0, 0, 1, 2], [-1, 0, 1, 1, 0, 4], [-1, 0, 0, 0, 1, 1]])
def test_tree_walk_matches_brute_force(parents):
    """Exhaustive over node tokens and row argmaxes on V = 2: the oracle's
    path is the longest root path whose every token equals its parent's
    argmax (smallest final index on ties)."""
    import itertools
    N, V = len(parents), 2
    depth = trees.depths(parents)
    cases_t, cases_tok, expect = [], [], []
    for argmaxes in itertools.product(range(V), repeat=N):
        for toks in itertools.product(range(V), repeat=N - 1):
            tok = [0] + list(toks)
            cases_t.append(_tree_logits_with_argmax(argmaxes, V))
            cases_tok.append(tok)
            expect.append((trees.longest_valid_path(parents, tok, argmaxes), argmaxes))
    tgt = np.stack(cases_t)
    r = oracle.verify_tree(tgt, parents, depth, np.array(cases_tok), max(depth))
    for b, (path, argmaxes) in enumerate(expect):
        L = int(r["path_len"][b])
        assert list(r["path"][b, :L]) == path
        assert all(x == -1 for x in r["path"][b, L:])
        assert r["bonus"][b] == argmaxes[path[-1]]


def test_chain_shaped_tree_equals_greedy_chain():
    rng = np.random.default_rng(8)
    B, gamma, V = 100, 4, 30
    tgt = rng.normal(0, 1, (B, gamma + 1, V)).astype(np.float32)
    g = tgt.argmax(2)
    ids = np.where(rng.random((B, gamma)) < 0.7, g[:, :gamma], rng.integers(0, V, (B, gamma))).astype(np.int32)
    parents = [-1] + list(range(gamma))
    depth = list(range(gamma + 1))
    tok = np.concatenate([np.zeros((B, 1), np.int32), ids], axis=1)
    t = oracle.verify_tree(tgt, parents, depth, tok, gamma)
    c = oracle.verify_greedy(tgt, ids)
    assert np.array_equal(t["path_len"] - 1, c["n"])
    for b in range(B):
        n = int(c["n"][b])
        assert list(t["path"][b, :n + 1]) == list(range(n + 1))
        assert t["bonus"][b] == c["tokens"][b, n]


def test_tree_longest_path_vs_first_match_walk():
    """Two matching siblings: Exercise 5's walk takes the first, the longest-path
    rule the one with the deeper surviving subtree."""
    V = 4
    parents = [-1, 0, 0, 2]
    depth = [0, 1, 1, 2]
    rows = _tree_logits_with_argmax([1, 3, 2, 0], V)
    tok = np.array([[0, 1, 1, 2]], np.int32)  # nodes 1 and 2 both match argmax(root)=1
    r = oracle.verify_tree(rows[None], parents, depth, tok, 2)
    assert list(r["path"][0]) == [0, 2, 3] and r["bonus"][0] == 0
    assert r["first_match_node"][0] == 1


def test_malformed_tree_reported():
    V = 3
    rows = np.zeros((1, 3, V), np.float32)
    tok = np.zeros((1, 3), np.int32)
    for parents, depth in (([-1, 0, 2], [0, 1, 2]), ([-1, 0, 0], [0, 1, 2]), ([0, 0, 1], [0, 1, 2])):
        r = oracle.verify_tree(rows, parents, depth, tok, 2)
        assert r["path_len"][0] == oracle.SEQ_BAD_TREE and r["bonus"][0] == -1
    r = oracle.verify_tree(rows, [-1, 0, 1], [0, 1, 2], tok, 1)
    assert r["path_len"][0] == oracle.SEQ_BAD_TREE


def test_accept_test_is_strict():
    """'accept with probability a': with u in [0, 1) the test is u < a, so a
    draft with a = 0 is never accepted, not even by u = 0, and a = 1 always is."""
    V = 4
    tgt = np.zeros((2, 2, V), np.float32)
    tgt[:, 0, 1] = -1000.0  # p(1) underflows to exactly 0 in the ratio
    dft = np.zeros((2, 1, V), np.float32)
    ids = np.array([[1], [2]], np.int32)
    u = np.array([[0.0], [1.0 - 2.0 ** -24]])
    r = oracle.verify_sample(tgt, dft, ids, np.ones(2, np.float32), u_override=u)
    assert r["accept_prob"][0, 0] == 0.0 and r["n"][0] == 0
    assert r["accept_prob"][1, 0] == 1.0 and r["n"][1] == 1


def _tokens_histogram(col):
    obs = {}
    for v in col:
        obs[(int(v),)] = obs.get((int(v),), 0) + 1
    return obs


def test_empty_residual_falls_back_to_p():
    """An empty residual (p <= q everywhere, reachable only when p = q up to
    rounding) makes the repository's fallback draw the correction from p at
    the rejected row, with the same noise. Pinned two ways: q = p exactly with
    a forced rejection (u = 1 is not below a = 1), and an input where the
    drafted token's draft logit differs by an amount no fp64 sum can hold
    (so p and q agree bit for bit everywhere else and a is about e^-60). The
    draws must follow p of the rejected row, not of another row."""
    rng = np.random.default_rng(31)
    V, B, T = 10, 100000, 0.9
    rows = rng.normal(0, 1.0, (3, V)).astype(np.float32)
    # q = p on row 1, forced rejection there after an accepted row 0.
    tgt = np.broadcast_to(rows, (B, 3, V)).copy()
    dft = np.broadcast_to(rows[:2], (B, 2, V)).copy()
    ids = np.broadcast_to(np.array([[3, 5]], np.int32), (B, 2)).copy()
    u = np.broadcast_to(np.array([[0.0, 1.0]]), (B, 2)).copy()
    r = oracle.verify_sample(tgt, dft, ids, np.full(B, T, np.float32), seed=5, u_override=u)
    assert np.all(r["n"] == 1)
    assert np.all(r["flags"] & oracle.FLAG_FALLBACK)
    assert np.all(r["residual_mass"] == 0.0)
    p1 = _softmax64(rows[1], T)
    assert _chi2_pvalue(_tokens_histogram(r["tokens"][:, 1]), {(v,): p1[v] for v in range(V)}, B) > 1e-4
    # The row the draw reads is the rejected one: row 2's law is rejected.
    p2 = _softmax64(rows[2], T)
    assert _chi2_pvalue(_tokens_histogram(r["tokens"][:, 1]), {(v,): p2[v] for v in range(V)}, B) < 1e-9
    # Rounding construction with the accept uniforms of the generator.
    x = 4
    tgt2 = np.broadcast_to(rows[:2], (B, 2, V)).copy()
    dft2 = np.broadcast_to(rows[:1], (B, 1, V)).copy()
    tgt2[:, 0, x] = -100.0
    dft2[:, 0, x] = -40.0
    ids2 = np.full((B, 1), x, np.int32)
    r2 = oracle.verify_sample(tgt2, dft2, ids2, np.full(B, 1.0, np.float32), seed=6)
    assert np.all(r2["n"] == 0) and np.all(r2["flags"] & oracle.FLAG_FALLBACK)
    assert np.all(r2["accept_prob"][:, 0] < 1e-25)
    p0 = _softmax64(tgt2[0, 0], 1.0)
    expect = {(v,): p0[v] for v in range(V) if p0[v] > 1e-12}
    assert _chi2_pvalue(_tokens_histogram(r2["tokens"][:, 0]), expect, B) > 1e-4


def test_tree_zero_mass_residual_leaves_p():
    """Sampled trees: after a rejection whose residual has zero mass (the same
    rounding construction as for chains: the child's draft logit is below what
    an fp64 sum can hold, so p and q agree elsewhere), the target distribution
    stays p; with every child rejected the token is then a draw from p at the
    node."""
    rng = np.random.default_rng(32)
    V, B, T = 10, 60000, 1.0
    parents = np.array([-1, 0], np.int32)
    depth = np.array([0, 1], np.int32)
    row = rng.normal(0, 1.0, V).astype(np.float32)
    x = 7
    tgt = np.broadcast_to(np.stack([row, row]), (B, 2, V)).copy()
    dft = tgt.copy()
    tgt[:, 0, x] = -100.0
    dft[:, 0, x] = -40.0
    tok = np.zeros((B, 2), np.int32)
    tok[:, 1] = x
    r = oracle.verify_tree_sample(tgt, dft, parents, depth, tok, np.full(B, T, np.float32), 1, seed=9)
    assert np.all(r["path_len"] == 1) and np.all(r["rejections"] == 1)
    assert np.all(r["flags"] & oracle.FLAG_FALLBACK)
    p0 = _softmax64(tgt[0, 0], T)
    expect = {(v,): p0[v] for v in range(V) if p0[v] > 1e-12}
    assert _chi2_pvalue(_tokens_histogram(r["token"]), expect, B) > 1e-4


def test_masked_entries_have_probability_zero():
    """-inf logits are tokens of probability 0 ([SB] "A From-Scratch
    Implementation" asks for care when a probability is tiny): the accept
    probability and log-normalizer equal those of the vocabulary with the
    masked entries removed; a drafted token with p(x) = 0 gets a = 0, one with
    q(x) = 0 gets a = 1, and a row with one finite entry is one-hot there."""
    rng = np.random.default_rng(33)
    V, Vr = 12, 8
    keep = np.array([0, 1, 3, 4, 6, 7, 9, 11])
    tgt = rng.normal(0, 1.5, (1, 3, V)).astype(np.float32)
    dft = rng.normal(0, 1.5, (1, 2, V)).astype(np.float32)
    masked = np.setdiff1d(np.arange(V), keep)
    tgt[:, :, masked] = -np.inf
    dft[:, :, masked] = -np.inf
    ids = np.array([[keep[2], keep[5]]], np.int32)
    T = np.array([0.8], np.float32)
    full = oracle.verify_sample(tgt, dft, ids, T, seed=1)
    red = oracle.verify_sample(np.ascontiguousarray(tgt[:, :, keep]), np.ascontiguousarray(dft[:, :, keep]),
                               np.array([[2, 5]], np.int32), T, seed=1)
    assert np.allclose(full["accept_prob"], red["accept_prob"], rtol=0, atol=1e-15)
    assert np.allclose(full["logz_target"], red["logz_target"], rtol=0, atol=1e-15)
    assert np.allclose(full["logz_draft"], red["logz_draft"], rtol=0, atol=1e-15)
    # p(x) = 0 and q(x) = 0.
    t2 = rng.normal(0, 1.0, (2, 2, V)).astype(np.float32)
    d2 = rng.normal(0, 1.0, (2, 1, V)).astype(np.float32)
    t2[0, 0, 5] = -np.inf
    d2[1, 0, 6] = -np.inf
    r = oracle.verify_sample(t2, d2, np.array([[5], [6]], np.int32), np.ones(2, np.float32),
                             u_override=np.array([[0.0], [1.0 - 2.0 ** -24]]))
    assert r["accept_prob"][0, 0] == 0.0 and r["n"][0] == 0 and r["tokens"][0, 0] != 5
    assert r["accept_prob"][1, 0] == 1.0 and r["n"][1] == 1
    # One finite entry: p is one-hot, its token is always accepted and the
    # bonus row's single finite entry is always drawn.
    t3 = np.full((4, 2, V), -np.inf, np.float32)
    t3[:, 0, 2] = 1.5
    t3[:, 1, 9] = -3.0
    d3 = rng.normal(0, 1.0, (4, 1, V)).astype(np.float32)
    r3 = oracle.verify_sample(t3, d3, np.full((4, 1), 2, np.int32), np.ones(4, np.float32), seed=3)
    assert np.all(r3["n"] == 1) and np.all(r3["tokens"][:, 1] == 9)
    assert np.all(r3["logz_target"][:, 0] == 1.5)


def test_rows_without_a_distribution_are_reported():
    """The repository's contract for sampled sequences: every row the accept
    tests read must define softmax(row / T) (an entry above -inf, none NaN or
    +inf), and a bonus row must have a finite entry to draw from; otherwise the
    sequence gets code -5 and tokens -1. Greedy sequences take the argmax of
    anything but NaN (+inf is the largest value)."""
    rng = np.random.default_rng(34)
    V = 16
    B = 6
    tgt = rng.normal(0, 1.0, (B, 3, V)).astype(np.float32)
    dft = rng.normal(0, 1.0, (B, 2, V)).astype(np.float32)
    tgt[0, 1, 3] = np.inf          # target row 1
    dft[1, 0, 4] = np.nan          # draft row 0
    tgt[2, 0, :] = -np.inf         # a row with no finite entry
    tgt[3, 2, :] = -np.inf         # bonus row without a finite entry
    tgt[4, 2, 5] = np.inf          # +inf in the bonus row only
    ids = rng.integers(0, V, size=(B, 2)).astype(np.int32)
    u = np.zeros((B, 2))           # accept every scored draft
    r = oracle.verify_sample(tgt, dft, ids, np.ones(B, np.float32), seed=2, u_override=u)
    assert r["n"].tolist()[:4] == [oracle.SEQ_BAD_LOGITS] * 4
    assert np.all(r["tokens"][:4] == -1)
    # +inf in the bonus row: the row's law puts all mass on it.
    assert r["n"][4] == 2 and r["tokens"][4, 2] == 5
    assert r["n"][5] == 2
    # Greedy: +inf is the argmax, lowest index among equal values.
    g = tgt.copy()
    g[0, 0, :] = -np.inf
    g[0, 0, [6, 9]] = np.inf
    rg = oracle.verify_sample(g, None, np.array([[6, 1]] * B, np.int32), np.zeros(B, np.float32))
    assert rg["n"][0] >= 1 and rg["tokens"][0, 0] == 6
