"""Exact-rational enumeration of one speculative verify step.

TEST INFRASTRUCTURE ONLY. Pure Python over ``fractions.Fraction`` for tiny
vocabularies and draft lengths. It restates the rule of "7.6 Speculative
Decoding: Draft Models, Medusa, EAGLE & Lookahead" ("The rule", "The proof that
this is exact", "Extending to a chain of γ draft tokens"):

  * the drafter proposes x_i ~ q_i;
  * x_i is accepted with probability min(1, p_i(x_i) / q_i(x_i));
  * on the first rejection the replacement is drawn from (p_i - q_i)_+ / beta_i
    and the step ends;
  * if all gamma drafts are accepted the bonus token is drawn from p_gamma.

Every draft sequence, accept/reject outcome and replacement draw is enumerated
with its exact probability, so the result is the exact law of the step's output.
"""
from __future__ import annotations

from fractions import Fraction
from itertools import product


def residual(p, q):
    """(p - q)_+ and its mass beta (the residual normalizer)."""
    r = [max(Fraction(0), pv - qv) for pv, qv in zip(p, q)]
    return r, sum(r)


def accept_prob(p, q, x):
    """min(1, p(x) / q(x)) for a draft token with q(x) > 0."""
    return min(Fraction(1), Fraction(p[x]) / Fraction(q[x]))


def step_law(ps, qs):
    """Exact law of one verify step.

    ps: gamma+1 target distributions (lists of Fractions over V tokens);
    qs: gamma draft distributions. Returns {(n, tokens): probability}, where
    tokens are the n accepted drafts followed by the replacement or bonus.
    """
    gamma = len(qs)
    V = len(ps[0])
    law: dict[tuple, Fraction] = {}

    def add(key, w):
        if w:
            law[key] = law.get(key, Fraction(0)) + w

    for xs in product(range(V), repeat=gamma):
        w = Fraction(1)
        for i, x in enumerate(xs):
            w *= qs[i][x]
        if w == 0:
            continue
        reach = w  # probability of this draft AND reaching position i
        for i, x in enumerate(xs):
            a = accept_prob(ps[i], qs[i], x)
            r, beta = residual(ps[i], qs[i])
            if a < 1:
                for v in range(V):
                    if r[v]:
                        add((i, tuple(xs[:i]) + (v,)), reach * (1 - a) * r[v] / beta)
            reach *= a
            if reach == 0:
                break
        else:
            for v in range(V):
                add((gamma, tuple(xs) + (v,)), reach * ps[gamma][v])
    return law


def position_marginals(law, gamma, V):
    """P(reach position i) and P(token at position i = v | reach i) from a law."""
    reach = [Fraction(0)] * (gamma + 1)
    emit = [[Fraction(0)] * V for _ in range(gamma + 1)]
    for (n, toks), w in law.items():
        for i in range(n + 1):
            reach[i] += w
            emit[i][toks[i]] += w
    cond = [[e / reach[i] if reach[i] else None for e in emit[i]] for i in range(gamma + 1)]
    return reach, cond


def acceptance_rate(p, q):
    """alpha = sum_x min(p(x), q(x)) = 1 - TV(p, q)."""
    return sum(min(pv, qv) for pv, qv in zip(p, q))


def total_variation(p, q):
    return sum(abs(pv - qv) for pv, qv in zip(p, q)) / 2
