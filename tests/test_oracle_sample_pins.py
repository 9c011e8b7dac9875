"""Pins of the sampling-epilogue oracle to facts other than itself (no GPU).

Each ``check_*`` takes a SampleOracle and raises AssertionError on a
mismatch.  The tests run them against the real oracle, and the mutant test at
the end runs them against copies of ``oracle/verify_sample.c`` with planted
mistakes, each of which at least one pin must catch.

What pins what:

* candidate order: numpy's lexsort (value descending, then index) on rows
  full of ties;
* target probabilities: closed forms written out with ``math.exp`` for
  temperature 1 and 1/2, and hand-worked top-p prefixes (including a prefix
  whose mass equals top_p exactly, where "reaches" must mean >=);
* greedy: the argmax is emitted and accepted only when drafted;
* the accept test and the residual draw: hand-worked rows (the strict
  inequality u q < p, a residual with one token and one with two);
* exactness of the whole rule: over many draws of (drafted token ~ q, u, v)
  the emitted token's frequency matches p -- the property that makes
  speculative sampling exact, which fails for a wrong sign, a swapped test
  or a residual drawn from the wrong distribution.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle import sample as so_mod


def _softmax_closed(logits, T):
    w = [math.exp(l / T) for l in logits]
    z = sum(w)
    return [x / z for x in w]


def check_topk_vs_lexsort(so):
    rng = np.random.default_rng(1)
    lg = rng.integers(0, 12, size=(5, 300)).astype(np.float32) * 0.5 - 2.0
    for k in (1, 7, 32):
        idx, val = so.topk(lg, k)
        for m in range(lg.shape[0]):
            order = np.lexsort((np.arange(lg.shape[1]), -lg[m]))[:k]
            assert np.array_equal(idx[m], order), (k, m)
            assert np.array_equal(val[m], lg[m, order])


def check_topk_errors(so):
    lg = np.zeros((1, 40), dtype=np.float32)
    for bad in (0, 33, 41):
        with pytest.raises(ValueError):
            so.topk(lg, bad)


def _row(so, logits, k, T, top_p, d=0, didx=(), dq=(), u=0.0, v=0.0):
    lg = np.asarray([logits], dtype=np.float32)
    idx, val = so.topk(lg, k)
    kd = len(didx)
    out = so.sample(idx, val, T, top_p, [d],
                    np.asarray([didx], dtype=np.int32).reshape(1, kd),
                    np.asarray([dq], dtype=np.float64).reshape(1, kd),
                    [u], [v])
    return idx[0], out


def check_softmax_closed_form(so):
    logits = [3.0, 1.0, 0.0, -2.0]   # exact in fp32
    for T in (1.0, 0.5):
        idx, out = _row(so, logits, 4, T, 1.0)
        want = _softmax_closed(logits, T)
        assert list(idx) == [0, 1, 2, 3]
        assert np.allclose(out["p"][0], want, rtol=1e-12, atol=0), T
        assert abs(out["p"][0].sum() - 1.0) < 1e-12


def check_top_p_prefix(so):
    # probabilities 0.5, 0.3, 0.15, 0.05 (logits are their logs, in fp32)
    base = [0.5, 0.3, 0.15, 0.05]
    logits = [math.log(x) for x in base]
    for top_p, keep in ((0.79, 2), (0.81, 3), (1.0, 4), (0.2, 1)):
        _, out = _row(so, logits, 4, 1.0, top_p)
        want = np.array(base[:keep] + [0.0] * (4 - keep))
        want[:keep] /= sum(base[:keep])
        assert np.allclose(out["p"][0], want, atol=1e-6), (top_p, keep)
    # four equal logits: p = 1/4 exactly, so after two the mass is exactly
    # 1/2; top_p = 1/2 keeps two (the mass reaches top_p), not three
    _, out = _row(so, [1.0, 1.0, 1.0, 1.0], 4, 1.0, 0.5)
    assert np.array_equal(out["p"][0], [0.5, 0.5, 0.0, 0.0])
    # top-k itself truncates: k = 2 of four equal logits
    _, out = _row(so, [1.0, 1.0, 1.0, 1.0], 2, 1.0, 1.0)
    assert np.array_equal(out["p"][0], [0.5, 0.5])


def check_greedy(so):
    logits = [0.5, 2.5, 1.0, 2.0]
    for d, acc in ((1, 1), (3, 0), (0, 0)):
        idx, out = _row(so, logits, 3, 0.0, 1.0, d=d, didx=[d], dq=[0.9],
                        u=0.7, v=0.3)
        assert out["greedy"][0] == 1
        assert np.array_equal(out["p"][0], [1.0, 0.0, 0.0])
        assert out["accept"][0] == acc, d
        assert out["token"][0] == 1


def check_accept_rule_strict(so):
    # two equal logits: p = (1/2, 1/2); the draft is sure of token 0
    for u, acc in ((0.49, 1), (0.5, 0), (0.51, 0)):
        _, out = _row(so, [1.0, 1.0], 2, 1.0, 1.0, d=0, didx=[0], dq=[1.0],
                      u=u, v=0.9)
        assert out["accept"][0] == acc, u
        # residual max(p - q, 0) = (0, 1/2): token 1 whatever v is
        assert out["token"][0] == (0 if acc else 1)


def check_residual_draws(so):
    # p = (0.6, 0.4); q = 0.9 on token 0, 0.1 on token 1; u q(0) = 0.891
    _, out = _row(so, [math.log(0.6), math.log(0.4)], 2, 1.0, 1.0, d=0,
                  didx=[0, 1], dq=[0.9, 0.1], u=0.99, v=0.0)
    assert out["accept"][0] == 0 and out["token"][0] == 1
    # accepted below u = p/q = 2/3
    _, out = _row(so, [math.log(0.6), math.log(0.4)], 2, 1.0, 1.0, d=0,
                  didx=[0, 1], dq=[0.9, 0.1], u=0.6, v=0.0)
    assert out["accept"][0] == 1 and out["token"][0] == 0
    # p = (0.5, 0.3, 0.2); q = 0.7 on 0, 0.05 on 1, 0.25 on token 9 (outside
    # the candidates): residual (0, 0.25, 0.2), mass 0.45
    logits = [math.log(0.5), math.log(0.3), math.log(0.2), -30.0, -30.0,
              -30.0, -30.0, -30.0, -30.0, -30.0]
    for v, tok in ((0.5, 1), (0.6, 2), (0.0, 1), (0.999, 2)):
        _, out = _row(so, logits, 3, 1.0, 1.0, d=0, didx=[0, 1, 9],
                      dq=[0.7, 0.05, 0.25], u=0.99, v=v)
        assert out["accept"][0] == 0
        assert out["token"][0] == tok, v


def check_draft_token_outside_candidates(so):
    # p(d) = 0: never accepted; the residual is p itself (q and p disjoint):
    # candidates tokens 4 and 0, p = softmax(5, 2) = (0.953, 0.047)
    logits = [2.0, 1.0, 0.0, -1.0, 5.0]
    for v, tok in ((0.0, 4), (0.95, 4), (0.96, 0), (0.99, 0)):
        _, out = _row(so, logits, 2, 1.0, 1.0, d=3, didx=[3], dq=[1.0],
                      u=0.0, v=v)
        assert out["accept"][0] == 0
        assert out["token"][0] == tok
    # no draft list at all: q(d) = 0, accepted iff p(d) > 0
    _, out = _row(so, logits, 2, 1.0, 1.0, d=0, u=0.99)
    assert out["accept"][0] == 1 and out["token"][0] == 0
    _, out = _row(so, logits, 2, 1.0, 1.0, d=1, u=0.0, v=0.0)
    assert out["accept"][0] == 0 and out["token"][0] == 4


def check_monte_carlo_exactness(so):
    """Draft token d ~ q, u, v uniform: the emitted token is distributed as
    the target's p (speculative sampling is exact)."""
    rng = np.random.default_rng(7)
    V, k, kd, n = 40, 12, 8, 300_000
    logits = rng.normal(0, 1.5, size=V).astype(np.float32)
    order = np.lexsort((np.arange(V), -logits))
    # draft candidates: 5 inside the target's top-k, 3 outside it
    didx = np.concatenate([order[[0, 2, 3, 6, 9]], order[[15, 20, 30]]])
    dq = rng.dirichlet(np.ones(kd))
    d = didx[rng.choice(kd, size=n, p=dq)]
    idx, val = so.topk(logits[None, :], k)
    idx = np.repeat(idx, n, axis=0)
    val = np.repeat(val, n, axis=0)
    out = so.sample(idx, val, 0.9, 0.95, d, np.tile(didx, (n, 1)),
                    np.tile(dq, (n, 1)), rng.random(n), rng.random(n))
    p = out["p"][0]
    pos = {int(t): i for i, t in enumerate(idx[0])}
    slot = np.array([pos.get(int(t), k) for t in out["token"]])
    freq = np.bincount(slot, minlength=k + 1) / n
    assert freq[k] == 0.0, "a token outside the candidates was emitted"
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq[:k] - p) <= 5 * sigma + 1e-4), (freq[:k], p)


ALL_CHECKS = [check_topk_vs_lexsort, check_topk_errors,
              check_softmax_closed_form, check_top_p_prefix, check_greedy,
              check_accept_rule_strict, check_residual_draws,
              check_draft_token_outside_candidates,
              check_monte_carlo_exactness]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_sample_oracle_pin(check):
    check(so_mod.default())


# -------------------------------------------------------------- mutants

MUTANTS = {
    "residual_sign": ("r[i] = p[i] > qi ? p[i] - qi : 0.0;",
                      "r[i] = qi > p[i] ? qi - p[i] : 0.0;"),
    "residual_is_p": ("r[i] = p[i] > qi ? p[i] - qi : 0.0;", "r[i] = p[i];"),
    "accept_swapped": ("accept[m] = u[m] * qd < pd;",
                       "accept[m] = u[m] * pd < qd;"),
    "accept_not_strict": ("accept[m] = u[m] * qd < pd;",
                          "accept[m] = u[m] * qd <= pd;"),
    "no_renormalise": ("p[i] = i < n ? p[i] / kept : 0.0;",
                       "p[i] = i < n ? p[i] : 0.0;"),
    "top_p_strict": ("if (c >= top_p) {", "if (c > top_p) {"),
    "ties_larger_index_first": (
        "return (x->index > y->index) - (x->index < y->index);",
        "return (x->index < y->index) - (x->index > y->index);"),
    "temperature_ignored": ("(double)tv[0]) / T);", "(double)tv[0]));"),
    "draft_lookup_first": ("if (didx[j] == t) return dq[j];",
                           "if (didx[j] == t) return dq[0];"),
    "greedy_emits_draft": ("p[0] = 1.0;\n      for (int i = 1; i < k; ++i) p[i] = 0.0;",
                           "for (int i = 0; i < k; ++i) p[i] = 1.0 / k;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_sample_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    with open(oracle.SAMPLE_SOURCE) as fh:
        src = fh.read()
    assert src.count(find) == 1, f"mutation anchor not unique: {find!r}"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(find, repl))
    lib = oracle.compile_source(str(path), str(tmp_path / f"{name}.so"),
                                extra=("-Wno-error",))
    so = so_mod.SampleOracle(lib)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(so)
        except (AssertionError, ValueError):
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
