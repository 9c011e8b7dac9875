"""Pins of the Gated DeltaNet state oracle to facts other than itself (no GPU).

Each ``check_*`` takes a GdnOracle and raises AssertionError on a mismatch.
The tests run them against the real oracle; the mutant test at the end runs
them against copies of ``oracle/gdn_state.c`` with planted mistakes, each of
which at least one pin must catch.

What pins what (the gated delta rule S <- a S (I - b k k^T) + b v k^T,
output o = S q after the update):

* one-hot keys k = e_j make every column of S evolve on its own: column j
  becomes a (1 - b) col + b v, every other column a col.  That scalar
  recurrence, walked along the path by hand, fixes the gate, the strength,
  the sign of the projection, the value term and the order of the tokens,
  for the commit and for each tree node's output (whose path is read off
  the parent pointers here, independently of the oracle);
* the delta property: with b = 1 and a unit key the new state maps k to v
  exactly, whatever the gate, and scales directions orthogonal to k by a;
* b = 0 is pure decay, a = 0 forgets the old state;
* the same key written twice: the later value wins;
* key heads: value head h reads key head h / (H / Hk);
* a tree node's output equals the committed state of its own path applied
  to its query (the tree output is that state by definition).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import gdn as gdn_mod


def _one_hot_case(rng, L, M, H, Hk, d):
    """Keys one-hot per (layer, node, key head); gates and values random."""
    S = rng.normal(size=(L, H, d, d))
    j = rng.integers(0, d, size=(L, M, Hk))
    # make repeats likely: draw from a few columns only
    j = j % 3
    k = np.zeros((L, M, Hk, d), dtype=np.float32)
    for l in range(L):
        for n in range(M):
            for g in range(Hk):
                k[l, n, g, j[l, n, g]] = 1.0
    v = rng.normal(size=(L, M, H, d)).astype(np.float32)
    a = rng.uniform(0.3, 1.0, size=(L, M, H)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, size=(L, M, H)).astype(np.float32)
    return S.astype(np.float32), j, k, v, a, b


def _columns_along(S0, j, v, a, b, H, Hk, path):
    """The column recurrence for one-hot keys, for one layer's [H, d, d]."""
    S = S0.astype(np.float64).copy()
    G = H // Hk
    for n in path:
        for h in range(H):
            col = j[n, h // G]
            for c in range(S.shape[2]):
                S[h, :, c] *= float(a[n, h])
            S[h, :, col] = (S[h, :, col] * (1.0 - float(b[n, h]))
                            + float(b[n, h]) * v[n, h].astype(np.float64))
    return S


def check_commit_one_hot(go):
    rng = np.random.default_rng(1)
    L, M, H, Hk, d = 2, 6, 4, 2, 8
    S, j, k, v, a, b = _one_hot_case(rng, L, M, H, Hk, d)
    path = [0, 2, 3, 5]
    got = go.commit(S, k, v, a, b, path)
    for l in range(L):
        want = _columns_along(S[l], j[l], v[l], a[l], b[l], H, Hk, path)
        assert np.allclose(got[l], want, rtol=1e-12, atol=1e-12), l


def check_commit_empty_path(go):
    rng = np.random.default_rng(2)
    S, j, k, v, a, b = _one_hot_case(rng, 1, 3, 2, 1, 4)
    got = go.commit(S, k, v, a, b, [])
    assert np.array_equal(got, S.astype(np.float64))


def check_delta_property(go):
    """b = 1, unit key: S_new k = v for any gate; x orthogonal to k: a S x."""
    rng = np.random.default_rng(3)
    d, H = 16, 3
    S = rng.normal(size=(1, H, d, d)).astype(np.float32)
    kk = rng.normal(size=d)
    kk /= np.linalg.norm(kk)
    k = kk.astype(np.float32).reshape(1, 1, 1, d)
    kd = k.reshape(d).astype(np.float64)
    v = rng.normal(size=(1, 1, H, d)).astype(np.float32)
    a = np.array([[[0.25, 0.6, 1.0]]], dtype=np.float32)
    b = np.ones((1, 1, H), dtype=np.float32)
    got = go.commit(S, k, v, a, b, [0])
    x = rng.normal(size=d)
    x -= kd * (kd @ x) / (kd @ kd)
    for h in range(H):
        # the key in fp32 is unit only to ~1e-7
        assert np.allclose(got[0, h] @ kd, v[0, 0, h], atol=1e-5), h
        assert np.allclose(got[0, h] @ x, a[0, 0, h] * (S[0, h] @ x),
                           atol=1e-5), h


def check_decay_and_forget(go):
    rng = np.random.default_rng(4)
    d = 8
    S = rng.normal(size=(1, 2, d, d)).astype(np.float32)
    k = rng.normal(size=(1, 3, 1, d)).astype(np.float32)
    v = rng.normal(size=(1, 3, 2, d)).astype(np.float32)
    a = np.array([[[0.5, 0.9], [0.75, 0.8], [0.5, 1.0]]], dtype=np.float32)
    b = np.zeros((1, 3, 2), dtype=np.float32)
    got = go.commit(S, k, v, a, b, [0, 1, 2])
    for h in range(2):
        gain = float(np.prod(a[0, :, h].astype(np.float64)))
        assert np.allclose(got[0, h], gain * S[0, h].astype(np.float64),
                           rtol=1e-14, atol=0), h
    # a = 0 forgets: the state becomes b v k^T of the last token
    a0 = np.zeros((1, 3, 2), dtype=np.float32)
    b1 = np.full((1, 3, 2), 0.5, dtype=np.float32)
    got = go.commit(S, k, v, a0, b1, [1, 2])
    for h in range(2):
        want = 0.5 * np.outer(v[0, 2, h].astype(np.float64),
                              k[0, 2, 0].astype(np.float64))
        assert np.allclose(got[0, h], want, rtol=1e-14, atol=1e-15), h


def check_last_write_wins(go):
    rng = np.random.default_rng(5)
    d = 8
    S = rng.normal(size=(1, 1, d, d)).astype(np.float32)
    kk = np.zeros(d, dtype=np.float32)
    kk[:4] = 0.5                              # unit norm, exact in fp32
    k = np.stack([kk, kk]).reshape(1, 2, 1, d)
    v = rng.normal(size=(1, 2, 1, d)).astype(np.float32)
    a = np.ones((1, 2, 1), dtype=np.float32)
    b = np.ones((1, 2, 1), dtype=np.float32)
    got = go.commit(S, k, v, a, b, [0, 1])
    assert np.allclose(got[0, 0] @ kk.astype(np.float64), v[0, 1, 0],
                       atol=1e-12)
    got = go.commit(S, k, v, a, b, [1, 0])
    assert np.allclose(got[0, 0] @ kk.astype(np.float64), v[0, 0, 0],
                       atol=1e-12)


def _path_to(parent, i):
    path = []
    while i >= 0:
        path.append(i)
        i = parent[i]
    return path[::-1]


TREE = [-1, 0, 0, 1, -1, 3, 2, 5]


def check_tree_out_one_hot(go):
    rng = np.random.default_rng(6)
    M, H, Hk, d = len(TREE), 4, 2, 8
    S, j, k, v, a, b = _one_hot_case(rng, 1, M, H, Hk, d)
    q = rng.normal(size=(M, Hk, d)).astype(np.float32)
    out = go.tree_out(S[0], q, k[0], v[0], a[0], b[0], TREE)
    G = H // Hk
    for i in range(M):
        Si = _columns_along(S[0], j[0], v[0], a[0], b[0], H, Hk,
                            _path_to(TREE, i))
        for h in range(H):
            want = Si[h] @ q[i, h // G].astype(np.float64)
            assert np.allclose(out[i, h], want, rtol=1e-12, atol=1e-12), (i, h)


def check_tree_out_is_path_commit(go):
    rng = np.random.default_rng(7)
    M, H, Hk, d = len(TREE), 2, 1, 8
    S = rng.normal(size=(H, d, d)).astype(np.float32)
    q = rng.normal(size=(M, Hk, d)).astype(np.float32)
    k = rng.normal(size=(M, Hk, d)).astype(np.float32) / np.sqrt(d)
    v = rng.normal(size=(M, H, d)).astype(np.float32)
    a = rng.uniform(0.5, 1.0, size=(M, H)).astype(np.float32)
    b = rng.uniform(0.0, 1.0, size=(M, H)).astype(np.float32)
    out = go.tree_out(S, q, k, v, a, b, TREE)
    for i in range(M):
        Si = go.commit(S[None], k[None], v[None], a[None], b[None],
                       _path_to(TREE, i))[0]
        for h in range(H):
            assert np.allclose(out[i, h], Si[h] @ q[i, 0].astype(np.float64),
                               rtol=1e-12, atol=1e-12), (i, h)


def check_errors(go):
    S = np.zeros((2, 4, 4), dtype=np.float32)
    z = np.zeros((2, 1, 4), dtype=np.float32)
    zv = np.zeros((2, 2, 4), dtype=np.float32)
    g = np.ones((2, 2), dtype=np.float32)
    for bad in ([-1, 1], [0, -1], [-2, 0]):
        with pytest.raises(ValueError):
            go.tree_out(S, z, z, zv, g, g, bad)
    with pytest.raises(ValueError):
        go.commit(S[None], z[None], zv[None], g[None], g[None], [2])
    Sh = np.zeros((1, 3, 4, 4), dtype=np.float32)
    with pytest.raises(ValueError):       # 3 value heads over 2 key heads
        go.commit(Sh, np.zeros((1, 1, 2, 4)), np.zeros((1, 1, 3, 4)),
                  np.ones((1, 1, 3)), np.ones((1, 1, 3)), [0])


ALL_CHECKS = [check_commit_one_hot, check_commit_empty_path,
              check_delta_property, check_decay_and_forget,
              check_last_write_wins, check_tree_out_one_hot,
              check_tree_out_is_path_commit, check_errors]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_gdn_oracle_pin(check):
    check(gdn_mod.default())


# -------------------------------------------------------------- mutants

MUTANTS = {
    "gate_dropped": ("S[r * dk + b] = alpha * T[r * dk + b] + beta",
                     "S[r * dk + b] = T[r * dk + b] + beta"),
    "gate_on_value_too": (
        "alpha * T[r * dk + b] + beta * (double)v[r] * (double)k[b];",
        "alpha * (T[r * dk + b] + beta * (double)v[r] * (double)k[b]);"),
    "no_strength_on_value": ("+ beta * (double)v[r] * (double)k[b];",
                             "+ (double)v[r] * (double)k[b];"),
    "projection_sign": ("(a == b ? 1.0 : 0.0) - beta",
                        "(a == b ? 1.0 : 0.0) + beta"),
    "outer_transposed": ("+ beta * (double)v[r] * (double)k[b];",
                         "+ beta * (double)v[b] * (double)k[r];"),
    "state_transposed": ("acc += S[r * dk + a] * P[a * dk + b];",
                         "acc += S[a * dk + r] * P[a * dk + b];"),
    "tree_path_reversed": ("for (int s = depth - 1; s >= 0; --s) {",
                           "for (int s = 0; s < depth; ++s) {"),
    "tree_output_before_own_update": (
        "for (int s = depth - 1; s >= 0; --s) {",
        "for (int s = depth - 1; s >= 1; --s) {"),
    "tree_parent_skipped": ("for (int n = i; n >= 0; n = parent[n])",
                            "for (int n = i; n >= 0; n = n > 0 ? n - 1 : -1)"),
    "commit_key_head": ("const size_t tk = ((size_t)l * M + path[s]) * Hk + h / G;",
                        "const size_t tk = ((size_t)l * M + path[s]) * Hk + h % Hk;"),
    "commit_reversed": ("for (int s = 0; s < a; ++s) {\n        const size_t t",
                        "for (int s = a - 1; s >= 0; --s) {\n        const size_t t"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gdn_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    with open(oracle.GDN_SOURCE) as fh:
        src = fh.read()
    assert src.count(find) == 1, f"mutation anchor not unique: {find!r}"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(find, repl))
    lib = oracle.compile_source(str(path), str(tmp_path / f"{name}.so"),
                                extra=("-Wno-error",))
    go = gdn_mod.GdnOracle(lib)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(go)
        except (AssertionError, ValueError):
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
