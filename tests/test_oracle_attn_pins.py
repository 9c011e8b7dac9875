"""Pins of the tree-verify attention oracle to facts other than itself (no
GPU).

Each ``check_*`` takes an AttnOracle and raises AssertionError on a mismatch.
The tests run them against the real oracle; the mutant test at the end runs
them against copies of ``oracle/tree_attn.c`` with planted mistakes, each of
which at least one pin must catch.

What pins what:

* zero keys give equal weights, so a node's output is the plain mean of the
  values it may see -- the visible set is read off the parent pointers here,
  independently of the oracle (mask, tree offset, value scale, layout);
* one key far above the rest gives that position's value exactly (transposed
  value layout, page table, key scale);
* two visible positions with hand-set scores: the softmax written out with
  ``math.exp`` (the score scale and the normalisation);
* values constant per KV head expose which KV head each query head reads;
* changing a non-ancestor's key or value leaves a node's output bit for bit
  unchanged, changing an ancestor's does not;
* permuting the physical pages (with the page table) changes nothing;
* random caches against torch's float64 scaled-dot-product attention with a
  boolean mask on the dequantised keys and values (a library routine).

The second output, sum_p w_p |v_p|, is pinned by: the plain mean of |v| over
the visible set when the keys are zero; bitwise equality with the outputs
when every value is non-negative (same weights, same order); torch's
attention applied to |V|; and |o| <= sum_p w_p |v_p| everywhere.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attn as attn_mod

PAGE = 32


def bf16_bits(x):
    """Round-to-nearest-even bf16 bit patterns of float32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def make_cache(K8, ks, V8, vs, perm=None, spare=1):
    """Paged cache from per-position data.  K8, V8 int8 [T, Hkv, D]; ks, vs
    float32 [T, Hkv].  Returns (k_pages, v_pages, k_scale, v_scale,
    page_table) with logical page lp stored at physical page perm[lp]."""
    T, Hkv, D = K8.shape
    lp = (T + PAGE - 1) // PAGE
    pool = lp + spare
    perm = np.arange(lp) if perm is None else np.asarray(perm)
    kp = np.zeros((pool, Hkv, PAGE, D), dtype=np.int8)
    vp = np.zeros((pool, Hkv, D, PAGE), dtype=np.int8)
    ksp = np.zeros((pool, Hkv, PAGE), dtype=np.float32)
    vsp = np.zeros((pool, Hkv, PAGE), dtype=np.float32)
    for p in range(T):
        pg, s = perm[p // PAGE], p % PAGE
        kp[pg, :, s, :] = K8[p]
        vp[pg, :, :, s] = V8[p]
        ksp[pg, :, s] = ks[p]
        vsp[pg, :, s] = vs[p]
    # garbage in the unused tail of the last page: must never be seen
    last = perm[lp - 1]
    for s in range(T % PAGE or PAGE, PAGE):
        kp[last, :, s, :] = 77
        vp[last, :, :, s] = -99
        ksp[last, :, s] = 1e3
        vsp[last, :, s] = 1e3
    return kp, vp, ksp, vsp, perm.astype(np.int32)


def visible(parent, C, i):
    """Positions node i may see, from the parent pointers."""
    tree = []
    n = i
    while n >= 0:
        tree.append(C + n)
        n = parent[n]
    return list(range(C)) + sorted(tree)


def random_case(rng, C, parent, Hq=6, Hkv=2, D=32):
    M = len(parent)
    T = C + M
    K8 = rng.integers(-127, 128, size=(T, Hkv, D)).astype(np.int8)
    V8 = rng.integers(-127, 128, size=(T, Hkv, D)).astype(np.int8)
    ks = (rng.random((T, Hkv)) * 0.02 + 1e-3).astype(np.float32)
    vs = (rng.random((T, Hkv)) * 0.02 + 1e-3).astype(np.float32)
    q = bf16_bits(rng.normal(size=(M, Hq, D)).astype(np.float32))
    return q, K8, ks, V8, vs


TREE = [-1, 0, 0, 1, -1, 4, 2]


def check_zero_keys_mean(ao):
    rng = np.random.default_rng(1)
    C, Hq, Hkv, D = 37, 4, 2, 16
    q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
    K8[:] = 0
    cache = make_cache(K8, ks, V8, vs)
    out = ao.attention(q, *cache, C, attn_mod.ancestor_masks(TREE), 0.125)
    G = Hq // Hkv
    for i in range(len(TREE)):
        pos = visible(TREE, C, i)
        for h in range(Hq):
            g = h // G
            want = np.mean([V8[p, g].astype(np.float64) * float(vs[p, g])
                            for p in pos], axis=0)
            assert np.allclose(out[i, h], want, rtol=1e-13, atol=1e-15), (i, h)


def check_dominant_key(ao):
    rng = np.random.default_rng(2)
    C, Hq, Hkv, D = 70, 2, 1, 8
    q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
    q[:] = 0
    q[:, :, 3] = bf16_bits(np.float32(1.0))
    K8[:] = 0
    star = 41                       # a context position on the second page
    K8[star, 0, 3] = 127
    ks[star, 0] = 1.0
    cache = make_cache(K8, ks, V8, vs, perm=[2, 0, 1])
    out = ao.attention(q, *cache, C, attn_mod.ancestor_masks(TREE), 1.0)
    want = V8[star, 0].astype(np.float64) * float(vs[star, 0])
    for i in range(len(TREE)):
        for h in range(Hq):
            assert np.allclose(out[i, h], want, rtol=1e-12, atol=1e-30), (i, h)


def check_two_position_softmax(ao):
    """Context of 1, one root node: positions 0 and 1, scores set by hand."""
    D = 4
    q = bf16_bits(np.array([[[0.5, -1.0, 2.0, 0.25]]], dtype=np.float32))
    K8 = np.array([[[10, 0, 3, -4]], [[-7, 2, 1, 8]]], dtype=np.int8)
    ks = np.array([[0.5], [0.25]], dtype=np.float32)
    V8 = np.array([[[1, 2, 3, 4]], [[-5, 6, -7, 8]]], dtype=np.int8)
    vs = np.array([[0.125], [0.5]], dtype=np.float32)
    scale = 0.75
    cache = make_cache(K8, ks, V8, vs)
    out = ao.attention(q, *cache, 1, np.array([1], dtype=np.uint32), scale)
    qd = [0.5, -1.0, 2.0, 0.25]
    s0 = scale * sum(a * b * 0.5 for a, b in zip(qd, [10, 0, 3, -4]))
    s1 = scale * sum(a * b * 0.25 for a, b in zip(qd, [-7, 2, 1, 8]))
    w0 = math.exp(s0) / (math.exp(s0) + math.exp(s1))
    want = [w0 * a * 0.125 + (1 - w0) * b * 0.5
            for a, b in zip([1, 2, 3, 4], [-5, 6, -7, 8])]
    assert np.allclose(out[0, 0], want, rtol=1e-14, atol=0)


def check_query_head_groups(ao):
    rng = np.random.default_rng(3)
    C, Hq, Hkv, D = 20, 12, 4, 8
    q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
    for g in range(Hkv):
        V8[:, g, :] = g + 1
    vs[:] = 1.0
    cache = make_cache(K8, ks, V8, vs)
    out = ao.attention(q, *cache, C, attn_mod.ancestor_masks(TREE), 0.3)
    for h in range(Hq):
        assert np.allclose(out[:, h], h // 3 + 1, rtol=1e-13), h


def check_mask_invariance(ao):
    rng = np.random.default_rng(4)
    C, Hq, Hkv, D = 33, 4, 2, 16
    q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
    anc = attn_mod.ancestor_masks(TREE)
    base = ao.attention(q, *make_cache(K8, ks, V8, vs), C, anc, 0.2)
    # node 6's path is 0 -> 2 -> 6; node 3 is off it
    K2, V2 = K8.copy(), V8.copy()
    K2[C + 3] = -K2[C + 3]
    V2[C + 3] = 5
    other = ao.attention(q, *make_cache(K2, ks, V2, vs), C, anc, 0.2)
    for i in (0, 2, 6, 4, 5):         # nodes that do not see node 3
        assert np.array_equal(base[i], other[i]), i
    for i in (3,):
        assert not np.allclose(base[i], other[i]), i
    K3 = K8.copy()
    K3[C + 2] = -K3[C + 2]            # node 2 is an ancestor of node 6
    third = ao.attention(q, *make_cache(K3, ks, V8, vs), C, anc, 0.2)
    assert not np.allclose(base[6], third[6])
    assert np.array_equal(base[3], third[3])


def check_page_permutation(ao):
    rng = np.random.default_rng(5)
    C, Hq, Hkv, D = 100, 4, 2, 16
    q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
    anc = attn_mod.ancestor_masks(TREE)
    a = ao.attention(q, *make_cache(K8, ks, V8, vs), C, anc, 0.1)
    b = ao.attention(q, *make_cache(K8, ks, V8, vs, perm=[3, 1, 0, 2],
                                    spare=2), C, anc, 0.1)
    assert np.array_equal(a, b)


def check_against_torch_sdpa(ao):
    rng = np.random.default_rng(6)
    for C in (0, 31, 64, 90):
        Hq, Hkv, D = 6, 2, 32
        q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
        anc = attn_mod.ancestor_masks(TREE)
        out = ao.attention(q, *make_cache(K8, ks, V8, vs), C, anc, 0.17)
        M, T = len(TREE), C + len(TREE)
        Kd = torch.from_numpy(K8.astype(np.float64) * ks[..., None].astype(np.float64))
        Vd = torch.from_numpy(V8.astype(np.float64) * vs[..., None].astype(np.float64))
        Q = torch.from_numpy(bits_to_f64(q))
        mask = torch.zeros((M, T), dtype=torch.bool)
        for i in range(M):
            mask[i, visible(TREE, C, i)] = True
        G = Hq // Hkv
        for h in range(Hq):
            g = h // G
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[:, h][None], Kd[:, g][None], Vd[:, g][None],
                attn_mask=mask[None], scale=0.17)[0]
            assert np.allclose(out[:, h], ref.numpy(), rtol=1e-11, atol=1e-14), (C, h)


def check_abs_zero_keys_mean(ao):
    rng = np.random.default_rng(7)
    C, Hq, Hkv, D = 45, 4, 2, 16
    q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
    K8[:] = 0
    cache = make_cache(K8, ks, V8, vs)
    _, absw = ao.attention(q, *cache, C, attn_mod.ancestor_masks(TREE), 0.5,
                           with_abs=True)
    G = Hq // Hkv
    for i in range(len(TREE)):
        pos = visible(TREE, C, i)
        for h in range(Hq):
            g = h // G
            want = np.mean([np.abs(V8[p, g].astype(np.float64)) * float(vs[p, g])
                            for p in pos], axis=0)
            assert np.allclose(absw[i, h], want, rtol=1e-13, atol=1e-15), (i, h)


def check_abs_nonnegative_values(ao):
    """With every value >= 0 the two sums are the same terms in the same
    order; with signed values |o| <= sum w |v|, and somewhere strictly."""
    rng = np.random.default_rng(8)
    C, Hq, Hkv, D = 60, 6, 2, 16
    q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
    anc = attn_mod.ancestor_masks(TREE)
    Vp = np.abs(V8.astype(np.int16)).clip(0, 127).astype(np.int8)
    out, absw = ao.attention(q, *make_cache(K8, ks, Vp, vs), C, anc, 0.2,
                             with_abs=True)
    assert np.array_equal(out, absw)
    out, absw = ao.attention(q, *make_cache(K8, ks, V8, vs), C, anc, 0.2,
                             with_abs=True)
    assert (np.abs(out) <= absw).all()
    assert (np.abs(out) < 0.5 * absw).any()


def check_abs_against_torch_sdpa(ao):
    rng = np.random.default_rng(9)
    for C in (0, 33, 96):
        Hq, Hkv, D = 4, 2, 16
        q, K8, ks, V8, vs = random_case(rng, C, TREE, Hq, Hkv, D)
        anc = attn_mod.ancestor_masks(TREE)
        _, absw = ao.attention(q, *make_cache(K8, ks, V8, vs), C, anc, 0.23,
                               with_abs=True)
        M, T = len(TREE), C + len(TREE)
        Kd = torch.from_numpy(K8.astype(np.float64) * ks[..., None].astype(np.float64))
        Va = torch.from_numpy(np.abs(V8.astype(np.float64)) *
                              vs[..., None].astype(np.float64))
        Q = torch.from_numpy(bits_to_f64(q))
        mask = torch.zeros((M, T), dtype=torch.bool)
        for i in range(M):
            mask[i, visible(TREE, C, i)] = True
        G = Hq // Hkv
        for h in range(Hq):
            g = h // G
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[:, h][None], Kd[:, g][None], Va[:, g][None],
                attn_mask=mask[None], scale=0.23)[0]
            assert np.allclose(absw[:, h], ref.numpy(), rtol=1e-11, atol=1e-14), (C, h)


def check_errors(ao):
    q = np.zeros((1, 2, 4), dtype=np.uint16)
    K8 = np.zeros((3, 1, 4), dtype=np.int8)
    s = np.ones((3, 1), dtype=np.float32)
    kp, vp, ksp, vsp, pt = make_cache(K8, s, K8, s)
    with pytest.raises(ValueError):
        ao.attention(q, kp, vp, ksp, vsp, np.array([5], dtype=np.int32), 2,
                     np.array([1], dtype=np.uint32), 1.0)
    q3 = np.zeros((1, 3, 4), dtype=np.uint16)
    kp2 = np.zeros((2, 2, 32, 4), dtype=np.int8)
    vp2 = np.zeros((2, 2, 4, 32), dtype=np.int8)
    s2 = np.ones((2, 2, 32), dtype=np.float32)
    with pytest.raises(ValueError):   # 3 query heads over 2 KV heads
        ao.attention(q3, kp2, vp2, s2, s2, np.array([0], dtype=np.int32), 2,
                     np.array([1], dtype=np.uint32), 1.0)


ALL_CHECKS = [check_zero_keys_mean, check_dominant_key,
              check_two_position_softmax, check_query_head_groups,
              check_mask_invariance, check_page_permutation,
              check_against_torch_sdpa, check_abs_zero_keys_mean,
              check_abs_nonnegative_values, check_abs_against_torch_sdpa,
              check_errors]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_attn_oracle_pin(check):
    check(attn_mod.default())


def test_ancestor_masks():
    m = attn_mod.ancestor_masks(TREE)
    assert list(m) == [0b1, 0b11, 0b101, 0b1011, 0b10000, 0b110000,
                       0b1000101]


# -------------------------------------------------------------- mutants

MUTANTS = {
    "key_scale_ignored": ("dot += bf16_to_double(qi[d]) * ((double)k8 * ks);",
                          "dot += bf16_to_double(qi[d]) * ((double)k8);"),
    "value_scale_ignored": ("o[d] += w * ((double)v8 * vs);",
                            "o[d] += w * ((double)v8);"),
    "values_not_transposed": (
        "v_pages[base * 32 * (size_t)D + (size_t)d * 32 + slot];",
        "v_pages[base * 32 * (size_t)D + (size_t)slot * D + d];"),
    "keys_transposed": ("k_pages[(base * 32 + slot) * D + d];",
                        "k_pages[base * 32 * D + (size_t)d * 32 + slot];"),
    "mask_sees_whole_tree": (
        "(unsigned char)((anc[i] >> (p - ctx_len)) & 1u);", "1;"),
    "mask_off_by_one": ("(anc[i] >> (p - ctx_len)) & 1u",
                        "(anc[i] >> (p - ctx_len + 1)) & 1u"),
    "kv_head_modulo": ("const int g = h / G;", "const int g = h % Hkv;"),
    "page_table_ignored": ("return page_table[p / 32];", "return p / 32;"),
    "score_scale_ignored": ("s[p] = scale * dot;", "s[p] = dot;"),
    "not_normalised": ("const double w = s[p] / den;", "const double w = s[p];"),
    "abs_signed": ("ao[d] += w * fabs((double)v8 * vs);",
                   "ao[d] += w * ((double)v8 * vs);"),
    "abs_unweighted": ("ao[d] += w * fabs((double)v8 * vs);",
                       "ao[d] += fabs((double)v8 * vs);"),
    "abs_value_scale_ignored": ("ao[d] += w * fabs((double)v8 * vs);",
                                "ao[d] += w * fabs((double)v8);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attn_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    with open(oracle.ATTN_SOURCE) as fh:
        src = fh.read()
    assert src.count(find) == 1, f"mutation anchor not unique: {find!r}"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(find, repl))
    lib = oracle.compile_source(str(path), str(tmp_path / f"{name}.so"),
                                extra=("-Wno-error",))
    ao = attn_mod.AttnOracle(lib)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(ao)
        except (AssertionError, ValueError):
            caught.append(check.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
