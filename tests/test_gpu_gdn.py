"""GPU parity of the Gated DeltaNet state commit against the CPU oracle.

The kernel applies the accepted nodes' gated delta-rule updates to every
layer's fp32 state; the oracle does the same in fp64 with full matrices.

Tolerance, from the arithmetic: per node a row's dot product S_r . k (128
products, FMA chains of 16 then an 8-lane tree) is off by at most about
gamma_19 * ||S_r||_2 for a unit key, and the row update adds a rounding of
eps * |S|.  Errors add over the n nodes (each update is a contraction for
unit keys, gate <= 1 and strength in [0, 1]), so an element may be off by
(n + 1) * 32 * eps32 * R, R the largest row norm of the state before or
after the commit.  A wrong index, sign or order gives errors of order one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import gdn as go

pytestmark = pytest.mark.gpu

EPS32 = float(np.finfo(np.float32).eps)


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemm_q4_amd as lib
    lib.load()
    return lib


def _say(*a):
    print(*a, flush=True)


def _commit(q4, inp, path, n=None, status=True, M=None):
    dev = inp["S"].device
    M = inp["k"].shape[1] if M is None else M
    p = torch.zeros(M, dtype=torch.int32, device=dev)
    if len(path):
        p[:len(path)] = torch.tensor(path, dtype=torch.int32, device=dev)
    cnt = torch.tensor([len(path) if n is None else n], dtype=torch.int32,
                       device=dev)
    st = torch.full((1,), 12345, dtype=torch.int32, device=dev) \
        if status else None
    S = inp["S"].clone()
    q4.q4_gdn_commit(S, inp["k"], inp["v"], inp["alpha"], inp["beta"], p,
                     cnt, st)
    torch.cuda.synchronize()
    return S, (None if st is None else int(st.item()))


def _tol(S0, want, n):
    R = max(np.linalg.norm(S0, axis=-1).max(), np.linalg.norm(want,
                                                             axis=-1).max())
    return (n + 1) * 32 * EPS32 * R


def _check_heads(got, inp, path, heads):
    """Compare the GPU states of the given (layer, head) pairs with the
    oracle, one head at a time."""
    S0 = inp["S"].cpu().numpy()
    k = inp["k"].cpu().numpy()
    v = inp["v"].cpu().numpy()
    a = inp["alpha"].cpu().numpy()
    b = inp["beta"].cpu().numpy()
    H, Hk = S0.shape[1], k.shape[2]
    G = H // Hk
    g = got.cpu().numpy()
    worst = 0.0
    for l, h in heads:
        want = go.commit(S0[l:l + 1, h:h + 1], k[l:l + 1, :, h // G:h // G + 1],
                         v[l:l + 1, :, h:h + 1], a[l:l + 1, :, h:h + 1],
                         b[l:l + 1, :, h:h + 1], path)[0, 0]
        err = np.abs(g[l, h].astype(np.float64) - want).max()
        tol = _tol(S0[l, h], want, len(path))
        assert err <= tol, (l, h, err, tol)
        worst = max(worst, err / tol)
    return worst


@pytest.mark.parametrize("L,H,Hk,M,dv,path", [
    (2, 4, 2, 16, 128, [0, 1, 3, 7, 8]),
    (1, 3, 3, 8, 256, [2, 5]),
    (2, 2, 1, 4, 64, [3, 1]),
    (3, 2, 1, 32, 128, list(range(32))),
    (1, 1, 1, 1, 128, [0]),
])
def test_commit_matches_oracle(q4, L, H, Hk, M, dv, path):
    dev = torch.device("cuda")
    _say(f"case gdn commit L={L} H={H} Hk={Hk} M={M} dv={dv} n={len(path)}")
    inp = synth.gdn_inputs(L, H, Hk, M, dv=dv, seed=L * 7 + H, device=dev)
    S, st = _commit(q4, inp, path)
    assert st == 0
    heads = [(l, h) for l in range(L) for h in range(H)]
    _check_heads(S, inp, path, heads)


def test_full_state_sampled(q4):
    """48 layers x 48 value heads (16 key heads) x 128 x 128, a tree of 16
    nodes and an accepted path of 7: sampled heads against the oracle, and
    the heads' states outside the sample checked to have changed."""
    dev = torch.device("cuda")
    _say("case gdn commit full 48x48x128x128 n=7")
    inp = synth.gdn_inputs(48, 48, 16, 16, seed=21, device=dev)
    path = synth.tree_path(inp["parent"], 15)[:7]
    if len(path) < 7:
        path = list(range(7))
    S, st = _commit(q4, inp, path)
    assert st == 0
    rng = np.random.default_rng(22)
    heads = [(0, 0), (47, 47), (13, 31)] + [
        (int(rng.integers(48)), int(rng.integers(48))) for _ in range(9)]
    _check_heads(S, inp, path, heads)
    assert torch.isfinite(S).all()
    assert not torch.equal(S, inp["S"])


def test_zero_count_leaves_state(q4):
    dev = torch.device("cuda")
    inp = synth.gdn_inputs(2, 4, 2, 8, seed=3, device=dev)
    S, st = _commit(q4, inp, [], n=0)
    assert st == 0
    assert torch.equal(S, inp["S"])


@pytest.mark.parametrize("n,path", [(-1, [0]), (9, [0]), (3, [0, 8, 1]),
                                    (2, [0, -1])])
def test_bad_count_or_path_is_reported(q4, n, path):
    """Out-of-range count or path entries: status -1, the state untouched."""
    dev = torch.device("cuda")
    inp = synth.gdn_inputs(2, 4, 2, 8, seed=4, device=dev)
    S, st = _commit(q4, inp, path, n=n)
    assert st == -1
    assert torch.equal(S, inp["S"])


def test_gates_near_and_at_zero(q4):
    """Gates of 1e-4 drive the running gate factor under 2^-30 (rescale
    branch); a gate of exactly 0 forgets the state."""
    dev = torch.device("cuda")
    inp = synth.gdn_inputs(1, 4, 2, 8, seed=5, device=dev)
    a = inp["alpha"]
    a[0, 1:5, :2] = 1e-4
    a[0, 6, 2] = 0.0
    a[0, 2, 3] = 1.0
    path = [0, 1, 2, 3, 4, 5, 6]
    S, st = _commit(q4, inp, path)
    assert st == 0
    _check_heads(S, inp, path, [(0, h) for h in range(4)])


def test_deterministic(q4):
    dev = torch.device("cuda")
    inp = synth.gdn_inputs(4, 8, 4, 16, seed=6, device=dev)
    path = [0, 2, 4, 6, 8]
    a, _ = _commit(q4, inp, path)
    b, _ = _commit(q4, inp, path)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_without_status_pointer(q4):
    dev = torch.device("cuda")
    inp = synth.gdn_inputs(1, 2, 1, 4, seed=7, device=dev)
    S, st = _commit(q4, inp, [1, 3], status=False)
    assert st is None
    _check_heads(S, inp, [1, 3], [(0, 0), (0, 1)])


# ---------------------------------------------------------------- tree outputs
# Node i's output is S_i q_i, S_i the state after the updates on i's path.
# The kernel forms it from the rows' products with the tree's keys and
# queries and a per-row recurrence on the update coefficients; each of those
# terms carries the rounding of a 128-term dot product (gamma_19 for the FMA
# chains and the 8-lane tree) per node on the path, against a state row of
# norm at most R, the largest row norm of S_0 and of every S_i.  With unit
# queries an output may be off by (depth + 1) * 64 * eps32 * R; a wrong
# index, sign, gate or parent gives errors of the order of R / sqrt(128).

def _tree_out(q4, inp, parent=None, status=True):
    dev = inp["S"].device
    par = torch.tensor(inp["parent"] if parent is None else parent,
                       dtype=torch.int32, device=dev)
    st = torch.full((1,), 12345, dtype=torch.int32, device=dev) \
        if status else None
    shape = (inp["k"].shape[1], inp["S"].shape[1], inp["S"].shape[2])
    out = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    q4.q4_gdn_tree_out(inp["S"][0], inp["q"][0], inp["k"][0], inp["v"][0],
                       inp["alpha"][0], inp["beta"][0], par, out, st)
    torch.cuda.synchronize()
    return out, (None if st is None else int(st.item()))


def _check_tree(got, inp, heads=None):
    """Compare node outputs of the given value heads (all by default; a
    subset must be whole key heads' groups) with the oracle."""
    S0 = inp["S"][0].cpu().numpy()
    q = inp["q"][0].cpu().numpy()
    k = inp["k"][0].cpu().numpy()
    v = inp["v"][0].cpu().numpy()
    a = inp["alpha"][0].cpu().numpy()
    b = inp["beta"][0].cpu().numpy()
    parent = np.asarray(inp["parent"], dtype=np.int32)
    H, Hk = S0.shape[0], k.shape[1]
    G = H // Hk
    hs = list(range(H)) if heads is None else list(heads)
    kh = sorted({h // G for h in hs})
    assert hs == [h for g in kh for h in range(g * G, (g + 1) * G)]
    want = go.tree_out(S0[hs], q[:, kh], k[:, kh], v[:, hs], a[:, hs],
                       b[:, hs], parent)
    g = got.cpu().numpy()[:, hs].astype(np.float64)
    assert np.isfinite(g).all()
    M = len(parent)
    worst = 0.0
    for i in range(M):
        path = synth.tree_path(parent, i)
        Si = go.commit(S0[hs][None], k[None][:, :, kh], v[None][:, :, hs],
                       a[None][:, :, hs], b[None][:, :, hs], path)[0]
        R = max(np.linalg.norm(S0[hs], axis=-1).max(),
                np.linalg.norm(Si, axis=-1).max())
        tol = (len(path) + 1) * 64 * EPS32 * R
        err = np.abs(g[i] - want[i]).max()
        assert err <= tol, (i, len(path), err, tol)
        worst = max(worst, err / tol)
    _say(f"   tree outputs: worst error / bound = {worst:.3e}")


@pytest.mark.parametrize("H,Hk,M,dv", [(2, 1, 1, 32), (4, 2, 5, 64),
                                       (6, 2, 16, 128), (3, 3, 32, 32),
                                       (4, 1, 9, 96)])
def test_tree_out_matches_oracle(q4, H, Hk, M, dv):
    dev = torch.device("cuda")
    _say(f"case gdn tree out H={H} Hk={Hk} M={M} dv={dv}")
    inp = synth.gdn_inputs(1, H, Hk, M, dv=dv, seed=20 + M, device=dev)
    out, st = _tree_out(q4, inp)
    assert st == 0
    _check_tree(out, inp)


def test_tree_out_full_shape_sampled(q4):
    """The 27B layer: 48 value heads over 16 key heads of 128 x 128, a
    16-node tree; one key head's three value heads against the oracle."""
    dev = torch.device("cuda")
    _say("case gdn tree out full 48/16 x 128 x 128, M=16")
    inp = synth.gdn_inputs(1, 48, 16, 16, seed=30, device=dev)
    out, st = _tree_out(q4, inp)
    assert st == 0
    assert torch.isfinite(out).all()
    _check_tree(out, inp, heads=[21, 22, 23])


def test_tree_out_chain_and_star(q4):
    """A chain (every node the child of the previous) and a star (every
    node a child of the context): the deepest and the shallowest trees."""
    dev = torch.device("cuda")
    for name, par in (("chain", list(range(-1, 15))), ("star", [-1] * 16)):
        _say(f"case gdn tree out {name}")
        inp = synth.gdn_inputs(1, 4, 2, 16, seed=31, device=dev)
        inp["parent"] = np.asarray(par, dtype=np.int32)
        out, st = _tree_out(q4, inp)
        assert st == 0
        _check_tree(out, inp)


@pytest.mark.parametrize("M", [17, 24, 31])
def test_tree_out_deep_trees_past_16(q4, M):
    """The 32-node kernel (17..32 nodes): a chain of M nodes (a path 24 and
    31 deep), a star, and the random tree of the generator; the zero padding
    past node M - 1 must add nothing."""
    dev = torch.device("cuda")
    for name, par in (("chain", list(range(-1, M - 1))), ("star", [-1] * M),
                      ("random", None)):
        _say(f"case gdn tree out M={M} {name}")
        inp = synth.gdn_inputs(1, 6, 2, M, dv=64, seed=35 + M, device=dev)
        if par is not None:
            inp["parent"] = np.asarray(par, dtype=np.int32)
        out, st = _tree_out(q4, inp)
        assert st == 0
        _check_tree(out, inp)


def test_tree_out_full_shape_32_nodes(q4):
    """The 27B layer at 32 tree nodes: 48 value heads over 16 key heads of
    128 x 128; two key heads' value heads against the oracle."""
    dev = torch.device("cuda")
    _say("case gdn tree out full 48/16 x 128 x 128, M=32")
    inp = synth.gdn_inputs(1, 48, 16, 32, seed=36, device=dev)
    out, st = _tree_out(q4, inp)
    assert st == 0
    assert torch.isfinite(out).all()
    _check_tree(out, inp, heads=[0, 1, 2, 45, 46, 47])


def test_tree_out_gates_near_zero(q4):
    """Tiny and zero gates: the path weights underflow towards 0, and a
    zero gate forgets everything above it on the path."""
    dev = torch.device("cuda")
    inp = synth.gdn_inputs(1, 4, 2, 12, seed=32, device=dev)
    inp["parent"] = np.asarray(list(range(-1, 11)), dtype=np.int32)
    a = inp["alpha"]
    a[0, 1:6, :2] = 1e-4
    a[0, 7, 2] = 0.0
    out, st = _tree_out(q4, inp)
    assert st == 0
    _check_tree(out, inp)


@pytest.mark.parametrize("parent", [[-1, 0, 2], [-1, -2, 0], [0, 0, 1],
                                    [-1, 0, 7]])
def test_tree_out_bad_parent_is_reported(q4, parent):
    """A parent that is not an earlier node (or -1): status -1, nothing
    written."""
    dev = torch.device("cuda")
    inp = synth.gdn_inputs(1, 2, 1, 3, dv=32, seed=33, device=dev)
    out, st = _tree_out(q4, inp, parent=parent)
    assert st == -1
    assert torch.isnan(out).all()


def test_tree_out_deterministic_and_without_status(q4):
    dev = torch.device("cuda")
    inp = synth.gdn_inputs(1, 6, 2, 16, seed=34, device=dev)
    a, _ = _tree_out(q4, inp)
    b, st = _tree_out(q4, inp, status=False)
    assert st is None
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
