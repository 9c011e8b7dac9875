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
