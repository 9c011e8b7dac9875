"""GPU parity of the verify sampling epilogue against the CPU oracle.

The GPU's top-k candidates must equal the oracle's exactly (indices and the
logit values, bit for bit: both order the same fp32 logits).  Probabilities
agree within fp32 rounding.  The accept test and the residual draw are
integer decisions taken on fp32 (GPU) and fp64 (oracle) probabilities: they
must agree wherever the oracle's margin exceeds 1e-5; inside that margin
either outcome is correct, and the GPU's token must still be a candidate the
draw could return.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import sample as so

pytestmark = pytest.mark.gpu

MARGIN = 1e-5


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemm_q4_amd as lib
    lib.load()
    return lib


def _say(*a):
    print(*a, flush=True)


def draft_inputs(logits_np, k, draft_k, seed, in_share=0.5):
    """Draft candidates that partly overlap the target's candidates (so that
    both accepts and rejects occur), q ~ Dirichlet, the drafted token drawn
    from q, and u, v uniform."""
    rng = np.random.default_rng(seed)
    M, V = logits_np.shape
    idx, _ = so.topk(logits_np, min(k, V))
    di = np.zeros((M, draft_k), dtype=np.int32)
    for m in range(M):
        inside = list(rng.permutation(idx[m])[:int(draft_k * in_share)])
        rest = [t for t in rng.permutation(V) if t not in inside]
        di[m] = (inside + rest)[:draft_k]
    dq = rng.dirichlet(np.ones(draft_k), size=M).astype(np.float32) \
        if draft_k else np.zeros((M, 0), dtype=np.float32)
    if draft_k:
        tok = np.array([di[m, rng.choice(draft_k, p=dq[m] / dq[m].sum())]
                        for m in range(M)], dtype=np.int32)
    else:
        tok = rng.integers(0, V, size=M).astype(np.int32)
    u = rng.random(M).astype(np.float32)
    v = rng.random(M).astype(np.float32)
    return tok, di, dq, u, v


def run_and_check(q4, logits, T, top_p, k, draft_k, seed, what):
    dev = logits.device
    L = logits.cpu().numpy()
    tok, di, dq, u, v = draft_inputs(L, k, draft_k, seed)
    t = lambda a: torch.from_numpy(a).to(dev)
    _say(f"case sample {what}: M={L.shape[0]} V={L.shape[1]} T={T} "
         f"top_p={top_p} k={k} draft_k={draft_k}")
    out = q4.verify_sample(logits, T, top_p, k, t(tok),
                           t(di) if draft_k else None,
                           t(dq) if draft_k else None, t(u), t(v))
    torch.cuda.synchronize()
    g = {n: x.cpu().numpy() for n, x in out.items()}
    idx, val = so.topk(L, k)
    assert np.array_equal(g["top_idx"], idx), what
    # same values, bit for bit, except that -0 is reported as +0
    assert np.array_equal(g["top_val"].view(np.uint32),
                          np.where(val == 0, np.float32(0), val).view(np.uint32))
    o = so.sample(idx, val, T, top_p, tok, di, dq.astype(np.float64),
                  u.astype(np.float64), v.astype(np.float64))
    assert np.allclose(g["top_prob"], o["p"], rtol=1e-5, atol=2e-6), what
    assert np.array_equal(g["greedy"], o["greedy"])
    clear_accept = np.abs(o["accept_margin"]) > MARGIN
    assert np.array_equal(g["accept"][clear_accept], o["accept"][clear_accept])
    same = g["accept"] == o["accept"]
    clear_token = same & ((o["accept"] == 1) | (o["draw_margin"] > MARGIN))
    assert np.array_equal(g["token"][clear_token], o["token"][clear_token])
    for m in np.nonzero(~clear_token)[0]:
        # an unclear decision: the GPU's token must be one the rule can emit
        assert g["token"][m] == tok[m] if g["accept"][m] else \
            g["token"][m] in idx[m][o["p"][m] > 0], (what, m)
    return g, o


def test_lm_head_rows(q4):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(1)
    logits = torch.randn((16, 248320), generator=gen, device=dev) * 3.0
    g, o = run_and_check(q4, logits, 1.0, 0.95, 20, 16, 2, "lm head")
    # the inputs exercise both branches
    assert 0 < o["accept"].sum() < 16


@pytest.mark.parametrize("T,top_p,k,draft_k", [(0.7, 1.0, 32, 16),
                                               (1.0, 0.5, 8, 4),
                                               (2.0, 0.99, 32, 0),
                                               (1.0, 1.0, 1, 1)])
def test_parameters(q4, T, top_p, k, draft_k):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(3)
    logits = torch.randn((9, 50000), generator=gen, device=dev) * 2.0
    run_and_check(q4, logits, T, top_p, k, draft_k, 4, f"T={T}")


def test_ties_break_by_smaller_index(q4):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(5)
    logits = torch.round(torch.randn((8, 7000), generator=gen,
                                     device=dev) * 2) / 2
    run_and_check(q4, logits, 1.0, 0.9, 32, 8, 6, "ties")
    # all equal: the candidates are tokens 0..k-1
    flat = torch.zeros((2, 3000), device=dev)
    g, _ = run_and_check(q4, flat, 1.0, 1.0, 32, 4, 7, "all equal")
    assert np.array_equal(g["top_idx"][0], np.arange(32))
    # full width: every slice has more tied keys than the survivor buffer
    # holds and takes the exact fallback; the row's lists then all tie
    flat = torch.full((2, 248320), -1.5, device=dev)
    flat[1, 200000:200005] = 0.25
    g, _ = run_and_check(q4, flat, 1.0, 1.0, 32, 4, 17, "all equal, full width")
    assert np.array_equal(g["top_idx"][0], np.arange(32))
    assert list(g["top_idx"][1][:6]) == [200000, 200001, 200002, 200003, 200004, 0]


def test_greedy(q4):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(8)
    logits = torch.randn((16, 248320), generator=gen, device=dev)
    g, o = run_and_check(q4, logits, 0.0, 1.0, 4, 16, 9, "greedy")
    assert np.array_equal(g["token"], g["greedy"])


# rows of 1 to 62 slices of 16384 columns (1000000 columns: 62 lists of 32
# candidates in the row merge)
@pytest.mark.parametrize("M,V,k", [(1, 7, 7), (3, 100, 32), (16, 64, 32),
                                   (2, 16385, 32), (5, 1, 1),
                                   (1024, 300, 16), (3, 262144, 32),
                                   (2, 300000, 32), (1, 1000000, 20)])
def test_shapes_and_edges(q4, M, V, k):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(10 + V)
    logits = torch.randn((M, V), generator=gen, device=dev)
    run_and_check(q4, logits, 1.0, 0.9, k, min(4, V), 11, f"{M}x{V}")


def test_extreme_logits(q4):
    """Huge, tiny and infinite values order correctly (the key keeps IEEE
    order, -inf last among real values)."""
    dev = torch.device("cuda")
    L = np.random.default_rng(12).normal(size=(2, 3000)).astype(np.float32)
    L[0, 10] = np.inf
    L[0, 20] = 3e38
    L[0, 30] = -np.inf
    L[1, :] = -np.inf
    L[1, 2999] = -1e30
    L[1, 5] = -0.0
    L[1, 6] = 0.0
    logits = torch.from_numpy(L).to(dev)
    idx, _ = so.topk(L, 8)
    out = q4.verify_sample(logits, 0.0, 1.0, 8,
                           torch.zeros(2, dtype=torch.int32, device=dev),
                           None, None, torch.zeros(2, device=dev),
                           torch.zeros(2, device=dev))
    assert np.array_equal(out["top_idx"].cpu().numpy(), idx)
    # the two zeros tie: token 5 (-0) before token 6 (+0)
    assert list(idx[1][:3]) == [5, 6, 2999]


def test_deterministic(q4):
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(13)
    logits = torch.randn((16, 248320), generator=gen, device=dev)
    inp = synth.sample_inputs(16, 248320, 16, seed=13, device=dev)
    a = q4.verify_sample(logits, 1.0, 0.95, 20, inp["draft_tok"],
                         inp["draft_idx"], inp["draft_q"], inp["u"], inp["v"])
    b = q4.verify_sample(logits, 1.0, 0.95, 20, inp["draft_tok"],
                         inp["draft_idx"], inp["draft_q"], inp["u"], inp["v"])
    for n in a:
        assert torch.equal(a[n].view(torch.int32), b[n].view(torch.int32)), n


def test_row_merge_structures(q4):
    """37 slices of about 16216 columns (more lists than candidates), with
    the best 32 all in one slice, one per slice near its start, after two
    slices' second keys, in a row of equal logits and all in the last
    slice: the row kernel reads only the lists whose heads reach the 32nd
    largest head."""
    dev = torch.device("cuda")
    V = 600000
    gen = torch.Generator(device=dev).manual_seed(16)
    logits = torch.randn((5, V), generator=gen, device=dev)
    logits[0, 300000:300040] = 10.0 + torch.arange(40, device=dev) * 0.01
    logits[1, ::16384] = 8.0 + torch.arange(37, device=dev) * 0.01
    logits[2, [5, 6, 20000, 20001]] = torch.tensor([9.0, 8.9, 9.05, 8.95],
                                                   device=dev)
    logits[3] = 1.5
    logits[4, V - 40:] = 6.0 - torch.arange(40, device=dev) * 0.01
    run_and_check(q4, logits, 1.0, 0.9, 32, 8, 17, "row merge")


def test_after_lm_head_gemm(q4):
    """The verify step end to end: the LM head (248320 x 5120 Q4, 16 verify
    rows) on the resident-activation kernel, then the sampling epilogue on
    its logits, against the oracle on the same logits."""
    dev = torch.device("cuda")
    N, K, M = 248320, 5120, 16
    W = synth.q4_weights(N, K, seed=14, device=dev)
    Wt = torch.empty_like(W)
    q4.q4_repack(W, Wt, N, K)
    x = synth.activations(M, K, seed=14, stream=1, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    q4.q4_gemm_verify_tiled(x, Wt, y, M, N, K)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    run_and_check(q4, y, 1.0, 0.95, 20, 16, 15, "after lm head")


# ------------------------------------------------- fused LM-head epilogue

def _fused_case(q4, N, K, M, T, top_p, k, draft_k, seed, zero_x=False):
    """q4_gemm_verify_sample against the same product written out by
    q4_gemm_verify_tiled and sampled by q4_verify_sample (itself checked
    against the oracle on those logits): every output bit for bit."""
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=seed, device=dev)
    Wt = torch.empty_like(W)
    q4.q4_repack(W, Wt, N, K)
    x = synth.activations(M, K, seed=seed, stream=1, device=dev)
    if zero_x:
        x.zero_()
    logits = torch.empty((M, N), dtype=torch.float32, device=dev)
    q4.q4_gemm_verify_tiled(x, Wt, logits, M, N, K)
    torch.cuda.synchronize()
    g, _ = run_and_check(q4, logits, T, top_p, k, draft_k, seed,
                         f"unfused N={N} K={K} M={M}")
    tok, di, dq, u, v = draft_inputs(logits.cpu().numpy(), k, draft_k, seed)
    t = lambda a: torch.from_numpy(a).to(dev)
    _say(f"case fused sample N={N} K={K} M={M} T={T} k={k}")
    f = q4.gemm_verify_sample(x, Wt, N, K, T, top_p, k, t(tok),
                              t(di) if draft_k else None,
                              t(dq) if draft_k else None, t(u), t(v))
    torch.cuda.synchronize()
    for name, arr in g.items():
        got = f[name].cpu().numpy()
        assert np.array_equal(got.view(np.uint32) if got.dtype == np.float32
                              else got,
                              arr.view(np.uint32) if arr.dtype == np.float32
                              else arr), (name, N, K, M)
    return g


def test_fused_lm_head(q4):
    """The LM head of the 27B model (248320 x 5120) at 16 verify rows with
    top-20, top_p 0.95 and 16 draft candidates: the configuration the bench
    times."""
    g = _fused_case(q4, 248320, 5120, 16, 1.0, 0.95, 20, 16, 70)
    assert 0 < g["accept"].sum() < 16


@pytest.mark.parametrize("N,K,M,T,top_p,k,draft_k", [
    (50000, 2048, 1, 1.0, 0.9, 32, 8),
    (50000, 2048, 5, 0.7, 1.0, 16, 16),
    (16384, 6144, 8, 1.3, 0.8, 32, 4),     # 12 waves, row-staged activations
    (640, 512, 16, 1.0, 1.0, 32, 2),       # 16 columns per workgroup
    (48, 1024, 3, 0.0, 1.0, 5, 3),         # greedy, 3 tiles
])
def test_fused_shapes(q4, N, K, M, T, top_p, k, draft_k):
    _fused_case(q4, N, K, M, T, top_p, k, draft_k, 71)


def test_fused_all_logits_equal(q4):
    """Zero activations make every logit 0: every column of a workgroup
    passes the threshold (the survivor lists run past 64 keys and are merged
    in chunks), and ties go to the smaller token index."""
    g = _fused_case(q4, 50000, 1024, 4, 1.0, 1.0, 32, 4, 72, zero_x=True)
    assert (g["top_idx"] == np.arange(32)[None, :]).all()
