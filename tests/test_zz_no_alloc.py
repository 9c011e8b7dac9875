"""q4_gemm_verify_tiled_noalloc: the workspace GEMM with the library's static
device scratch, for callers that cannot allocate (GPU).

Two calls in a row through the C ABI, the second on a smaller input, each
checked against q4_gemm_verify_tiled_ws on the same inputs (same kernels and
plan, so bit for bit) and against the oracle's bound; device memory in use
is the same before and after the calls.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import oracle_threads

pytestmark = pytest.mark.gpu

REL, ABS = 2e-3, 1e-5


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemm_q4_amd as lib
    lib.load()
    return lib


def _case(q4, M, N, K, seed):
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=seed, device=dev)
    Wt = torch.empty_like(W)
    q4.q4_repack(W, Wt, N, K)
    x = synth.activations(M, K, seed=seed, stream=1, device=dev)
    ws = q4.workspace_for(M, N, K, dev)
    want = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    q4.q4_gemm_verify_tiled_ws(x, Wt, want, M, N, K, ws)
    torch.cuda.synchronize()
    return W, Wt, x, want


def test_noalloc_matches_workspace_path_twice(q4):
    cases = [(16, 5120, 17408, 60), (8, 1600, 7168, 61)]  # second smaller
    prepared = [_case(q4, *c) for c in cases]
    for (M, N, K, seed), (W, Wt, x, want) in zip(cases, prepared):
        plan = q4.q4_gemm_verify_tiled_ws_plan(M, N, K)
        assert plan["k_parts"] > 1 and plan["workspace_bytes"] > 0
        print(f"case noalloc M={M} N={N} K={K} parts={plan['k_parts']}",
              flush=True)
        y = torch.full((M, N), float("nan"), dtype=torch.float32,
                       device=x.device)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        q4.q4_gemm_verify_tiled_noalloc(x, Wt, y, M, N, K)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        assert torch.equal(y.view(torch.int32), want.view(torch.int32))
        _, y64, a64, _ = oracle.gemm(synth.bf16_bits(x), W.cpu().numpy(), N, K,
                                     threads=oracle_threads())
        err = np.abs(y.cpu().numpy().astype(np.float64) - y64)
        assert (err <= REL * a64 + ABS).all()


def test_noalloc_unsplit_and_too_large(q4):
    """A shape with no K split runs without touching the scratch; a shape
    whose split needs more than the scratch is refused before launch."""
    dev = torch.device("cuda")
    M, N, K = 8, 4096, 5120
    W, Wt, x, want = _case(q4, M, N, K, 62)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    q4.q4_gemm_verify_tiled_noalloc(x, Wt, y, M, N, K)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), want.view(torch.int32))
    N2, K2, M2 = 248320, 5120, 32
    assert q4.q4_gemm_verify_tiled_ws_plan(M2, N2, K2)["workspace_bytes"] > \
        q4.NOALLOC_SCRATCH_BYTES
    lib = q4.load()
    st = lib.q4_gemm_verify_tiled_noalloc(x.data_ptr(), Wt.data_ptr(),
                                          y.data_ptr(), M2, N2, K2, None)
    assert st == q4.ESCRATCH
