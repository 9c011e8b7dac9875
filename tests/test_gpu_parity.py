"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Every case calls the library through the C ABI (via the ctypes binding) on
seeded inputs and hands the oracle the very bytes the GPU consumed.

Bar (per output element): |y_gpu - y64| <= 2e-3 * sum_k |x_k w_k| + 1e-5,
with y64 and the absolute sum from the oracle's fp64 accumulation.  The
dequantisation hook must be bit-exact, and so must the GEMM wherever every
partial sum is an exact fp32 value (integer-valued inputs, one-hot rows).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import (assemble, bf16_bits_of, oracle_threads,
                           tiled_from_planar)

pytestmark = pytest.mark.gpu

REL, ABS = 2e-3, 1e-5


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemm_q4_amd as lib
    lib.load()
    return lib


def _say(*args):
    print(*args, flush=True)


def gemm(q4, x, W, M, N, K):
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=x.device)
    q4.q4_gemm_verify(x, W, y, M, N, K)
    torch.cuda.synchronize()
    return y


def assert_within_bound(y_gpu, y64, a64, what=""):
    got = y_gpu.cpu().numpy().astype(np.float64) if torch.is_tensor(y_gpu) \
        else y_gpu.astype(np.float64)
    assert got.shape == y64.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - y64)
    bound = REL * a64 + ABS
    ratio = float(np.max(err / bound))
    assert ratio <= 1.0, f"{what}: max err/bound {ratio:.3g}"
    return ratio


def repacked(q4, W, N, K):
    Wt = torch.empty_like(W)
    q4.q4_repack(W, Wt, N, K)
    torch.cuda.synchronize()
    return Wt


def gemm_tiled(q4, x, Wt, M, N, K):
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=x.device)
    q4.q4_gemm_verify_tiled(x, Wt, y, M, N, K)
    torch.cuda.synchronize()
    return y


def oracle_check(q4, M, N, K, seed, what, tiled=False):
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=seed, device=dev)
    x = synth.activations(M, K, seed=seed, stream=1, device=dev)
    _say(f"case {what}: M={M} N={N} K={K} seed={seed} tiled={tiled}")
    if tiled:
        y = gemm_tiled(q4, x, repacked(q4, W, N, K), M, N, K)
    else:
        y = gemm(q4, x, W, M, N, K)
    _, y64, a64, _ = oracle.gemm(synth.bf16_bits(x), W.cpu().numpy(), N, K)
    return assert_within_bound(y, y64, a64, what)


# -------------------------------------------------------------- dequant

@pytest.mark.parametrize("N,K", [(256, 512), (17, 192), (1, 64), (1000, 1088)])
def test_dequant_bit_exact(q4, N, K):
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=3, device=dev)
    out = torch.empty((N, K), dtype=torch.float32, device=dev)
    _say(f"case dequant N={N} K={K}")
    q4.q4_dequant(W, out, N, K)
    torch.cuda.synchronize()
    want = oracle.dequant(W.cpu().numpy(), N, K)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


# -------------------------------------------------------------- GEMM, small

@pytest.mark.parametrize("M", list(range(1, 17)))
def test_gemm_tiny_every_M(q4, M):
    oracle_check(q4, M, 256, 512, 0, "tiny")


# Shapes chosen to cover every launch configuration of the kernel family
# (waves per workgroup splitting K: 1, 2, 4, 8, 16), ragged row tails (N not
# a multiple of 16 or 64), a single group (K = 64), odd group counts and a
# long K.
RAGGED = [(1, 1, 64), (3, 17, 192), (16, 257, 640), (5, 1000, 1088),
          (16, 33, 4096), (7, 16, 65536), (2, 48000, 512), (16, 48001, 512),
          (1, 70000, 256), (13, 70001, 256), (16, 4099, 5120)]


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_gemm_ragged_shapes(q4, M, N, K):
    oracle_check(q4, M, N, K, 1, "ragged")


def test_gemm_integer_exact_bitwise(q4):
    """Integer codes/activations, scale 1, bias -8: every partial sum is an
    exact fp32 integer, so any summation order must reproduce the oracle's
    fp32 result bit for bit."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(5)
    for (M, N, K) in [(16, 300, 1024), (1, 64, 64), (9, 2000, 3072)]:
        q = rng.integers(0, 16, size=(N, K))
        G = K // 64
        codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
        Wh = assemble(codes, bf16_bits_of(np.ones((N, G))),
                      bf16_bits_of(np.full((N, G), -8.0)))
        xi = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
        W = torch.from_numpy(Wh).to(dev)
        x = torch.from_numpy(xi).to(torch.bfloat16).to(dev)
        _say(f"case integer-exact M={M} N={N} K={K}")
        y = gemm(q4, x, W, M, N, K).cpu().numpy()
        y32, _, _, _ = oracle.gemm(bf16_bits_of(xi), Wh, N, K)
        assert np.array_equal(y.view(np.uint32), y32.view(np.uint32))


def test_gemm_one_hot_bitwise(q4):
    """x rows e_k: y[m, n] must be the dequantised weight w[n, k_m] exactly
    (the scale product is exact and the bias adds with one rounding)."""
    dev = torch.device("cuda")
    N, K = 200, 640
    W = synth.q4_weights(N, K, seed=7, device=dev)
    ks = [0, 1, 7, 8, 15, 16, 63, 64, 130, 255, 300, 511, 512, 600, 638, 639]
    x = torch.zeros((len(ks), K), dtype=torch.bfloat16, device=dev)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    _say("case one-hot")
    y = gemm(q4, x, W, len(ks), N, K).cpu().numpy()
    w = oracle.dequant(W.cpu().numpy(), N, K)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m].view(np.uint32), w[:, k].view(np.uint32)), k


def test_rows_do_not_depend_on_M(q4):
    """Row m of a 16-row block equals, bit for bit, the same row computed in
    any smaller block (rows are computed independently, same order)."""
    dev = torch.device("cuda")
    N, K = 1000, 2048
    W = synth.q4_weights(N, K, seed=8, device=dev)
    x = synth.activations(16, K, seed=8, stream=1, device=dev)
    _say("case M-invariance")
    full = gemm(q4, x, W, 16, N, K)
    for M in range(1, 16):
        part = gemm(q4, x[:M].contiguous(), W, M, N, K)
        assert torch.equal(part.view(torch.int32), full[:M].view(torch.int32)), M
    # and a row alone at another position of the block
    single = gemm(q4, x[11:12].contiguous(), W, 1, N, K)
    assert torch.equal(single.view(torch.int32), full[11:12].view(torch.int32))


def test_deterministic(q4):
    dev = torch.device("cuda")
    N, K, M = 5120, 17408, 16
    W = synth.q4_weights(N, K, seed=9, device=dev)
    x = synth.activations(M, K, seed=9, stream=1, device=dev)
    _say("case determinism")
    a = gemm(q4, x, W, M, N, K)
    b = gemm(q4, x, W, M, N, K)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_matches_torch_fp32_reference(q4):
    """Against plain PyTorch fp32: the kernels' own dequantised matrix times
    x in fp32 (a cross-check of the GEMM against the dequant hook)."""
    dev = torch.device("cuda")
    N, K, M = 3000, 2560, 8
    W = synth.q4_weights(N, K, seed=10, device=dev)
    x = synth.activations(M, K, seed=10, stream=1, device=dev)
    w = torch.empty((N, K), dtype=torch.float32, device=dev)
    q4.q4_dequant(W, w, N, K)
    _say("case torch-fp32")
    y = gemm(q4, x, W, M, N, K)
    ref = x.float() @ w.t()
    absum = x.float().abs() @ w.abs().t()
    assert torch.all((y - ref).abs() <= REL * absum + ABS)


# -------------------------------------------------------------- full shapes

FULL = {
    "gate_up": (34816, 5120),
    "down": (5120, 17408),
    "lm_head": (248320, 5120),
    "attn_in": (14336, 5120),
    "o_proj": (5120, 6144),
    "gdn_in": (16640, 5120),
}


def full_check(y, x, W, N, K, what):
    """Every output element of the call against the oracle, on the bytes the
    GPU consumed (the oracle runs on the host's CPU share of threads)."""
    assert torch.isfinite(y).all(), f"{what}: non-finite output"
    _, y64, a64, _ = oracle.gemm(synth.bf16_bits(x), W.cpu().numpy(), N, K,
                                 threads=oracle_threads())
    return assert_within_bound(y, y64, a64, what)


@pytest.mark.parametrize("name,M", [(n, m) for n in FULL for m in (1, 16)] +
                         [("gate_up", m) for m in (2, 4, 8)] +
                         [("down", m) for m in (2, 4, 8)])
def test_full_shape(q4, name, M):
    dev = torch.device("cuda")
    N, K = FULL[name]
    W = synth.q4_weights(N, K, seed=11, stream=list(FULL).index(name),
                          device=dev)
    x = synth.activations(M, K, seed=11, stream=2000 + M, device=dev)
    _say(f"case full {name}: M={M} N={N} K={K}")
    y = gemm(q4, x, W, M, N, K)
    full_check(y, x, W, N, K, f"{name} M={M}")


def test_lm_head_two_calls(q4):
    """The LM head serves two activation blocks per step (draft readout,
    then verify) from one resident weight buffer."""
    dev = torch.device("cuda")
    N, K, M = 248320, 5120, 16
    W = synth.q4_weights(N, K, seed=12, device=dev)
    for call in range(2):
        x = synth.activations(M, K, seed=12, stream=call, device=dev)
        _say(f"case lm-head call {call}")
        y = gemm(q4, x, W, M, N, K)
        full_check(y, x, W, N, K, f"lm head call {call}")


# -------------------------------------------------------------- tiled layout

TILED = [(16, 16, 256), (1, 16, 256), (16, 256, 512), (5, 1600, 1024),
         (5, 1600, 2048), (16, 5120, 6144), (3, 5120, 17408),
         (16, 80000, 1024), (7, 1040, 256), (16, 2048, 4096),
         # K-slice kernel: an odd record count (the last wave takes one),
         # 23 records, and 20 tiles per workgroup (two reduction batches);
         # M >= 8 stages the activations through LDS: odd records, 8 and
         # 11 rows, 12 waves
         (4, 4800, 1280), (16, 512, 5888), (16, 81920, 5120),
         (8, 4800, 1280), (11, 1600, 6144), (9, 48, 5632)]


@pytest.mark.parametrize("N,K", [(16, 256), (256, 512), (1600, 2048),
                                 (5120, 6144)])
def test_repack_bytes(q4, N, K):
    """q4_repack against the layout restated in numpy from its definition."""
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=20, device=dev)
    _say(f"case repack N={N} K={K}")
    Wt = repacked(q4, W, N, K).cpu().numpy()
    assert np.array_equal(Wt, tiled_from_planar(W.cpu().numpy(), N, K))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 9, 15, 16])
def test_tiled_tiny(q4, M):
    oracle_check(q4, M, 256, 512, 0, "tiled tiny", tiled=True)


def test_resident_empty_waves_after_other_lds_users(q4):
    """Small shapes where most of a workgroup's waves get no records (their
    weight loads all fall past their range and return at once), each call
    preceded by kernels that leave other data in LDS: the K-slice kernel
    (one or two row tiles, parts of K in turn) must not read another
    kernel's LDS for its partial sums or running sums."""
    dev = torch.device("cuda")
    Wp = synth.q4_weights(2048, 4096, seed=40, device=dev)
    Wtp = repacked(q4, Wp, 2048, 4096)
    xp = synth.activations(16, 4096, seed=40, stream=1, device=dev)
    yp = torch.empty((16, 2048), dtype=torch.float32, device=dev)
    for N, K in [(16, 256), (16, 512), (48, 256), (256, 512), (32, 5120)]:
        W = synth.q4_weights(N, K, seed=41, device=dev)
        Wt = repacked(q4, W, N, K)
        for M in (1, 4, 16, 24):
            p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
            assert p["kernel"] == q4.KERNEL_TILED_KSLICE
            assert p["m_tiles"] == (2 if M > 16 else 1)
            x = synth.activations(M, K, seed=41 + M, stream=1, device=dev)
            _, y64, a64, _ = oracle.gemm(synth.bf16_bits(x), W.cpu().numpy(),
                                         N, K)
            for rep in range(3):
                # both other kernels leave their own data in LDS
                q4.q4_gemm_verify(xp, Wp, yp, 16, 2048, 4096)
                q4.q4_gemm_verify_tiled(xp, Wtp, yp, 16, 2048, 4096)
                _say(f"case small tiled shapes: N={N} K={K} M={M} rep={rep}")
                y = gemm_tiled(q4, x, Wt, M, N, K)
                assert_within_bound(y, y64, a64,
                                    f"tiled N={N} K={K} M={M} rep={rep}")


@pytest.mark.parametrize("M,N,K", TILED)
def test_tiled_shapes(q4, M, N, K):
    """Shapes covering every launch configuration of the tiled kernel."""
    oracle_check(q4, M, N, K, 2, "tiled", tiled=True)


def test_tiled_integer_exact_and_M_invariance(q4):
    dev = torch.device("cuda")
    rng = np.random.default_rng(21)
    N, K = 2048, 3072
    q = rng.integers(0, 16, size=(N, K))
    G = K // 64
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    Wh = assemble(codes, bf16_bits_of(np.ones((N, G))),
                  bf16_bits_of(np.full((N, G), -8.0)))
    xi = rng.integers(-4, 5, size=(16, K)).astype(np.float32)
    Wt = repacked(q4, torch.from_numpy(Wh).to(dev), N, K)
    x = torch.from_numpy(xi).to(torch.bfloat16).to(dev)
    _say("case tiled integer-exact")
    y = gemm_tiled(q4, x, Wt, 16, N, K)
    y32, _, _, _ = oracle.gemm(bf16_bits_of(xi), Wh, N, K)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y32.view(np.uint32))
    # random data: rows do not depend on M, and the planar kernel agrees
    W = synth.q4_weights(N, K, seed=22, device=dev)
    Wt = repacked(q4, W, N, K)
    xr = synth.activations(16, K, seed=22, stream=1, device=dev)
    full = gemm_tiled(q4, xr, Wt, 16, N, K)
    for M in (1, 5, 12):
        part = gemm_tiled(q4, xr[:M].contiguous(), Wt, M, N, K)
        assert torch.equal(part.view(torch.int32), full[:M].view(torch.int32))
    _, y64, a64, _ = oracle.gemm(synth.bf16_bits(xr), W.cpu().numpy(), N, K)
    assert_within_bound(full, y64, a64, "tiled random")


def test_tiled_one_hot_bitwise(q4):
    dev = torch.device("cuda")
    N, K = 160, 768
    W = synth.q4_weights(N, K, seed=23, device=dev)
    ks = [0, 1, 63, 64, 255, 256, 300, 511, 512, 767]
    x = torch.zeros((len(ks), K), dtype=torch.bfloat16, device=dev)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    _say("case tiled one-hot")
    y = gemm_tiled(q4, x, repacked(q4, W, N, K), len(ks), N, K).cpu().numpy()
    w = oracle.dequant(W.cpu().numpy(), N, K)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m].view(np.uint32), w[:, k].view(np.uint32)), k


@pytest.mark.parametrize("name,M", [(n, m) for n in FULL for m in (1, 16)] +
                         [(n, m) for n in ("gate_up", "down", "o_proj")
                          for m in (2, 4, 8)])
def test_tiled_full_shape(q4, name, M):
    dev = torch.device("cuda")
    N, K = FULL[name]
    W = synth.q4_weights(N, K, seed=13, stream=list(FULL).index(name),
                          device=dev)
    Wt = repacked(q4, W, N, K)
    x = synth.activations(M, K, seed=13, stream=3000 + M, device=dev)
    _say(f"case tiled full {name}: M={M} N={N} K={K}")
    y = gemm_tiled(q4, x, Wt, M, N, K)
    full_check(y, x, W, N, K, f"tiled {name} M={M}")


# -------------------------------------------------------------- workspace path

def gemm_tiled_ws(q4, x, Wt, M, N, K, fill=float("nan")):
    y = torch.full((M, N), fill, dtype=torch.float32, device=x.device)
    ws = q4.workspace_for(M, N, K, x.device)
    if ws is not None:
        ws.fill_(0xFF)  # stale workspace bytes must not matter
    q4.q4_gemm_verify_tiled_ws(x, Wt, y, M, N, K, ws)
    torch.cuda.synchronize()
    return y


# K > 5120 (split across workgroups, partial sums reduced in part order),
# including tiny N (most waves empty) and a part count above 4
WS_SHAPES = [(16, 5120, 6400), (16, 5120, 7168), (3, 5120, 17408), (1, 16, 10496),
             (16, 48, 10240), (8, 1600, 7168), (16, 256, 65536),
             (9, 32, 6656)]


@pytest.mark.parametrize("M,N,K", WS_SHAPES)
def test_workspace_split_shapes(q4, M, N, K):
    dev = torch.device("cuda")
    p = q4.q4_gemm_verify_tiled_ws_plan(M, N, K)
    assert p["k_parts"] > 1 and p["workspace_bytes"] > 0
    W = synth.q4_weights(N, K, seed=30, device=dev)
    x = synth.activations(M, K, seed=30, stream=1, device=dev)
    _say(f"case workspace split: M={M} N={N} K={K} parts={p['k_parts']}")
    y = gemm_tiled_ws(q4, x, repacked(q4, W, N, K), M, N, K)
    _, y64, a64, _ = oracle.gemm(synth.bf16_bits(x), W.cpu().numpy(), N, K)
    assert_within_bound(y, y64, a64, f"workspace M={M} N={N} K={K}")


def test_workspace_integer_exact_M_invariance_determinism(q4):
    dev = torch.device("cuda")
    rng = np.random.default_rng(31)
    N, K = 512, 6656
    q = rng.integers(0, 16, size=(N, K))
    G = K // 64
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    Wh = assemble(codes, bf16_bits_of(np.ones((N, G))),
                  bf16_bits_of(np.full((N, G), -8.0)))
    xi = rng.integers(-4, 5, size=(16, K)).astype(np.float32)
    Wt = repacked(q4, torch.from_numpy(Wh).to(dev), N, K)
    x = torch.from_numpy(xi).to(torch.bfloat16).to(dev)
    _say("case workspace integer-exact")
    y = gemm_tiled_ws(q4, x, Wt, 16, N, K)
    y32, _, _, _ = oracle.gemm(bf16_bits_of(xi), Wh, N, K)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y32.view(np.uint32))
    # random data: rows do not depend on M; calls repeat bit for bit
    N, K = 5120, 17408
    W = synth.q4_weights(N, K, seed=32, device=dev)
    Wt = repacked(q4, W, N, K)
    xr = synth.activations(16, K, seed=32, stream=1, device=dev)
    _say("case workspace M-invariance")
    full = gemm_tiled_ws(q4, xr, Wt, 16, N, K)
    again = gemm_tiled_ws(q4, xr, Wt, 16, N, K, fill=0.0)
    assert torch.equal(full.view(torch.int32), again.view(torch.int32))
    for M in (1, 2, 5, 8, 13):
        part = gemm_tiled_ws(q4, xr[:M].contiguous(), Wt, M, N, K)
        assert torch.equal(part.view(torch.int32), full[:M].view(torch.int32)), M


def test_workspace_path_equals_plain_call_when_unsplit(q4):
    """For K <= 5120 the workspace call runs the plain call's kernel."""
    dev = torch.device("cuda")
    N, K, M = 4096, 5120, 16
    assert q4.q4_gemm_verify_tiled_ws_plan(M, N, K)["workspace_bytes"] == 0
    W = synth.q4_weights(N, K, seed=33, device=dev)
    Wt = repacked(q4, W, N, K)
    x = synth.activations(M, K, seed=33, stream=1, device=dev)
    _say("case workspace unsplit")
    a = gemm_tiled(q4, x, Wt, M, N, K)
    b = gemm_tiled_ws(q4, x, Wt, M, N, K)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("name,M", [(n, m) for n in FULL for m in (1, 16)] +
                         [(n, m) for n in ("gate_up", "down", "o_proj")
                          for m in (2, 4, 8)])
def test_workspace_full_shape(q4, name, M):
    """The workspace entry point at every production shape (the launch the
    bench times), every output element against the oracle."""
    dev = torch.device("cuda")
    N, K = FULL[name]
    W = synth.q4_weights(N, K, seed=14, stream=list(FULL).index(name),
                          device=dev)
    Wt = repacked(q4, W, N, K)
    x = synth.activations(M, K, seed=14, stream=4000 + M, device=dev)
    _say(f"case workspace full {name}: M={M} N={N} K={K}")
    y = gemm_tiled_ws(q4, x, Wt, M, N, K)
    full_check(y, x, W, N, K, f"workspace {name} M={M}")


# -------------------------------------------------------------- 17..32 rows

@pytest.mark.parametrize("M", [17, 20, 24, 31, 32])
def test_two_row_tiles_tiny(q4, M):
    """Plain tiled call, K <= 2560: both row tiles from LDS, one split-free
    pass (the multi-lane shapes of the Splash engine)."""
    oracle_check(q4, M, 256, 512, 0, "two row tiles", tiled=True)


@pytest.mark.parametrize("M,N,K", [(32, 5120, 6144), (24, 48, 10240),
                                   (17, 16, 5120), (32, 1600, 2560),
                                   (25, 256, 17408)])
def test_two_row_tiles_workspace(q4, M, N, K):
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=50, device=dev)
    x = synth.activations(M, K, seed=50, stream=1, device=dev)
    p = q4.q4_gemm_verify_tiled_ws_plan(M, N, K)
    assert p["m_tiles"] == 2
    _say(f"case two row tiles workspace: M={M} N={N} K={K} "
         f"parts={p['k_parts']}")
    y = gemm_tiled_ws(q4, x, repacked(q4, W, N, K), M, N, K)
    _, y64, a64, _ = oracle.gemm(synth.bf16_bits(x), W.cpu().numpy(), N, K)
    assert_within_bound(y, y64, a64, f"two row tiles M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(32, 34816, 5120), (24, 5120, 17408),
                                   (17, 5120, 6144), (32, 16, 3072),
                                   (29, 2064, 6656)])
def test_two_row_tiles_plain_call(q4, M, N, K):
    """17..32 rows without a workspace: two row tiles, K beyond 12 records
    in parts taken one after another; every output against the oracle, and
    bitwise equal to the workspace call when that one runs unsplit."""
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=54, device=dev)
    x = synth.activations(M, K, seed=54, stream=1, device=dev)
    p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
    assert p["kernel"] == q4.KERNEL_TILED_KSLICE and p["m_tiles"] == 2
    _say(f"case two row tiles plain: M={M} N={N} K={K} "
         f"seq={p['k_seq_parts']}")
    Wt = repacked(q4, W, N, K)
    y = gemm_tiled(q4, x, Wt, M, N, K)
    full_check(y, x, W, N, K, f"two row tiles plain M={M} N={N} K={K}")
    if p["k_seq_parts"] == 1:
        assert torch.equal(y.view(torch.int32),
                           gemm_tiled_ws(q4, x, Wt, M, N, K).view(torch.int32))


def test_two_row_tiles_integer_exact_and_M_invariance(q4):
    """Integer-valued inputs: bitwise equal to the oracle at 32 rows; rows
    do not depend on M within 17..32 (the same plan and summation order)."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(51)
    N, K = 512, 5120
    q = rng.integers(0, 16, size=(N, K))
    G = K // 64
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    Wh = assemble(codes, bf16_bits_of(np.ones((N, G))),
                  bf16_bits_of(np.full((N, G), -8.0)))
    xi = rng.integers(-4, 5, size=(32, K)).astype(np.float32)
    Wt = repacked(q4, torch.from_numpy(Wh).to(dev), N, K)
    x = torch.from_numpy(xi).to(torch.bfloat16).to(dev)
    _say("case two row tiles integer-exact")
    y = gemm_tiled_ws(q4, x, Wt, 32, N, K)
    y32, _, _, _ = oracle.gemm(bf16_bits_of(xi), Wh, N, K)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y32.view(np.uint32))
    W = synth.q4_weights(34816 // 4, K, seed=52, device=dev)
    Wt = repacked(q4, W, 34816 // 4, K)
    xr = synth.activations(32, K, seed=52, stream=1, device=dev)
    full = gemm_tiled_ws(q4, xr, Wt, 32, 34816 // 4, K)
    for M in (17, 24, 31):
        part = gemm_tiled_ws(q4, xr[:M].contiguous(), Wt, M, 34816 // 4, K)
        assert torch.equal(part.view(torch.int32), full[:M].view(torch.int32)), M


@pytest.mark.parametrize("name,M", [("gate_up", 32), ("down", 24),
                                    ("lm_head", 32)])
def test_two_row_tiles_full_shape(q4, name, M):
    dev = torch.device("cuda")
    N, K = FULL[name]
    W = synth.q4_weights(N, K, seed=53, stream=list(FULL).index(name),
                          device=dev)
    Wt = repacked(q4, W, N, K)
    x = synth.activations(M, K, seed=53, stream=5000 + M, device=dev)
    _say(f"case two row tiles full {name}: M={M} N={N} K={K}")
    y = gemm_tiled_ws(q4, x, Wt, M, N, K)
    full_check(y, x, W, N, K, f"two row tiles {name} M={M}")


# -------------------------------------------------------------- probes

def test_stream_probes(q4):
    dev = torch.device("cuda")
    src = torch.randint(0, 255, (1 << 22,), dtype=torch.uint8, device=dev)
    dst = torch.zeros_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    _say("case probes")
    q4.q4_stream_copy(src, dst, src.numel())
    q4.q4_stream_read(src, src.numel(), sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# -------------------------------------------------------------- planar K-slice

def test_planar_kslice_one_hot_and_integer_exact(q4):
    """q4_gemm_verify on the planar layout takes the K-slice kernel for
    K % 256 == 0: one-hot rows reproduce dequantised weights bit for bit
    (the code words are regrouped across lanes and the activations permuted
    to match, which must not change any product), and integer-valued inputs
    give the oracle's fp32 result bit for bit, also with sequential parts of
    K (K = 6656: two parts) and a ragged N."""
    dev = torch.device("cuda")
    for N, K in [(200, 768), (37, 6656)]:
        plan = q4.q4_gemm_verify_plan(16, N, K, q4.LAYOUT_PLANAR)
        assert plan["kernel"] == q4.KERNEL_TILED_KSLICE
        W = synth.q4_weights(N, K, seed=80, device=dev)
        ks = [0, 1, 7, 8, 63, 64, 130, 255, 256, 300, 511, K - 257, K - 64,
              K - 9, K - 2, K - 1]
        x = torch.zeros((len(ks), K), dtype=torch.bfloat16, device=dev)
        for m, k in enumerate(ks):
            x[m, k] = 1.0
        _say(f"case planar one-hot N={N} K={K} seq={plan['k_seq_parts']}")
        y = gemm(q4, x, W, len(ks), N, K).cpu().numpy()
        w = oracle.dequant(W.cpu().numpy(), N, K)
        for m, k in enumerate(ks):
            assert np.array_equal(y[m].view(np.uint32), w[:, k].view(np.uint32)), (N, K, k)
    rng = np.random.default_rng(81)
    for M, N, K in [(16, 300, 1024), (9, 1000, 3072), (16, 77, 6656)]:
        q = rng.integers(0, 16, size=(N, K))
        G = K // 64
        codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
        Wh = assemble(codes, bf16_bits_of(np.ones((N, G))),
                      bf16_bits_of(np.full((N, G), -8.0)))
        xi = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
        W = torch.from_numpy(Wh).to(dev)
        x = torch.from_numpy(xi).to(torch.bfloat16).to(dev)
        _say(f"case planar integer-exact M={M} N={N} K={K}")
        y = gemm(q4, x, W, M, N, K).cpu().numpy()
        y32, _, _, _ = oracle.gemm(bf16_bits_of(xi), Wh, N, K)
        assert np.array_equal(y.view(np.uint32), y32.view(np.uint32)), (M, N, K)


def test_sequential_parts_M_invariance_determinism(q4):
    """K beyond 24 records without a workspace: each workgroup takes the
    parts of K in turn (planar and tiled).  Rows do not depend on M, repeated
    calls agree bit for bit, and the result is within the bound."""
    dev = torch.device("cuda")
    N, K = 5120, 17408
    W = synth.q4_weights(N, K, seed=82, device=dev)
    Wt = repacked(q4, W, N, K)
    x = synth.activations(16, K, seed=82, stream=1, device=dev)
    for layout, Wx, call in ((q4.LAYOUT_PLANAR, W, gemm),
                             (q4.LAYOUT_TILED16, Wt, gemm_tiled)):
        plan = q4.q4_gemm_verify_plan(16, N, K, layout)
        assert plan["k_seq_parts"] > 1 and plan["workspace_bytes"] == 0
        _say(f"case sequential parts layout={layout} seq={plan['k_seq_parts']}")
        full = call(q4, x, Wx, 16, N, K)
        again = call(q4, x, Wx, 16, N, K)
        assert torch.equal(full.view(torch.int32), again.view(torch.int32))
        for M in (1, 3, 8, 13):
            part = call(q4, x[:M].contiguous(), Wx, M, N, K)
            assert torch.equal(part.view(torch.int32), full[:M].view(torch.int32)), (layout, M)
        full_check(full, x, W, N, K, f"sequential parts layout {layout}")


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(1, 34816, 5120), (16, 5120, 6144),
                                   (5, 5120, 17408), (16, 5120, 17408),
                                   (8, 4112, 6656)])
def test_planar_equals_tiled_bitwise(q4, M, N, K):
    """The planar entry point and the tiled one multiply the same products
    in the same order (the same K slice per MFMA operand slot, the same
    parts): their outputs are equal bit for bit on the model's shapes, and
    both within the oracle's bound."""
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=21, device=dev)
    x = synth.activations(M, K, seed=21, stream=1, device=dev)
    _say(f"case planar==tiled: M={M} N={N} K={K}")
    pl = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_PLANAR)
    tl = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
    assert pl["kernel"] == tl["kernel"] == q4.KERNEL_TILED_KSLICE
    assert pl["k_seq_parts"] == tl["k_seq_parts"]
    yp = gemm(q4, x, W, M, N, K)
    yt = gemm_tiled(q4, x, repacked(q4, W, N, K), M, N, K)
    assert torch.equal(yp.view(torch.int32), yt.view(torch.int32))
    full_check(yp, x, W, N, K, "planar==tiled")


# -------------------------------------------------------------- VALU variant

@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (4, 256, 512), (3, 48, 256),
                                   (2, 4112, 5120), (4, 5120, 6144),
                                   (1, 34816, 5120), (4, 34816, 5120)])
def test_dot_variant(q4, M, N, K):
    """The v_dot2 variant (M <= 4): every output within the oracle's bound;
    it sums in another order than the MFMA path, so only the bound ties
    the two."""
    dev = torch.device("cuda")
    W = synth.q4_weights(N, K, seed=60, device=dev)
    x = synth.activations(M, K, seed=60, stream=1, device=dev)
    Wt = repacked(q4, W, N, K)
    _say(f"case dot variant: M={M} N={N} K={K}")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    q4.q4_gemm_verify_tiled_dot(x, Wt, y, M, N, K)
    torch.cuda.synchronize()
    full_check(y, x, W, N, K, f"dot M={M} N={N} K={K}")


@pytest.mark.gpu
def test_dot_variant_integer_exact_and_M_invariance(q4):
    """Integer-valued codes and activations (scale 1, bias -8): every
    partial sum is an exact fp32 integer, so the v_dot2 path equals the
    oracle bit for bit; rows do not depend on M."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(61)
    N, K = 1024, 6144
    q = rng.integers(0, 16, size=(N, K))
    G = K // 64
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    Wh = assemble(codes, bf16_bits_of(np.ones((N, G))),
                  bf16_bits_of(np.full((N, G), -8.0)))
    xi = rng.integers(-4, 5, size=(4, K)).astype(np.float32)
    Wt = repacked(q4, torch.from_numpy(Wh).to(dev), N, K)
    x = torch.from_numpy(xi).to(torch.bfloat16).to(dev)
    _say("case dot variant integer-exact")
    y = torch.empty((4, N), dtype=torch.float32, device=dev)
    q4.q4_gemm_verify_tiled_dot(x, Wt, y, 4, N, K)
    torch.cuda.synchronize()
    y32, _, _, _ = oracle.gemm(bf16_bits_of(xi), Wh, N, K)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y32.view(np.uint32))
    for M in (1, 2, 3):
        part = torch.empty((M, N), dtype=torch.float32, device=dev)
        q4.q4_gemm_verify_tiled_dot(x[:M].contiguous(), Wt, part, M, N, K)
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int32), y[:M].view(torch.int32)), M
