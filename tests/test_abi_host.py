"""The C ABI library on the host (no GPU): exports, layout, argument checks.

Every call here either is host-only (q4_pack_layout, q4_status_string) or is
rejected by the argument checks before the library touches the HIP runtime.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import re

import pytest
import torch

import oracle
import synth
import speculative_verify_gemm_q4_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4verify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q4.LIB_PATH):
        pytest.fail("libq4verify.so is not built (run __graft_entry__.build())")
    return q4.load()


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_\w+)\s*\(", text)))


def test_header_declares_the_binding_entry_points():
    assert declared_functions() == q4.lib_exports()


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", q4.LIB_PATH],
                        capture_output=True, text=True, check=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", nm, flags=re.M), name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, -6):
        s = q4.q4_status_string(st)
        assert s.startswith("Q4_")
    assert q4.q4_status_string(12345) == "unknown q4 status"


@pytest.mark.parametrize("N,K", [(1, 64), (3, 192), (256, 512), (34816, 5120),
                                 (5120, 17408), (248320, 5120), (5120, 6144),
                                 (7, 1088)])
def test_layout_matches_oracle_and_generator(lib, N, K):
    lay = q4.q4_pack_layout(N, K)
    assert lay["abi_version"] == 2 and lay["layout_id"] == 0
    assert lay["N"] == N and lay["K"] == K and lay["group"] == 64
    assert lay["total_bytes"] == oracle.packed_bytes(N, K)
    assert lay["total_bytes"] == synth.packed_size(N, K)
    assert lay["code_off"] == 0 and lay["code_bytes"] == N * K // 2
    assert lay["scale_off"] == N * K // 2 and lay["scale_bytes"] == N * K // 32
    assert lay["bias_off"] == lay["scale_off"] + lay["scale_bytes"]
    assert lay["bias_off"] + lay["bias_bytes"] == lay["total_bytes"]
    # the generator's plane views start where the library says
    if N * K <= 1 << 20:
        W = torch.zeros(lay["total_bytes"], dtype=torch.uint8)
        c, s, b = synth.planes(W, N, K)
        base = W.data_ptr()
        assert c.data_ptr() - base == lay["code_off"]
        assert s.data_ptr() - base == lay["scale_off"]
        assert b.data_ptr() - base == lay["bias_off"]


@pytest.mark.parametrize("N,K", [(16, 256), (256, 512), (34816, 5120),
                                 (5120, 17408), (248320, 5120), (5120, 6144)])
def test_tiled_layout(lib, N, K):
    lay = q4.q4_pack_layout(N, K, q4.LAYOUT_TILED16)
    assert lay["layout_id"] == 1
    assert lay["total_bytes"] == oracle.packed_bytes(N, K)
    assert lay["tile_rows"] == 16 and lay["record_groups"] == 4
    assert lay["record_bytes"] == 2304 == 16 * 4 * 64 * 9 // 16
    assert lay["total_bytes"] == (N // 16) * (K // 256) * lay["record_bytes"]
    assert lay["code_bytes"] == lay["scale_bytes"] == lay["bias_bytes"] == 0


def test_tiled_shape_rules(lib):
    from speculative_verify_gemm_q4_amd._lib import _Layout
    out = _Layout()
    f = lib.q4_pack_layout
    assert f(17, 256, 1, ctypes.byref(out)) == -1      # N % 16
    assert f(16, 192, 1, ctypes.byref(out)) == -1      # K % 256
    assert f(16, (1 << 26) + 256, 1, ctypes.byref(out)) == -1  # K > 2^26
    g = lib.q4_gemm_verify_tiled
    X, W, Y = 0x10000, 0x20000, 0x30000
    assert g(X, W, Y, 1, 17, 256, None) == -1
    assert g(X, W, Y, 1, 16, 320, None) == -1
    assert g(X, W, Y, 0, 16, 256, None) == -1
    assert g(X, W, Y, 33, 16, 256, None) == -1        # M above 32
    # M > 16 and K beyond 12 records: parts in turn, valid (stops at the
    # device check); with more than 16 tiles per workgroup (the LM head) it
    # needs the workspace call
    assert g(X, W, Y, 17, 16, 2816, None) == -4
    assert g(X, W, Y, 32, 248320, 5120, None) == -1
    assert g(X, W, Y, 17, 16, 256, None) == -4        # valid: stops at device
    assert g(X + 8, W, Y, 1, 16, 256, None) == -2
    r = lib.q4_repack
    assert r(W, X, 17, 256, None) == -1
    assert r(W, X, 16, 320, None) == -1
    assert r(W + 4, X, 16, 256, None) == -2
    assert r(W, X + 4, 16, 256, None) == -2


def test_layout_errors(lib):
    from speculative_verify_gemm_q4_amd._lib import _Layout
    out = _Layout()
    f = lib.q4_pack_layout
    assert f(0, 64, 0, ctypes.byref(out)) == -1
    assert f(4, 96, 0, ctypes.byref(out)) == -1
    assert f(4, 64, 7, ctypes.byref(out)) == -1
    assert f(4, 64, 0, None) == -1
    assert f(1 << 40, 1 << 30, 0, ctypes.byref(out)) == -3
    assert out.total_bytes == 0  # untouched on error


def test_gemm_argument_errors(lib):
    """Each rejected before any device work (fake, never-dereferenced
    pointers)."""
    g = lib.q4_gemm_verify
    X, W, Y = 0x10000, 0x20000, 0x30000
    assert g(X, W, Y, 0, 256, 512, None) == -1        # M = 0 (empty block)
    assert g(X, W, Y, 17, 256, 512, None) == -1       # M above 16
    assert g(X, W, Y, 1, 0, 512, None) == -1          # N = 0 (empty matrix)
    assert g(X, W, Y, 1, 256, 0, None) == -1          # K = 0
    assert g(X, W, Y, 1, 256, 500, None) == -1        # K not a multiple of 64
    assert g(X, W, Y, 1, 1 << 31, 64, None) == -1     # N beyond int32
    assert g(None, W, Y, 1, 256, 512, None) == -1
    assert g(X, None, Y, 1, 256, 512, None) == -1
    assert g(X, W, None, 1, 256, 512, None) == -1
    assert g(X + 2, W, Y, 1, 256, 512, None) == -2    # x not 16-B aligned
    assert g(X, W + 8, Y, 1, 256, 512, None) == -2    # W not 16-B aligned
    assert g(X, W, Y + 2, 1, 256, 512, None) == -2    # y not 4-B aligned


def test_workspace_gemm_argument_errors(lib):
    """The workspace path: same rules as the tiled call, plus the workspace
    (too small, missing or misaligned) -- all rejected before device work."""
    g = lib.q4_gemm_verify_tiled_ws
    X, W, Y, S = 0x10000, 0x20000, 0x30000, 0x40000
    need = q4.q4_gemm_verify_tiled_ws_plan(16, 5120, 17408)["workspace_bytes"]
    assert need == 3 * 16 * 5120 * 4
    assert g(X, W, Y, 16, 5120, 17408, None, 0, None) == -1
    assert g(X, W, Y, 16, 5120, 17408, S, need - 16, None) == -1
    assert g(X, W, Y, 16, 5120, 17408, S + 8, need, None) == -2
    assert g(X, W, Y, 0, 5120, 17408, S, need, None) == -1
    assert g(X, W, Y, 16, 5121, 17408, S, need, None) == -1   # N % 16
    assert g(X, W, Y, 16, 5120, 17400, S, need, None) == -1   # K % 256
    # K <= 5120 needs no workspace, K > 5120 needs (P - 1) M N floats
    assert q4.q4_gemm_verify_tiled_ws_plan(16, 34816, 5120)[
        "workspace_bytes"] == 0
    p = q4.q4_gemm_verify_tiled_ws_plan(3, 5120, 6144)
    assert p["workspace_bytes"] == (p["k_parts"] - 1) * 3 * 5120 * 4


@pytest.mark.parametrize("layout", [0, 1])
def test_plans_of_many_shapes(lib, layout):
    """The planners over small, odd and large shapes, every M: each returns
    a plan (or a clean error) whose grid, waves and parts fit the kernels'
    limits; none may fault on the host."""
    Ks = [64, 128, 192, 256, 512, 640, 1024, 5120, 6144, 6400, 6656, 17408,
          65536, 262144]
    Ns = [1, 15, 16, 17, 100, 5120, 34816, 248320]
    for K in Ks:
        for N in Ns:
            if layout == 1 and (N % 16 or K % 256):
                continue
            for M in (1, 2, 7, 8, 16, 17, 32):
                try:
                    p = q4.q4_gemm_verify_plan(M, N, K, layout)
                except q4.Q4Error:
                    continue
                assert 1 <= p["grid"] and 64 <= p["block"] <= 1024, (M, N, K, p)
                assert p["k_parts"] >= 1 and p["k_seq_parts"] >= 1
                assert p["layout_id"] == layout
                if p["kernel"] == q4.KERNEL_TILED_KSLICE:
                    assert p["block"] // 64 <= 12
                    assert p["m_tiles"] == (2 if M > 16 else 1)
                    records = K // 256
                    parts = p["k_parts"] * p["k_seq_parts"]
                    assert parts <= records
                    assert -(-records // parts) <= (12 if M > 16 else 24)
                    if p["k_seq_parts"] > 1:
                        assert p["row_tiles"] <= 16
                # planar: the K-slice kernel whenever one part of K fits, or
                # the sequential parts' tile accumulators hold a workgroup's
                # share of the rows
                per = -(-(-(-N // 16)) // 256)  # 256 CUs without a device
                if (layout == 0 and M <= 16 and K % 256 == 0 and K >= 256
                        and (K <= 6144 or per <= 4)):
                    assert p["kernel"] == q4.KERNEL_TILED_KSLICE, (M, N, K)


def test_noalloc_gemm_argument_errors(lib):
    """The no-allocation entry point: the tiled call's rules, and a shape
    whose K split needs more than the static scratch is refused with
    Q4_ESCRATCH -- all before any device work."""
    g = lib.q4_gemm_verify_tiled_noalloc
    X, W, Y = 0x10000, 0x20000, 0x30000
    assert q4.ESCRATCH == -6 and q4.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert g(X, W, Y, 0, 5120, 17408, None) == -1
    assert g(X, W, Y, 33, 5120, 17408, None) == -1
    assert g(X, W, Y, 16, 5121, 17408, None) == -1   # N % 16
    assert g(X, W, Y, 16, 5120, 17400, None) == -1   # K % 256
    assert g(X + 8, W, Y, 16, 5120, 17408, None) == -2
    assert g(None, W, Y, 16, 5120, 17408, None) == -1
    # the LM head at 32 rows splits K in two: 30 MiB of partial products
    assert q4.q4_gemm_verify_tiled_ws_plan(32, 248320, 5120)[
        "workspace_bytes"] > q4.NOALLOC_SCRATCH_BYTES
    assert g(X, W, Y, 32, 248320, 5120, None) == -6
    # every projection of the model fits at 32 rows but that one
    for N, K in [(34816, 5120), (5120, 17408), (14336, 5120), (5120, 6144),
                 (16640, 5120)]:
        assert q4.q4_gemm_verify_tiled_ws_plan(32, N, K)[
            "workspace_bytes"] <= q4.NOALLOC_SCRATCH_BYTES


def test_fused_sample_argument_errors(lib):
    """q4_gemm_verify_sample: shapes outside its rule (K beyond one part
    of the K-slice kernel, more than 64 tiles per workgroup, M > 16) and a
    small workspace are rejected before any device work."""
    ws = q4.q4_gemm_verify_sample_workspace
    assert ws(16, 248320, 5120) == 16 * 255 * 32 * 8  # 255 workgroups
    for M, N, K in [(16, 5120, 6400), (17, 5120, 5120), (16, 16 * 64 * 256 + 16, 5120),
                    (16, 5120, 5000), (0, 5120, 5120)]:
        with pytest.raises(q4.Q4Error):
            ws(M, N, K)
    g = lib.q4_gemm_verify_sample
    X, W, P = 0x10000, 0x20000, 0x30000
    prm = q4._lib._SampleParams(1.0, 0.9, 20, 0)
    outs = [P] * 9
    need = ws(16, 34816, 5120)
    assert g(X, W, 16, 34816, 5120, ctypes.byref(prm), P, None, None, P, P,
             *outs[:6], P, need - 8, None) == -1
    assert g(X, W, 16, 34816, 5120, ctypes.byref(prm), P, None, None, P, P,
             *outs[:6], P + 4, need, None) == -2
    bad = q4._lib._SampleParams(1.0, 0.9, 33, 0)
    assert g(X, W, 16, 34816, 5120, ctypes.byref(bad), P, None, None, P, P,
             *outs[:6], P, need, None) == -1


def test_verify_sample_argument_errors(lib):
    """Sizes and sampling parameters are rejected before device work."""
    from speculative_verify_gemm_q4_amd._lib import _SampleParams
    n = ctypes.c_uint64(0)
    w = lib.q4_verify_sample_workspace
    assert w(16, 248320, ctypes.byref(n)) == 0 and n.value == 16 * 16 * 32 * 8
    assert w(0, 100, ctypes.byref(n)) == -1
    assert w(1025, 100, ctypes.byref(n)) == -1
    assert w(1, 0, ctypes.byref(n)) == -1
    assert w(1, 1 << 31, ctypes.byref(n)) == -1
    # the longest row: 512 slices of 16384 columns
    assert w(1, 8388608, ctypes.byref(n)) == 0 and n.value == 512 * 32 * 8
    assert w(1, 8388609, ctypes.byref(n)) == -1
    f = lib.q4_verify_sample
    P = [0x10000 + 0x1000 * i for i in range(12)]   # fake device pointers
    WS, NWS = 0x90000, 4096

    def call(M=2, V=1000, T=1.0, top_p=0.9, k=20, kd=4, ptrs=P, ws=WS,
             nws=NWS):
        prm = _SampleParams(T, top_p, k, kd)
        return f(ptrs[0], M, V, ctypes.byref(prm), *ptrs[1:], ws, nws, None)
    assert call(k=0) == -1 and call(k=33) == -1 and call(V=10, k=11) == -1
    assert call(kd=17) == -1 and call(kd=-1) == -1
    assert call(T=-1.0) == -1 and call(T=float("nan")) == -1
    assert call(T=float("inf")) == -1
    assert call(top_p=0.0) == -1 and call(top_p=1.5) == -1
    assert call(M=0) == -1 and call(M=1025) == -1
    assert call(nws=2 * 1 * 32 * 8 - 8) == -1
    assert call(ws=0) == -1
    bad = list(P)
    bad[2] = 0                                        # draft_idx NULL, kd > 0
    assert call(ptrs=bad) == -1
    bad = list(P)
    bad[0] = P[0] + 2                                 # logits misaligned
    assert call(ptrs=bad) == -2
    assert call(ws=WS + 4) == -2


def test_gdn_commit_argument_errors(lib):
    """Sizes, NULL pointers and alignment are rejected before device work."""
    n = ctypes.c_int(0)
    assert lib.q4_gdn_commit_lds_bytes(16, ctypes.byref(n)) == 0
    assert n.value == 16 * (48 * 16 + 8)
    assert lib.q4_gdn_commit_lds_bytes(0, ctypes.byref(n)) == -1
    assert lib.q4_gdn_commit_lds_bytes(33, ctypes.byref(n)) == -1
    f = lib.q4_gdn_commit
    P = [0x10000 + 0x1000 * i for i in range(7)]    # fake device pointers

    def call(L=48, H=48, Hk=16, dv=128, dk=128, M=16, ptrs=P, status=None):
        return f(ptrs[0], L, H, Hk, dv, dk, M, *ptrs[1:], status, None)
    assert call(M=0) == -1 and call(M=33) == -1
    assert call(dk=64) == -1 and call(dv=32) == -1 and call(dv=96) == -1
    assert call(Hk=5) == -1 and call(Hk=0) == -1 and call(H=0) == -1
    assert call(L=0) == -1
    assert call(L=1 << 20, H=1 << 12, Hk=1) == -1    # grid beyond 2^31
    for i in range(7):
        bad = list(P)
        bad[i] = 0
        assert call(ptrs=bad) == -1, i
    for i, off in ((0, 8), (1, 4), (2, 8), (3, 2), (6, 1)):
        bad = list(P)
        bad[i] += off
        assert call(ptrs=bad) == -2, i
    assert call(status=0x90002) == -2


def test_gdn_tree_out_argument_errors(lib):
    """Sizes, NULL pointers and alignment are rejected before device work."""
    f = lib.q4_gdn_tree_out
    # S, q, k, v, alpha, beta, parent, out (fake device pointers)
    P = [0x10000 + 0x1000 * i for i in range(8)]

    def call(H=48, Hk=16, dv=128, dk=128, M=16, ptrs=P, status=None):
        return f(ptrs[0], H, Hk, dv, dk, M, *ptrs[1:], status, None)
    assert call(M=0) == -1 and call(M=33) == -1
    assert call(dk=64) == -1 and call(dv=16) == -1 and call(dv=48) == -1
    assert call(Hk=5) == -1 and call(Hk=0) == -1 and call(H=0) == -1
    for i in range(8):
        bad = list(P)
        bad[i] = 0
        assert call(ptrs=bad) == -1, i
    # S, q, k and out 16-byte aligned; v, alpha, beta, parent 4-byte
    for i, off in ((0, 8), (1, 4), (2, 8), (3, 2), (4, 1), (5, 2), (6, 1),
                   (7, 8)):
        bad = list(P)
        bad[i] += off
        assert call(ptrs=bad) == -2, i
    assert call(status=0x90002) == -2


def test_dequant_and_probe_argument_errors(lib):
    d = lib.q4_dequant
    assert d(0x10000, 0x20000, 0, 64, None) == -1
    assert d(0x10000, 0x20000, 4, 100, None) == -1
    assert d(None, 0x20000, 4, 64, None) == -1
    assert d(0x10008, 0x20000, 4, 64, None) == -2
    assert d(0x10000, 0x20004, 4, 64, None) == -2
    r = lib.q4_stream_read
    assert r(0x10000, 0, 0x20000, None) == -1
    assert r(0x10000, 24, 0x20000, None) == -1
    assert r(None, 64, 0x20000, None) == -1
    assert r(0x10004, 64, 0x20000, None) == -2
    c = lib.q4_stream_copy
    assert c(0x10000, 0x20000, 8, None) == -1
    assert c(0x10000, 0x20008, 64, None) == -2


def test_binding_rejects_host_tensors(lib):
    x = torch.zeros((1, 64), dtype=torch.bfloat16)
    W = torch.zeros(36, dtype=torch.uint8)
    y = torch.zeros((1, 1), dtype=torch.float32)
    with pytest.raises(ValueError):
        q4.q4_gemm_verify(x, W, y, 1, 1, 64)


def test_dot_variant_argument_errors(lib):
    """q4_gemm_verify_tiled_dot: M up to 4 and one part of K (K <= 6144),
    the tiled shape rules; all checked before any device work."""
    g = lib.q4_gemm_verify_tiled_dot
    X, W, Y = 0x10000, 0x20000, 0x30000
    assert g(X, W, Y, 0, 5120, 5120, None) == -1
    assert g(X, W, Y, 5, 5120, 5120, None) == -1
    assert g(X, W, Y, 1, 5120, 17408, None) == -1   # K beyond 24 records
    assert g(X, W, Y, 1, 5121, 5120, None) == -1    # N % 16
    assert g(X + 8, W, Y, 1, 5120, 5120, None) == -2
    assert g(X, W, Y, 4, 34816, 5120, None) == -4   # valid: stops at device


def test_attention_split_plan(lib):
    """The default split of q4_tree_attn_plan (256 CUs without a device):
    runs of about 8 pages, at least 16 runs as the pages allow, at most one
    per CU for each KV head, and never more than 1024 pages a run; the
    workspace holds each run's partial outputs and (max, sum) pairs."""
    M, Hq, Hkv = 16, 24, 4
    cases = {32: 2, 2048: 16, 4096: 16, 8192: 32, 16384: 64, 32768: 64,
             262144: 64, 1 << 20: 64}
    for ctx, want in cases.items():
        s, ws = q4.q4_tree_attn_plan(M, Hq, Hkv, ctx)
        pages = -(-(ctx + M) // 32)
        assert s == min(want, pages), (ctx, s)
        assert -(-pages // s) <= 1024
        assert ws == (0 if s == 1 else s * Hq * M * (256 + 2) * 4)
    # runs longer than 1024 pages are split further (131073 pages)
    assert q4.q4_tree_attn_plan(M, Hq, Hkv, 4 << 20)[0] == 129
    assert q4.q4_tree_attn_plan(M, 12, 2, 4 << 20)[0] == 129
    # fewer KV heads: up to one run per CU each
    assert q4.q4_tree_attn_plan(M, 12, 2, 32768)[0] == 128
    # an explicit split is taken as asked, capped at the pages
    assert q4.q4_tree_attn_plan(M, Hq, Hkv, 4096, splits=7)[0] == 7
    assert q4.q4_tree_attn_plan(M, Hq, Hkv, 100, splits=50)[0] == 4
