"""CPU model of the verify kernel's launch and memory accesses (no GPU).

The GPU kernel's indexing is restated here in numpy from its comment block
(lane l: j = l % 16, kb = l / 16; wave w: tile nt = w % row_tiles, split
ks = w / row_tiles; rows n0 + j with n0 = 16 * (block * row_tiles + nt);
groups [G*ks/k_splits, G*(ks+1)/k_splits)) and evaluated for every thread of
the launch plan the library reports.  It checks, before any GPU run, that
every load is inside its buffer and aligned for its width, that every code
byte is read exactly once, and that every output is written exactly once.
"""
from __future__ import annotations

import numpy as np
import pytest

import speculative_verify_gemm_q4_amd as q4

SHAPES = [(1, 1, 64), (3, 17, 192), (16, 257, 640), (5, 1000, 1088),
          (16, 33, 4096), (7, 16, 65536), (2, 48000, 512), (16, 48001, 512),
          (1, 70000, 256), (13, 70001, 256), (16, 4099, 5120),
          (1, 256, 512), (16, 256, 512), (16, 5120, 17408), (1, 5120, 6144),
          (16, 14336, 5120), (16, 16640, 5120), (1, 34816, 5120),
          (16, 34816, 5120)]


def model(M, N, K):
    p = q4.q4_gemm_verify_plan(M, N, K)
    ntw, ksw, grid, block = p["row_tiles"], p["k_splits"], p["grid"], p["block"]
    assert block == 64 * ntw * ksw and block <= 1024
    assert ntw * ksw in (4, 8, 16)
    assert grid * ntw * 16 >= N > (grid - 1) * ntw * 16
    G = K // 64
    NK = N * K
    code_bytes, scale_off, bias_off = NK // 2, NK // 2, NK // 2 + NK // 32
    total = NK * 9 // 16
    # LDS of the split-K reduction: f32x4 [k_splits][row_tiles][64]
    assert (ksw * ntw * 64 * 16 if ksw > 1 else 0) <= 65536

    bx = np.arange(grid)[:, None, None, None]
    nt = np.arange(ntw)[None, :, None, None]
    j = np.arange(16)[None, None, :, None]
    kb = np.arange(4)[None, None, None, :]
    n = (bx * ntw + nt) * 16 + j                       # [grid, ntw, 16, 1]
    n = np.broadcast_to(n, (grid, ntw, 16, 4))
    kb = np.broadcast_to(kb, n.shape)
    row_ok = n < N

    bounds = [(G * ks // ksw, G * (ks + 1) // ksw) for ks in range(ksw)]
    # the splits partition the groups
    assert bounds[0][0] == 0 and bounds[-1][1] == G
    assert all(bounds[i][1] == bounds[i + 1][0] for i in range(ksw - 1))
    return p, n, kb, row_ok, bounds, (code_bytes, scale_off, bias_off, total)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_plan_accesses_in_bounds_and_exact(M, N, K):
    p, n, kb, row_ok, bounds, (cb, so, bo, total) = model(M, N, K)
    G = K // 64
    nv, kbv = n[row_ok], kb[row_ok]
    # every row < N appears exactly once per kb lane
    counts = np.bincount(nv, minlength=N)
    assert counts.shape[0] == N and np.all(counts == 4)
    for gb, ge in bounds:
        if gb == ge:
            continue
        for g in (gb, ge - 1):
            start = nv.astype(np.int64) * (K // 2) + kbv * 8 + 32 * g
            assert start.min() >= 0 and (start + 8).max() <= cb
            assert np.all(start % 8 == 0)
            sidx = nv.astype(np.int64) * G + g
            assert (so + 2 * sidx).min() >= so and (so + 2 * sidx + 2).max() <= bo
            assert (bo + 2 * sidx + 2).max() <= total
    # each 8-byte code chunk read exactly once (small shapes: explicit count)
    if N * K // 16 <= 4_000_000:
        hits = np.zeros(N * K // 16, dtype=np.int32)
        for gb, ge in bounds:
            for g in range(gb, ge):
                chunk = nv.astype(np.int64) * (K // 16) + kbv + 4 * g
                np.add.at(hits, chunk, 1)
        assert np.all(hits == 1)
    # activation loads: lanes j < M read 16 elements at j*K + 16kb + 64g
    jv = np.arange(16)[:, None]
    kbx = np.arange(4)[None, :]
    for gb, ge in bounds:
        if gb == ge:
            continue
        for g in (gb, ge - 1):
            e = jv * K + 16 * kbx + 64 * g
            e = e[:M]
            assert e.min() >= 0 and (e + 16).max() <= M * K
            assert np.all((2 * e) % 16 == 0)
    # outputs: lane (j, kb) writes rows 4kb..4kb+3 < M of column n, once
    out = np.zeros(M * N, dtype=np.int32)
    for r in range(4):
        m = kbv * 4 + r
        sel = m < M
        np.add.at(out, m[sel].astype(np.int64) * N + nv[sel], 1)
    assert np.all(out == 1)


def test_plan_rejects_bad_shapes():
    with pytest.raises(q4.Q4Error):
        q4.q4_gemm_verify_plan(0, 16, 64)
    with pytest.raises(q4.Q4Error):
        q4.q4_gemm_verify_plan(17, 16, 64)
    with pytest.raises(q4.Q4Error):
        q4.q4_gemm_verify_plan(1, 16, 96)
