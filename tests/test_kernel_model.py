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
    p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_PLANAR)
    if p["kernel"] == q4.KERNEL_TILED_KSLICE:
        return p, None, None, None, None, None
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
    p, n, kb, row_ok, bounds, sizes = model(M, N, K)
    if n is None:
        return kslice_model(M, N, K, p)
    cb, so, bo, total = sizes
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
    with pytest.raises(q4.Q4Error):
        q4.q4_gemm_verify_plan(1, 24, 256, q4.LAYOUT_TILED16)
    with pytest.raises(q4.Q4Error):
        q4.q4_gemm_verify_plan(1, 16, 64, 7)


# --------------------------------------------------------------------------
# tiled layout: wave (nt, ks) of block b takes tile set b*NTW + nt, i.e. tiles
# set*TNT + t, and records [Q*ks/KSW, Q*(ks+1)/KSW) of each; its buffer
# resources cover exactly those records (tiles past N get an empty range).
# Lane l reads units l, 64 + l and 128 + j of a record (16-byte units), and
# activation elements j*K + 16*kb + 256*q + 64*gi + 0..15 (j < M, else the
# load falls past the M*K*2-byte activation range and reads nothing).

TILED_SHAPES = [(16, 16, 256), (16, 256, 512), (5, 1600, 1024),
                (5, 1600, 2048), (16, 5120, 6144), (3, 5120, 17408),
                (16, 80000, 1024), (16, 34816, 5120), (1, 248320, 5120),
                (16, 14336, 5120), (16, 16640, 5120), (16, 1040, 256)]


@pytest.mark.parametrize("M,N,K", TILED_SHAPES)
def test_tiled_plan_reads_every_record_once(M, N, K):
    p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
    if p["kernel"] == q4.KERNEL_TILED_KSLICE:
        return kslice_model(M, N, K, p)
    if p["kernel"] == q4.KERNEL_TILED_RESIDENT:
        return resident_model(M, N, K, p)
    assert p["kernel"] == q4.KERNEL_TILED_STREAM and K > 6144
    tnt, ksw, grid, block = (p["tiles_per_wave"], p["k_splits"], p["grid"],
                             p["block"])
    ntw = p["row_tiles"] // tnt
    assert block == 64 * ntw * ksw <= 1024 and ntw * ksw in (1, 2, 4, 8, 16)
    T, Q = N // 16, K // 256
    assert grid * ntw * tnt >= T > (grid - 1) * ntw * tnt
    # LDS of the split-K reduction: f32x4 [KSW][NTW][TNT][64]
    assert (ksw * ntw * tnt * 64 * 16 if ksw > 1 else 0) <= 65536
    bounds = [(Q * ks // ksw, Q * (ks + 1) // ksw) for ks in range(ksw)]
    assert bounds[0][0] == 0 and bounds[-1][1] == Q
    assert all(bounds[i][1] == bounds[i + 1][0] for i in range(ksw - 1))
    hits = np.zeros(T * Q, dtype=np.int32)
    total = T * Q * 2304
    for b in range(grid):
        for nt in range(ntw):
            for t in range(tnt):
                tile = (b * ntw + nt) * tnt + t
                if tile >= T:
                    continue
                for qb, qe in bounds:
                    hits[tile * Q + qb: tile * Q + qe] += 1
                    # the wave's resource range lies inside the buffer
                    assert (tile * Q + qe) * 2304 <= total
    assert np.all(hits == 1)
    # activation offsets in bytes fit the 32-bit buffer offset, and rows < M
    # stay inside the M*K*2 bytes
    j = np.arange(16)[:, None]
    kb = np.arange(4)[None, :]
    last = (j * K + 16 * kb + 256 * (Q - 1) + 64 * 3 + 8) * 2 + 16
    assert last.max() < 2 ** 32
    assert last[:M].max() <= M * K * 2
    first_out = (j[M:] * K) * 2
    assert np.all(first_out >= M * K * 2)
    # every output written once: tiles < T, rows 4kb+r < M
    out = np.zeros((M, N), dtype=np.int32)
    for tile in range(T):
        for kbv in range(4):
            for r in range(4):
                m = 4 * kbv + r
                if m < M:
                    out[m, tile * 16: tile * 16 + 16] += 1
    assert np.all(out == 1)


# --------------------------------------------------------------------------
# K-slice kernel (M <= 16, K <= 6144): workgroup b owns tiles
# [T b / G, T (b+1) / G) with G = min(T, CUs); its W = ceil(Q / 2) waves take
# records 2w and 2w + 1 of every one of those tiles (wave w's activations:
# inputs 256 q + 64 gi + 16 kb + 8 h .. +7 of row j for lane (j, kb)); the
# tiles are written in batches of NB = LDS / (W KiB), each tile once, the
# waves' partial sums added in wave order.

IN_MAX_TILES = 16   # tile running sums of the sequential parts
PLANAR_CODE_LDS = 4096  # planar: a wave's two records of one tile's codes
PLANAR_SB_LDS = 2 * 16 * 24 * 8  # planar: one tile's scales and biases
IN_MAX_TILES_PLANAR = 4


def planar_word(j, kb, h):
    """Planar K-slice: the code word of a group (and so the activations)
    that operand h of lane (j, kb) takes: 2 kb + h."""
    return 2 * kb + h


def test_planar_code_staging():
    """The planar codes' path through LDS: load i of record qq, lane l,
    brings chunk (l & 7) ^ (l >> 3) of row 8i + (l >> 3) and lands at
    qq 2048 + i 1024 + l 16; lane (j, kb) then reads 8 bytes of group g at
    qq 2048 + j 128 + ((2g + (kb >> 1)) ^ (j & 7)) 16 + (kb & 1) 8, which
    must be words 2 kb, 2 kb + 1 of group g of row j.  Every load covers
    whole 128-byte row runs (8 lanes per row).  The inputs in an MFMA
    operand slot must not depend on the lane's row: slot kb of every row
    of x meets slot kb of every row of W.  Eight consecutive lanes read 8
    distinct 16-byte bank groups."""
    lds = {}
    for qq in range(2):
        for i in range(2):
            rows = {}
            for lane in range(64):
                r, c = 8 * i + (lane >> 3), (lane & 7) ^ (lane >> 3)
                rows.setdefault(r, set()).add(c)
                for b in range(16):
                    addr = qq * 2048 + i * 1024 + lane * 16 + b
                    assert addr not in lds and addr < PLANAR_CODE_LDS
                    lds[addr] = (qq, r, 16 * c + b)  # byte of the row's record
            assert len(rows) == 8 and all(v == set(range(8)) for v in rows.values())
    assert len(lds) == PLANAR_CODE_LDS
    for qq in range(2):
        for g in range(4):
            slots = []
            for lane in range(64):
                j, kb = lane & 15, lane >> 4
                base = qq * 2048 + j * 128 + (((2 * g + (kb >> 1)) ^ (j & 7)) * 16) + (kb & 1) * 8
                got = [lds[base + b] for b in range(8)]
                want = [(qq, j, 32 * g + 4 * planar_word(j, kb, 0) + b) for b in range(8)]
                assert got == want, (qq, g, lane)
                assert planar_word(j, kb, 1) == planar_word(j, kb, 0) + 1
                slots.append((base % 128) // 8)
            for s8 in range(8):
                assert len({x // 2 for x in slots[8 * s8: 8 * s8 + 8]}) == 8
    # the slots' words over kb are a permutation of the group's 8 words,
    # the same for every row
    for j in range(16):
        assert sorted(planar_word(j, kb, h) for kb in range(4) for h in range(2)) == list(range(8))
        assert all(planar_word(j, kb, h) == planar_word(0, kb, h)
                   for kb in range(4) for h in range(2))


def kslice_model(M, N, K, p):
    """Work split of the K-slice kernel for plan p: workgroup b has rank
    (b % 8) G/8 + b/8 (XCD after XCD), takes part group pk = rank // Gt of
    K and tile group rank % Gt; the part group holds parts pk Pin .. +Pin-1
    (Pin = k_seq_parts, taken one after another with tile running sums in
    LDS), part pp = records [Q pp / Ptot, Q (pp+1) / Ptot) with
    Ptot = P Pin; wave w takes the part's records R w .. R w + R - 1
    (R = 2, or R = 1 with two row tiles at M = 17..32: the activation
    operand units u = 0, 1 are then rows 16 u .. 16 u + 15 of one record)."""
    planar = p["layout_id"] == q4.LAYOUT_PLANAR
    T, Q = -(-N // 16), K // 256
    P, Pin = p["k_parts"], p["k_seq_parts"]
    Ptot = P * Pin
    W = p["block"] // 64
    Qp = -(-Q // Ptot)
    RT = p["m_tiles"]
    R = 1 if RT == 2 else 2
    assert RT == (2 if M > 16 else 1) and M <= 32
    assert Qp <= (12 if RT == 2 else 24) and W == -(-Qp // R)
    assert planar or N % 16 == 0
    assert not (planar and RT == 2)
    G = p["grid"]
    g0 = min(T, 256 // P)
    per = -(-T // g0)
    Gt = -(-T // per) if per >= 3 else g0
    assert G == Gt * P and p["row_tiles"] == per
    if planar:
        # codes per wave, two tiles' scales and biases, running sums of at
        # most IN_MAX_TILES_PLANAR tiles
        tacc = IN_MAX_TILES_PLANAR * 1024 if Pin > 1 else 0
        fixed = W * PLANAR_CODE_LDS + 2 * PLANAR_SB_LDS + tacc
        NB = (LDS_BYTES - fixed) // (W * 1024)
    elif RT == 2:
        # two row tiles: 2 KiB of partial sums per wave and tile
        tacc = IN_MAX_TILES * 2048 if Pin > 1 else 0
        fixed = tacc
        NB = (LDS_BYTES - 1024 - tacc) // (W * 2048)
    else:
        tacc = IN_MAX_TILES * 1024 if Pin > 1 else 0
        fixed = tacc
        NB = (LDS_BYTES - IN_MAX_TILES * 1024) // (W * 1024)
    assert NB * RT >= 8  # the activation staging areas alias the partial sums
    # the plan sizes the area for the tiled kernel's 8 row pairs (M > 4)
    part_tiles = max(NB, 16) if kslice_dma_x(W, planar, RT, Pin > 1, 8, NB) else NB
    assert p["lds_bytes"] == part_tiles * W * 1024 * RT + fixed <= LDS_BYTES
    assert p["workspace_bytes"] == (P - 1) * M * N * 4
    hits = np.zeros((T, Q), dtype=np.int32)
    writes = np.zeros((P, T), dtype=np.int32)
    ranks = [(b & 7) * (G >> 3) + min(b & 7, G & 7) + (b >> 3)
             for b in range(G)]
    assert sorted(ranks) == list(range(G))
    # the packed arguments (M | P << 8 | Pin << 20, per, Gt | rem << 16)
    # and the kernel's division-free index arithmetic
    assert M < 256 and P < 4096 and Pin < 4096 and Gt < 4096
    per_k, rem_k = T // Gt, T % Gt
    assert per_k * Gt + rem_k == T
    for b in range(G):
        r = ranks[b]
        pk = 0 if P == 1 else small_div_model(r, Gt)
        g = r - pk * Gt
        assert (pk, g) == divmod(r, Gt)
        assert g * per_k + small_div_model(g * rem_k, Gt) == T * g // Gt
        assert (g + 1) * per_k + small_div_model((g + 1) * rem_k, Gt) == T * (g + 1) // Gt
    qd = Q if Ptot == 1 else small_div_model(Q, Ptot)
    qr = Q - qd * Ptot
    assert (qd, qr) == divmod(Q, Ptot)
    for pp in range(Ptot):
        qa = Q * pp // Ptot
        nrec = Q * (pp + 1) // Ptot - qa
        assert 1 <= nrec <= R * W
        if Ptot > 1:
            assert qd * pp + small_div_model(qr * pp, Ptot) == qa
            assert qd * (pp + 1) + small_div_model(qr * (pp + 1), Ptot) - qa == nrec
        LR = row_pairs(M, RT, Pin > 1)
        if LR:
            kslice_row_staging_model(M, K, W, p["lds_bytes"] - tacc, qa, nrec,
                                     planar, RT,
                                     kslice_dma_x(W, planar, RT, Pin > 1, LR, NB))
        else:
            direct_operand_loads(M, K, W, qa, nrec, planar, RT)
    G8 = K // 64
    for b in range(G):
        r = ranks[b]
        pk, g = r // Gt, r % Gt
        t0, t1 = T * g // Gt, T * (g + 1) // Gt
        assert t1 > t0
        assert Pin == 1 or t1 - t0 <= (IN_MAX_TILES_PLANAR if planar else IN_MAX_TILES)
        assert t1 - t0 <= per
        rows = min(N - 16 * t0, 16 * (t1 - t0))
        span = rows * (K // 2) if planar else (t1 - t0) * Q * 2304
        assert span < 0x7FFFFFF0
        stored = set()  # tiles whose running sum holds parts so far
        for ip in range(Pin):
            pp = pk * Pin + ip
            qa = Q * pp // Ptot
            nrec = Q * (pp + 1) // Ptot - qa
            for w in range(W):
                nq = min(max(nrec - R * w, 0), R)
                q0 = qa + R * w
                for tl in range(t1 - t0):
                    for qq in range(nq):
                        if planar:
                            # rows j of the tile, 16 B at kb*16 and 64 + kb*16
                            # of the record's 128 B
                            for j in range(16):
                                o = (tl * 16 + j) * (K // 2) + (q0 + qq) * 128
                                if 16 * (t0 + tl) + j < N:
                                    assert o + 128 <= span
                                else:
                                    assert o >= span
                        else:
                            off = (tl * Q + q0 + qq) * 2304
                            assert off + 2304 <= span
                        hits[t0 + tl, q0 + qq] += 1

            if planar:
                planar_scale_loads(N, K, W, t0, t1, rows, qa, nrec)
            # batches: a flush after every NB tiles and after the last; the
            # sequential parts before the last keep running sums
            tb = t0
            for t in range(t0, t1):
                assert (t - tb) < NB
                if t - tb == NB - 1 or t == t1 - 1:
                    for tt in range(tb, t + 1):
                        if ip > 0:
                            assert tt in stored
                        if ip + 1 < Pin:
                            assert tt - t0 < IN_MAX_TILES
                            stored.add(tt)
                        else:
                            writes[pk, tt] += 1
                    tb = t + 1
    assert np.all(hits == 1)
    assert np.all(writes == 1)


def planar_scale_loads(N, K, W, t0, t1, rows, qa, nrec):
    """Planar scales and biases of one part for each tile: load k of array
    a (dealt to wave (a nk + k) mod W) lane l brings chunk f = 64k + l < 16
    cpr (row f // cpr, chunk f % cpr of the part's run) to LDS
    a 256 cpr + f 16.  Every chunk a wave with records reads (row j, chunk
    = wave) is loaded once, from the right bytes, inside the resource (one
    range over the scales and then the biases) or past it."""
    G8 = K // 64
    NK32 = N * K // 32
    cpr = (nrec + 1) // 2
    nk = -(-16 * cpr // 64)
    rng = NK32 + rows * G8 * 2  # the resource's range from the scales of t0
    assert rng < 0x7FFFFFF0
    for tl in range(t1 - t0):
        lds = {}
        for ins in range(2 * nk):
            a, k = ins >= nk, ins - (ins >= nk) * nk
            for lane in range(64):
                f = 64 * k + lane
                if f >= 16 * cpr:
                    continue
                r, c = f // cpr, f % cpr
                o = a * NK32 + ((tl * 16 + r) * G8 + 4 * qa) * 2 + 16 * c
                addr = a * 256 * cpr + f * 16
                assert addr + 16 <= PLANAR_SB_LDS and addr not in lds
                lds[addr] = (a, r, c, o)
                row = 16 * (t0 + tl) + r
                if row < N:
                    # a real row's run lies inside the range
                    assert o + 8 * min(2, nrec - 2 * c) <= rng
                elif a == 1:
                    # biases of a row past N: past the range (zeros); a
                    # scale row past N reads biases (finite) or zeros
                    assert o >= rng
        for w in range(W):
            if min(max(nrec - 2 * w, 0), 2) == 0:
                continue
            for j in range(16):
                for a in range(2):
                    got = lds[(a * 16 + j) * cpr * 16 + w * 16]
                    # scales of groups 4 (qa + 2w) .. +7 of row j
                    want_o = a * NK32 + ((tl * 16 + j) * G8 + 4 * (qa + 2 * w)) * 2
                    assert got == (a, j, w, want_o)


def row_pairs(M, RT, seq=False):
    """Activation row pairs a wave loads per record (or row tile); 0 for
    direct operand-layout loads (parts of K in turn at M <= 4)."""
    if RT == 2 or M > 4:
        return 8
    if seq:
        return 0
    return 2 if M > 2 else 1


def direct_operand_loads(M, K, W, qa, nrec, planar=False, RT=1):
    """Direct loads: lane (j, kb), operand (gi, h) of wave w reads inputs
    64 gi + 8 word .. +7 of row j of its record, inside the M x K
    activations for a real row of a real record, past them otherwise."""
    x_bytes = M * K * 2
    R = 1 if RT == 2 else 2
    for w in range(W):
        nq = min(max(nrec - R * w, 0), R)
        for lane in range(64):
            j, kb = lane & 15, lane >> 4
            for u in range(2):
                qu, ru = (u, 0) if RT == 1 else (0, u)
                row = 16 * ru + j
                for gi in range(4):
                    for h in range(2):
                        wd = planar_word(j, kb, h) if planar else 2 * kb + h
                        k = 256 * (qa + R * w + qu) + 64 * gi + 8 * wd
                        off = (row * K + k) * 2
                        if qu < nq and row < M:
                            assert k + 8 <= K and off + 16 <= x_bytes
                        elif qu < nq:
                            assert off >= x_bytes
                        else:
                            assert x_bytes <= off + 0x7FFFFFF0 < 2 ** 32


def small_div_model(a, d):
    """The kernel's floor(a / d) for 0 <= a < 2^24, 1 <= d < 2^24: the fp32
    product of a with the reciprocal of d, truncated, then one correction
    step on the remainder.  The reciprocal instruction is accurate to one
    ulp, so the product is tried with the correctly rounded reciprocal and
    its neighbours one ulp either side."""
    assert 0 <= a < 2 ** 24 and 1 <= d < 2 ** 24
    r0 = np.float32(1.0) / np.float32(d)
    out = set()
    for rc in (np.nextafter(r0, np.float32(0)), r0, np.nextafter(r0, np.float32(1))):
        q = int(np.float32(a) * np.float32(rc))
        rm = a - q * d
        q += int(rm >= d) - int(rm < 0)
        out.add(q)
    assert len(out) == 1, (a, d, out)
    return out.pop()


def kslice_dma_x(W, planar, RT, seq, LR, NB):
    """Whether the activation rows go from memory straight to LDS: both
    units of a wave at once, LR KB each (one part of K, one row tile), when
    the partial-sum area of NB tiles holds them or, tiled with at most 10
    waves, grows to."""
    return (RT == 1 and not seq and LR > 0 and
            (2 * LR <= NB or (not planar and W <= 10)))


def kslice_row_staging_model(M, K, W, lds_bytes, qa, nrec, planar=False,
                             RT=1, dma=False):
    """The activations arrive by row-contiguous loads (row_pairs(M, RT)
    loads of two rows per record) and pass through an 8 KB LDS area per
    wave; rows from 2 row_pairs on are zeros without a load or an LDS read.
    Every operand register must end up holding exactly the inputs of its
    operand-layout slot (row j, inputs 64 gi + 8 word .. +7 of the wave's
    record), or zeros for rows >= M; the LDS stores of one round must not
    collide, and the areas must fit.  The part's records are
    [qa, qa + nrec); unit u is record u of the wave's two (RT = 1) or rows
    16 u .. of its one record (RT = 2).  With dma the loads write LDS
    themselves: lane l of load i of unit u lands at the wave's area + 8 KB u
    + 1 KB i + 16 l, so it loads the chunk that belongs there,
    (l & 31) ^ (r & 7), and the area is 16 KB per wave."""
    x_bytes = M * K * 2
    R = 1 if RT == 2 else 2
    LR = row_pairs(M, RT)
    assert 2 * LR >= min(M, 16)
    span = 2048 * LR if dma else 8192
    assert W * span <= lds_bytes
    for w in range(W):
        nq = min(max(nrec - R * w, 0), R)
        for u in range(2):
            qq, ru = (u, 0) if RT == 1 else (0, u)
            base = w * span + (1024 * LR * u if dma else 0)
            # what lane l of load i holds: (row, input) or None (zeros)
            area = {}
            for i in range(LR):
                for lane in range(64):
                    r = 2 * i + (lane >> 5)
                    c = (lane & 31) ^ (r & 7) if dma else lane & 31
                    row = 16 * ru + r
                    k = 256 * (qa + R * w + qq) + 8 * c
                    off = (row * K + k) * 2
                    if qq < nq and row < M:
                        assert off + 16 <= x_bytes and k + 8 <= K
                        val = (row, k)
                    else:
                        assert off + (0 if qq < nq else 0x7FFFFFF0) >= x_bytes
                        val = None
                    addr = (base + 1024 * i + 16 * lane if dma
                            else base + r * 512 + (c ^ (r & 7)) * 16)
                    assert addr == base + r * 512 + (c ^ (r & 7)) * 16
                    assert addr not in area
                    area[addr] = val
            assert len(area) == 64 * LR
            for lane in range(64):
                j, kb = lane & 15, lane >> 4
                for gi in range(4):
                    for h in range(2):
                        wd = planar_word(j, kb, h) if planar else 2 * kb + h
                        c = (8 * gi + wd) ^ (j & 7)
                        got = area[base + j * 512 + c * 16] if j < 2 * LR else None
                        k = 256 * (qa + R * w + qq) + 64 * gi + 8 * wd
                        row = 16 * ru + j
                        want = (row, k) if (qq < nq and row < M) else None
                        assert got == want, (w, u, lane, gi, h)
    # bank groups of 16 B (128 B per LDS cycle): the 8 lanes of a group of
    # stores, and of a group of operand reads, hit 8 distinct groups
    for i in range(8):
        for g in range(8):
            lanes = range(8 * g, 8 * g + 8)
            banks = {((l & 31) ^ ((2 * i + (l >> 5)) & 7)) & 7 for l in lanes}
            assert len(banks) == 8
    for gi in range(4):
        for h in range(2):
            for g in range(8):
                lanes = range(8 * g, 8 * g + 8)
                wd = [planar_word(l & 15, l >> 4, h) if planar else 2 * (l >> 4) + h
                      for l in lanes]
                banks = {((8 * gi + wd[i]) ^ ((l & 15) & 7)) & 7
                         for i, l in enumerate(lanes)}
                assert len(banks) == 8


@pytest.mark.parametrize("M,N,K", [(1, 16, 256), (16, 16, 5120),
                                   (16, 48, 256), (7, 4096, 1024),
                                   (8, 4096, 1280), (9, 512, 6144),
                                   (16, 4112, 5120), (1, 6000 * 16, 768),
                                   (16, 34816, 5120), (16, 5120, 6144),
                                   (3, 16, 5888), (16, 248320, 5120)])
def test_kslice_plan_shapes(M, N, K):
    p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
    assert p["kernel"] == q4.KERNEL_TILED_KSLICE
    kslice_model(M, N, K, p)
    assert q4.q4_gemm_verify_tiled_ws_plan(M, N, K) == p


@pytest.mark.parametrize("layout", [q4.LAYOUT_PLANAR, q4.LAYOUT_TILED16])
@pytest.mark.parametrize("M,N,K", [(16, 5120, 17408), (3, 5120, 17408),
                                   (1, 16, 65536), (9, 4096, 6400),
                                   (16, 1024, 12288), (2, 48, 24832)])
def test_kslice_sequential_parts(layout, M, N, K):
    """K beyond one part's 24 records without a workspace: each workgroup
    takes the parts one after another (every record once, every tile
    written once after its last part)."""
    p = q4.q4_gemm_verify_plan(M, N, K, layout)
    assert p["kernel"] == q4.KERNEL_TILED_KSLICE
    assert p["k_parts"] == 1 and p["k_seq_parts"] == -(-(K // 256) // 24)
    assert p["workspace_bytes"] == 0
    kslice_model(M, N, K, p)


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (5, 17, 512), (16, 100, 768),
                                   (8, 4099, 5120), (13, 70001, 256)])
def test_planar_kslice_ragged_rows(M, N, K):
    """The planar K-slice kernel on N not a multiple of 16: rows past N
    read past their resource."""
    p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_PLANAR)
    assert p["kernel"] == q4.KERNEL_TILED_KSLICE
    kslice_model(M, N, K, p)


# resident-activation kernel (K <= 5120): workgroup b owns tiles
# [T b / G, T (b+1) / G); its U = tiles * Q records (tile-major) are split
# into W contiguous ranges [U w / W, U (w+1) / W).  A tile inside one range is
# written by that wave; a split tile by the wave holding its first record,
# which adds its tail sum and then the head sums of the following waves whose
# ranges start inside the tile.  Activations: fragment f = 8q + 2gi + h at
# LDS byte 1024 f, lane l at +16 l; partial sums reuse LDS bytes [0, 2 W KB).

LDS_BYTES = 163840


def resident_model(M, N, K, p):
    """Work split of the resident-activation kernel for plan p: workgroup b
    takes part p = b // Gt of K (records [Q p / P, Q (p+1) / P)) and the
    tiles [T g / Gt, T (g+1) / Gt) of group g = b % Gt."""
    T, Q = N // 16, K // 256
    P, W, RT = p["k_parts"], p["block"] // 64, p["m_tiles"]
    assert RT == (2 if M > 16 else 1)
    G = p["grid"]
    assert G % P == 0
    Gt = G // P
    assert p["lds_bytes"] == LDS_BYTES and p["block"] <= 1024
    assert Gt == min(T, max(1, 256 // P))
    assert p["workspace_bytes"] == (P - 1) * M * N * 4
    assert 2 * W * RT * 1024 <= LDS_BYTES
    hits = np.zeros((T, Q), dtype=np.int32)
    writes = np.zeros((P, T), dtype=np.int32)
    for b in range(G):
        part, g = b // Gt, b % Gt
        qa, qb = Q * part // P, Q * (part + 1) // P
        nq = qb - qa
        assert 0 < nq and 8 * RT * nq * 1024 <= LDS_BYTES
        t0, t1 = T * g // Gt, T * (g + 1) // Gt
        U = (t1 - t0) * nq
        rng = [(U * w // W, U * (w + 1) // W) for w in range(W)]
        owner_of = {}
        for w, (u0, u1) in enumerate(rng):
            if u1 > u0:
                # the wave's resource: whole tiles ft .. lt of its range
                ft, lt = u0 // nq, (u1 - 1) // nq
                span = (lt - ft + 1) * Q * 2304
                assert (t0 + ft) * Q * 2304 + span <= T * Q * 2304
                assert span < 0x7FFFFFF0
                for u in range(u0, u1):
                    tl, rq = u // nq, u % nq
                    off = ((tl - ft) * Q + qa + rq) * 2304
                    assert 0 <= off and off + 2304 <= span
                    hits[t0 + tl, qa + rq] += 1
            q, tl, head = u0 % nq, u0 // nq, u0 % nq != 0
            for _ in range(u1 - u0):
                q += 1
                if q == nq:
                    if not head:
                        writes[part, t0 + tl] += 1
                    head, q, tl = False, 0, tl + 1
            if u1 > u0:
                lt = (u1 - 1) // nq
                if lt * nq >= u0 and lt * nq + nq > u1:
                    owner_of[lt] = w
        for lt, w in owner_of.items():
            got = [w]
            for w2 in range(w + 1, W):
                a0, a1 = rng[w2]
                if a0 >= lt * nq + nq:
                    break
                if a1 > a0:
                    got.append(w2)
            want = [w2 for w2, (a0, a1) in enumerate(rng)
                    if a1 > a0 and a0 < lt * nq + nq and a1 > lt * nq]
            assert got == want
            u0, u1 = rng[w]
            assert u0 <= lt * nq < u1 < lt * nq + nq
            for w2 in got[1:]:
                assert lt * nq < rng[w2][0] < lt * nq + nq
            writes[part, t0 + lt] += 1
    assert np.all(hits == 1)
    assert np.all(writes == 1)


@pytest.mark.parametrize("M,N,K", [(17, 16, 256), (32, 16, 2560),
                                   (24, 48, 256), (20, 4096, 1024),
                                   (32, 4112, 2560), (17, 6000 * 16, 768),
                                   (32, 34816, 2560)])
def test_two_row_tile_plan_more_shapes(M, N, K):
    """17..32 rows run the K-slice kernel with two MFMA row tiles (one
    record per wave, at most 12 records a part)."""
    p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
    assert p["kernel"] == q4.KERNEL_TILED_KSLICE and p["m_tiles"] == 2
    kslice_model(M, N, K, p)


def test_resident_split_tile_sums_in_wave_order():
    # a workgroup of 8 waves over 3 tiles of 20 records: 60 records, 7 or 8
    # per wave, so tiles are split; check by direct simulation with exact
    # dyadic numbers that the owner's sum equals the plain sum of the tile
    W, Q, tiles = 8, 20, 3
    U = tiles * Q
    rng = [(U * w // W, U * (w + 1) // W) for w in range(W)]
    contrib = np.arange(U, dtype=np.float64) + 1.0  # record u adds u + 1
    head = np.zeros(W)
    tail = np.zeros(W)
    out = np.full(tiles, np.nan)
    for w, (u0, u1) in enumerate(rng):
        acc, q, tl, in_head = 0.0, u0 % Q, u0 // Q, u0 % Q != 0
        for u in range(u0, u1):
            acc += contrib[u]
            q += 1
            if q == Q:
                if in_head:
                    head[w] = acc
                    in_head = False
                else:
                    out[tl] = acc
                acc, q, tl = 0.0, 0, tl + 1
        if q != 0:
            if in_head:
                head[w] = acc
            else:
                tail[w] = acc
    for w, (u0, u1) in enumerate(rng):
        lt = (u1 - 1) // Q
        if lt * Q >= u0 and lt * Q + Q > u1:
            v = tail[w]
            for w2 in range(w + 1, W):
                a0, a1 = rng[w2]
                if a0 >= lt * Q + Q:
                    break
                if a1 > a0:
                    v += head[w2]
            out[lt] = v
    want = contrib.reshape(tiles, Q).sum(axis=1)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("M,K", [(1, 256), (16, 256), (5, 1280), (16, 5120),
                                 (17, 256), (32, 2560), (24, 768)])
def test_resident_lds_layout_gives_each_lane_its_operand(M, K):
    """Copy side: block f = (4q + gi) 2RT + r, slot s (lane s of the copy)
    holds inputs 256q + 64gi + 8(s%8) .. +7 of row 8r + s/8, rows >= M zero
    (RT = 2 row tiles when M > 16).  Read side: row tile rt of lane (j, kb),
    half h reads slot 8(j%8) + 2kb + h of block (4q + gi) 2RT + 2rt + j/8,
    and must get inputs 64gi + 16kb + 8h .. +7 of row 16 rt + j of record q
    (the MFMA A operand of the tiled layout)."""
    RT = 2 if M > 16 else 1
    Q = K // 256
    x = np.arange(32 * K, dtype=np.int64).reshape(32, K) + 1
    x[M:] = 0
    lds = np.zeros((8 * RT * Q, 64, 8), dtype=np.int64)
    assert lds.size * 2 <= LDS_BYTES
    for f in range(8 * RT * Q):
        q, gi, r = f // (8 * RT), (f // (2 * RT)) % 4, f % (2 * RT)
        for s in range(64):
            row = 8 * r + s // 8
            k0 = 256 * q + 64 * gi + 8 * (s % 8)
            # the copy's byte offset, as the kernel forms it
            voff = ((s >> 3) * K + 8 * (s & 7)) * 2 + 8 * r * K * 2
            soff = (256 * q + 64 * gi) * 2
            assert voff + soff == (row * K + k0) * 2
            if (voff + soff) + 16 <= M * K * 2:
                lds[f, s] = x[row, k0:k0 + 8]
    flat = lds.reshape(-1, 8)
    for q in range(Q):
        for gi in range(4):
            for rt in range(RT):
                for h in range(2):
                    for lane in range(64):
                        j, kb = lane & 15, lane >> 4
                        idx = q * 512 * RT + (j >> 3) * 64 + (j & 7) * 8 \
                            + 2 * kb + (gi * 2 * RT + 2 * rt) * 64 + h
                        k0 = 256 * q + 64 * gi + 16 * kb + 8 * h
                        assert np.array_equal(flat[idx],
                                              x[16 * rt + j, k0:k0 + 8])


@pytest.mark.parametrize("M,N,K", [(16, 5120, 17408), (1, 5120, 6144),
                                   (7, 5120, 6144), (16, 16, 5376),
                                   (16, 4096, 65536), (2, 48, 10240),
                                   (16, 5120, 6144), (3, 5120, 17408),
                                   (1, 16, 5376), (16, 48, 10240),
                                   (5, 1600, 7168), (16, 256, 65536),
                                   (9, 32, 5632), (4, 5120, 17408),
                                   (1, 16, 10496), (8, 1600, 7168)])
def test_workspace_plan_split_parts(M, N, K):
    p = q4.q4_gemm_verify_tiled_ws_plan(M, N, K)
    # up to 16 rows the K-slice kernel: one part up to 24 records, beyond
    # that P >= 4 parts (a power of two) of at most 24 records, whatever M
    Q = K // 256
    launch = lambda q: {k: v for k, v in q.items() if k != "workspace_bytes"}
    for M2 in range(1, 17):
        assert launch(q4.q4_gemm_verify_tiled_ws_plan(M2, N, K)) == launch(p)
    if Q <= 24:
        assert p == q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
        assert p["workspace_bytes"] == 0
        return
    assert p["kernel"] == q4.KERNEL_TILED_KSLICE and p["k_parts"] > 1
    P = p["k_parts"]
    assert P >= 4 and P & (P - 1) == 0 and -(-Q // P) <= 24
    assert P == 4 or -(-Q // (P // 2)) > 24
    kslice_model(M, N, K, p)



@pytest.mark.parametrize("M,N,K", [(17, 16, 256), (24, 34816, 2560),
                                   (32, 4096, 1024), (32, 256, 2816)])
def test_plain_plan_32_rows(M, N, K):
    """M > 16 without a workspace: the K-slice kernel with two row tiles,
    K beyond 12 records in parts taken one after another when a
    workgroup's tiles fit its running sums."""
    p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
    assert p["kernel"] == q4.KERNEL_TILED_KSLICE and p["m_tiles"] == 2
    assert p["k_parts"] == 1 and p["k_seq_parts"] == -(-(K // 256) // 12)
    assert p["workspace_bytes"] == 0
    kslice_model(M, N, K, p)


def test_plain_plan_32_rows_without_room():
    """32 rows, no workspace, K beyond 12 records and more than 16 tiles
    per workgroup (the LM head): no plan, before any device work."""
    with pytest.raises(q4.Q4Error):
        q4.q4_gemm_verify_plan(32, 248320, 5120, q4.LAYOUT_TILED16)


@pytest.mark.parametrize("M,N,K", [(24, 34816, 5120), (32, 5120, 17408),
                                   (32, 248320, 5120), (17, 5120, 6144),
                                   (32, 16, 5376), (25, 48, 10240)])
def test_workspace_plan_32_rows(M, N, K):
    """32 rows with a workspace: the K-slice kernel with two row tiles, K in
    P parts across workgroups (the least power of two with at most 12
    records a part)."""
    p = q4.q4_gemm_verify_tiled_ws_plan(M, N, K)
    assert p["kernel"] == q4.KERNEL_TILED_KSLICE and p["m_tiles"] == 2
    P, Q = p["k_parts"], K // 256
    assert P & (P - 1) == 0 and -(-Q // P) <= 12
    assert P == 1 or -(-Q // (P // 2)) > 12
    assert p["k_seq_parts"] == 1
    kslice_model(M, N, K, p)


def test_small_div_domain():
    """The kernel's fp32 quotient with one correction step equals floor(a/d)
    over the ranges its index arithmetic uses (d < 4096 workgroups or parts,
    a < 4096 d, and the record counts Q < 2^18 over a part count), for the
    correctly rounded reciprocal and for one ulp either side."""
    rng = np.random.default_rng(7)
    d = np.arange(1, 4096, dtype=np.int64)
    cols = [np.zeros_like(d), d - 1, d, d + 1, 4095 * d - 1, 4095 * d,
            rng.integers(0, 4096, size=d.size) * d + rng.integers(0, d),
            rng.integers(0, 4096 * d)]
    a = np.concatenate(cols)
    dd = np.tile(d, len(cols))
    q_big = rng.integers(0, 2 ** 18, size=20000)
    a = np.concatenate([a, q_big])
    dd = np.concatenate([dd, rng.integers(1, 4096, size=q_big.size)])
    keep = (a >= 0) & (a < 2 ** 24)
    a, dd = a[keep], dd[keep]
    r0 = np.float32(1.0) / dd.astype(np.float32)
    for rc in (np.nextafter(r0, np.float32(0)), r0, np.nextafter(r0, np.float32(1))):
        q = (a.astype(np.float32) * rc).astype(np.int64)
        rm = a - q * dd
        q = q + (rm >= dd) - (rm < 0)
        assert np.array_equal(q, a // dd)
