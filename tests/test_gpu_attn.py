"""GPU parity of tree-verify attention against the CPU oracle.

Tolerance, from the arithmetic (tests/helpers.py, ATTN_REL): the scores are
exact bf16 x int8 products summed in fp32, the softmax runs in fp32 with the
hardware exp2, and each probability times its value scale (over a power of
two) enters the value product rounded to fp16 against exact fp16 values.
Every output element is checked against |o_gpu - o| <= (2^-11 + 2^-12 +
2^-14) * sum_p w_p |v_p| + 1e-7, with sum_p w_p |v_p| returned by the oracle
for that element.  At the benchmarked 32K context that bound rejects an
output that lost the values of 1/256 of the pages
(tests/test_attn_bound.py).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from oracle import attn as ao
from tests.helpers import attn_bound

pytestmark = pytest.mark.gpu

SCALE = 1.0 / 16.0


@pytest.fixture(scope="module")
def q4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemm_q4_amd as lib
    lib.load()
    return lib


def _say(*a):
    print(*a, flush=True)


def _host(inp):
    """Host copies of the inputs, the bf16 queries as their bit patterns."""
    h = {k: (v.cpu().numpy() if hasattr(v, "cpu") else v)
         for k, v in inp.items() if k != "q"}
    h["q"] = inp["q"].view(torch.int16).cpu().numpy().view(np.uint16)
    return h


def _oracle_head(h, g, G):
    """Oracle outputs and sums of w|v| of the query heads of KV head g."""
    anc = h["anc"].view(np.uint32)
    return ao.attention(h["q"][:, g * G:(g + 1) * G],
                        h["k_pages"][:, g:g + 1], h["v_pages"][:, g:g + 1],
                        h["k_scale"][:, g:g + 1], h["v_scale"][:, g:g + 1],
                        h["page_table"], h["ctx_len"], anc, SCALE,
                        with_abs=True)


def _oracle(h):
    """(outputs, sums of w|v|) of every head; the KV heads run on threads
    (the oracle call releases the interpreter lock)."""
    Hq, Hkv = h["q"].shape[1], h["k_pages"].shape[1]
    G = Hq // Hkv
    with ThreadPoolExecutor(max_workers=min(Hkv, 8)) as ex:
        parts = list(ex.map(lambda g: _oracle_head(h, g, G), range(Hkv)))
    return (np.concatenate([p[0] for p in parts], axis=1),
            np.concatenate([p[1] for p in parts], axis=1))


def _check(got, want, absw, what):
    """Every element within the bound; report the worst ratio."""
    assert np.isfinite(got).all(), what
    ratio = np.abs(got - want) / attn_bound(absw)
    worst = float(ratio.max())
    _say(f"  {what}: max |err|/bound = {worst:.3f}")
    assert worst <= 1.0, (what, worst, np.unravel_index(ratio.argmax(), ratio.shape))


def _run(q4, inp, splits=0, status=None):
    out = q4.tree_attn(inp["q"], inp["k_pages"], inp["v_pages"],
                       inp["k_scale"], inp["v_scale"], inp["page_table"],
                       inp["ctx_len"], inp["anc"], SCALE, splits=splits,
                       status=status)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("M,Hq,Hkv,ctx,splits", [
    (7, 6, 1, 100, 0), (7, 6, 1, 100, 1), (7, 6, 1, 100, 3),
    (16, 12, 2, 0, 0), (1, 6, 1, 0, 0), (16, 24, 4, 31, 0), (16, 24, 4, 32, 2),
    (5, 8, 4, 257, 0), (9, 16, 4, 1000, 5), (16, 16, 2, 64, 0),
    (3, 32, 4, 500, 0),
    # each workgroup width the launch picks (256 CUs): 3 of 6 heads (two
    # head groups), 4 of 8, all 8, 4 of 4 and 2 of 2 (one group)
    (16, 24, 4, 2100, 24), (16, 32, 4, 2100, 24), (16, 32, 4, 2100, 64),
    (16, 16, 4, 2100, 64), (16, 8, 4, 2100, 64),
])
def test_attention_matches_oracle(q4, M, Hq, Hkv, ctx, splits):
    dev = torch.device("cuda")
    _say(f"case tree attn M={M} Hq={Hq} Hkv={Hkv} ctx={ctx} splits={splits}")
    inp = synth.attn_inputs(M, Hq, Hkv, ctx, seed=M + ctx, device=dev)
    got = _run(q4, inp, splits)
    want, absw = _oracle(_host(inp))
    _check(got, want, absw, "all heads")


@pytest.mark.parametrize("ctx", [4096, 32768])
def test_full_shape(q4, ctx):
    """24 query heads over 4 KV heads, 16 nodes, the contexts the bench
    times, in the launch it times: every output element of every head
    against the oracle."""
    dev = torch.device("cuda")
    _say(f"case tree attn full 16 x 24/4 x 256, ctx {ctx}")
    inp = synth.attn_inputs(16, 24, 4, ctx, seed=40, device=dev)
    got = _run(q4, inp)
    want, absw = _oracle(_host(inp))
    _check(got, want, absw, f"ctx {ctx}")


def test_splits_match_oracle(q4):
    """Every split count, one run per workgroup up to many, against the
    oracle under the same bound."""
    dev = torch.device("cuda")
    inp = synth.attn_inputs(16, 24, 4, 3000, seed=41, device=dev)
    want, absw = _oracle(_host(inp))
    for s in (1, 2, 7, 0, 94):
        _say(f"case tree attn ctx 3000 splits={s}")
        _check(_run(q4, inp, s), want, absw, f"splits {s}")


def test_longest_run(q4):
    """Runs of exactly 1024 pages, the most the kernel stages (its page ids
    fill its LDS list): 65520 context tokens and 16 nodes make 2048 pages,
    taken in two runs; every output against the oracle. One run of 2048
    pages is refused."""
    dev = torch.device("cuda")
    ctx = 65520
    _say(f"case tree attn longest run, ctx {ctx}, splits 2")
    inp = synth.attn_inputs(16, 24, 4, ctx, seed=43, device=dev)
    assert q4.q4_tree_attn_plan(16, 24, 4, ctx, splits=2)[0] == 2
    with pytest.raises(q4.Q4Error):
        q4.q4_tree_attn_plan(16, 24, 4, ctx, splits=1)
    want, absw = _oracle(_host(inp))
    _check(_run(q4, inp, 2), want, absw, "runs of 1024 pages")


def test_deterministic(q4):
    dev = torch.device("cuda")
    inp = synth.attn_inputs(16, 24, 4, 2000, seed=42, device=dev)
    a, b = _run(q4, inp), _run(q4, inp)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_mask_hides_other_branches(q4):
    """Overwriting a non-ancestor's cache entry leaves a node's output bit
    for bit as it was."""
    dev = torch.device("cuda")
    inp = synth.attn_inputs(8, 6, 1, 40, seed=43, device=dev)
    parent = inp["parent"]
    a = _run(q4, inp)
    anc = inp["anc"].cpu().numpy().view(np.uint32)
    j = 7                                     # the last node
    pos = 40 + j
    pp = int(inp["page_table"][pos // 32])
    inp["k_pages"][pp, :, pos % 32, :] = 127
    inp["v_pages"][pp, :, :, pos % 32] = -127
    b = _run(q4, inp)
    for i in range(8):
        sees = bool((anc[i] >> j) & 1)
        if sees:
            assert not np.array_equal(a[i], b[i]), i
        else:
            assert np.array_equal(a[i], b[i]), (i, list(parent))


def test_bad_page_id_is_reported(q4):
    dev = torch.device("cuda")
    inp = synth.attn_inputs(4, 6, 1, 60, seed=44, device=dev)
    inp["page_table"][1] = 999
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out = _run(q4, inp, status=status)
    assert int(status.item()) == -1
    assert out.shape == (4, 6, 256)
