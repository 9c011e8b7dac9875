"""GPU parity of tree-verify attention against the CPU oracle.

Tolerance, from the arithmetic: the scores are exact bf16 x int8 products
summed in fp32 (relative error about 256 * 2^-24), the softmax runs in fp32
with the hardware exp2, and the probabilities times the value scales are
rounded to bf16 (relative error <= 2^-9) before the value product.  An output
is therefore within 2^-9 * sum_p w_p |v_p| <= 2^-9 * max |v| of the exact
result, plus fp32 rounding; the test allows 2^-8 * max |v| + 1e-6, max |v|
over the cache.  A wrong mask, page, head or layout gives errors of the size
of the values themselves.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import attn as ao

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


def _oracle(h, heads=None):
    """Oracle outputs; `heads` restricts to the query heads of one KV head
    (g, G) to keep the CPU time small."""
    q = h["q"]
    kp, vp, ks, vs = h["k_pages"], h["v_pages"], h["k_scale"], h["v_scale"]
    anc = h["anc"].view(np.uint32)
    if heads is not None:
        g, G = heads
        q = q[:, g * G:(g + 1) * G]
        kp, vp = kp[:, g:g + 1], vp[:, g:g + 1]
        ks, vs = ks[:, g:g + 1], vs[:, g:g + 1]
    return ao.attention(q, kp, vp, ks, vs, h["page_table"], h["ctx_len"],
                        anc, SCALE)


def _tol(h):
    vmax = float(np.abs(h["v_pages"].astype(np.float64)).max() *
                 h["v_scale"].max())
    return 2.0 ** -8 * vmax + 1e-6


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
])
def test_attention_matches_oracle(q4, M, Hq, Hkv, ctx, splits):
    dev = torch.device("cuda")
    _say(f"case tree attn M={M} Hq={Hq} Hkv={Hkv} ctx={ctx} splits={splits}")
    inp = synth.attn_inputs(M, Hq, Hkv, ctx, seed=M + ctx, device=dev)
    got = _run(q4, inp, splits)
    h = _host(inp)
    want = _oracle(h)
    err = np.abs(got - want).max()
    assert err <= _tol(h), (err, _tol(h))


def test_full_shape_sampled(q4):
    """24 query heads over 4 KV heads, 16 nodes, a 32768-token context, the
    launch the bench times: one KV head's six query heads against the
    oracle, every output finite."""
    dev = torch.device("cuda")
    _say("case tree attn full 16 x 24/4 x 256, ctx 32768")
    inp = synth.attn_inputs(16, 24, 4, 32768, seed=40, device=dev)
    got = _run(q4, inp)
    assert np.isfinite(got).all()
    h = _host(inp)
    want = _oracle(h, heads=(2, 6))
    err = np.abs(got[:, 12:18] - want).max()
    assert err <= _tol(h), (err, _tol(h))


def test_splits_agree(q4):
    dev = torch.device("cuda")
    inp = synth.attn_inputs(16, 24, 4, 3000, seed=41, device=dev)
    a = _run(q4, inp, 1)
    h = _host(inp)
    for s in (2, 7, 0):
        b = _run(q4, inp, s)
        assert np.abs(a - b).max() <= 2 * _tol(h), s


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
