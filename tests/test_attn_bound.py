"""The tree-attention parity bound can fail (CPU only).

The GPU tests compare every output element with the oracle under
|o_gpu - o| <= ATTN_REL * sum_p w_p |v_p| + ATTN_ABS (tests/helpers.py).  At
the benchmarked shape the outputs are small sums of values of both signs, so
a bound relative to the largest value in the cache would let whole pages go
missing.  Here the oracle itself plays the broken kernel: its output with the
values of some context pages zeroed must fall outside the bound somewhere,
while the unbroken output (trivially) stays inside.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import attn as ao
from tests.helpers import attn_bound

SCALE = 1.0 / 16.0


@pytest.fixture(scope="module")
def full_shape():
    """The full-shape GPU test's inputs (16 nodes, 24 query heads over 4 KV
    heads, a 32768-token context), restricted to KV head 2 and its six query
    heads to keep the CPU time small."""
    inp = synth.attn_inputs(16, 24, 4, 32768, seed=40, device="cpu")
    g, G = 2, 6
    h = {
        "q": inp["q"].view(__import__("torch").int16).numpy().view(np.uint16)[:, g * G:(g + 1) * G],
        "k_pages": inp["k_pages"].numpy()[:, g:g + 1],
        "v_pages": inp["v_pages"].numpy()[:, g:g + 1].copy(),
        "k_scale": inp["k_scale"].numpy()[:, g:g + 1],
        "v_scale": inp["v_scale"].numpy()[:, g:g + 1],
        "page_table": inp["page_table"].numpy(),
        "anc": inp["anc"].numpy().view(np.uint32),
        "ctx": inp["ctx_len"],
    }
    out, absw = ao.attention(h["q"], h["k_pages"], h["v_pages"], h["k_scale"],
                             h["v_scale"], h["page_table"], h["ctx"], h["anc"],
                             SCALE, with_abs=True)
    return h, out, absw


def _zeroed(h, every):
    """Oracle outputs with the values of every `every`-th context page (by
    logical index) set to zero."""
    vp = h["v_pages"].copy()
    ctx_pages = h["ctx"] // 32
    for lp in range(0, ctx_pages, every):
        vp[h["page_table"][lp]] = 0
    return ao.attention(h["q"], h["k_pages"], vp, h["k_scale"], h["v_scale"],
                        h["page_table"], h["ctx"], h["anc"], SCALE)


@pytest.mark.parametrize("every", [256, 64, 16])
def test_bound_rejects_dropped_pages(full_shape, every):
    h, out, absw = full_shape
    broken = _zeroed(h, every)
    ratio = np.abs(broken - out) / attn_bound(absw)
    assert ratio.max() > 1.0, (every, float(ratio.max()))


def test_bound_scale_at_full_shape(full_shape):
    """The bound is far below the outputs' own spread: its relative part is
    under 2^-10 of sum w|v|, not a fraction of the largest value in the
    cache (it stays 16 times and more below 2^-8 of that value)."""
    h, out, absw = full_shape
    b = attn_bound(absw)
    vmax = float(np.abs(h["v_pages"].astype(np.float64)).max() * h["v_scale"].max())
    assert b.max() < 2.0 ** -8 * vmax / 16
    assert (np.abs(out) <= absw).all()
