"""CPU oracle of tree-verify attention over a paged int8 KV cache (test
infrastructure).

A ctypes view of ``tree_attn.c``, which states what is computed and the
readings it takes (Splash engine article: the attention shapes and the int8
KV page with a per-token fp32 scale; qwen-spec page: the tree seen through an
ancestor mask, the cache read in place).

Cache layout per physical page and KV head: keys [32][D] int8, values
transposed [D][32] int8, one fp32 scale per token for each.  The tree's keys
and values follow the context: node j at position ctx_len + j.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import ATTN_LIB_PATH, build

PAGE = 32


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def ancestor_masks(parent) -> np.ndarray:
    """uint32 [M]: bit j of entry i set iff node j is node i or one of its
    ancestors (parent[i] < i, -1 for a child of the context)."""
    M = len(parent)
    out = np.zeros(M, dtype=np.uint32)
    for i in range(M):
        n = i
        while n >= 0:
            out[i] |= np.uint32(1) << np.uint32(n)
            n = int(parent[n])
    return out


class AttnOracle:
    """ctypes view of one compiled copy of tree_attn.c."""

    def __init__(self, lib_path: str = ATTN_LIB_PATH):
        if lib_path == ATTN_LIB_PATH and not os.path.exists(lib_path):
            build(force=False)
        lib = ctypes.CDLL(lib_path)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.ta_tree_attention.argtypes = [P, I, I, I, I, P, P, P, P, P, I,
                                          ctypes.c_int64, P, ctypes.c_double,
                                          P, P]
        lib.ta_tree_attention.restype = I
        self.lib = lib

    def attention(self, q_bits, k_pages, v_pages, k_scale, v_scale,
                  page_table, ctx_len: int, anc, scale: float,
                  with_abs: bool = False):
        """Outputs [M, Hq, D] (float64); with ``with_abs`` the pair
        (outputs, absw), absw[i, h, d] = sum_p w_p |v_p[d]| with the same
        softmax weights (the scale of the rounding error of the terms).

        q_bits uint16 [M, Hq, D] (bf16 bit patterns); k_pages int8
        [pool, Hkv, 32, D]; v_pages int8 [pool, Hkv, D, 32]; k_scale,
        v_scale float32 [pool, Hkv, 32]; page_table int32 (logical page ->
        physical page); anc uint32 [M] ancestor-or-self masks."""
        q = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kp = np.ascontiguousarray(k_pages, dtype=np.int8)
        vp = np.ascontiguousarray(v_pages, dtype=np.int8)
        ks = np.ascontiguousarray(k_scale, dtype=np.float32)
        vs = np.ascontiguousarray(v_scale, dtype=np.float32)
        pt = np.ascontiguousarray(page_table, dtype=np.int32).reshape(-1)
        an = np.ascontiguousarray(anc, dtype=np.uint32).reshape(-1)
        M, Hq, D = q.shape
        pool, Hkv = kp.shape[0], kp.shape[1]
        if (kp.shape != (pool, Hkv, PAGE, D) or vp.shape != (pool, Hkv, D, PAGE)
                or ks.shape != (pool, Hkv, PAGE) or vs.shape != ks.shape
                or an.shape != (M,)):
            raise ValueError("attention: inconsistent shapes")
        if pt.size < (ctx_len + M + PAGE - 1) // PAGE:
            raise ValueError("attention: page table too short")
        out = np.zeros((M, Hq, D), dtype=np.float64)
        absw = np.zeros((M, Hq, D), dtype=np.float64) if with_abs else None
        st = self.lib.ta_tree_attention(_p(q), M, Hq, Hkv, D, _p(kp), _p(vp),
                                        _p(ks), _p(vs), _p(pt), pool,
                                        int(ctx_len), _p(an), float(scale),
                                        _p(out),
                                        None if absw is None else _p(absw))
        if st != 0:
            raise ValueError(f"ta_tree_attention status {st}")
        return (out, absw) if with_abs else out


_default = None


def default() -> AttnOracle:
    global _default
    if _default is None:
        _default = AttnOracle()
    return _default


def attention(*a, **kw):
    return default().attention(*a, **kw)
