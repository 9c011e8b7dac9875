"""CPU oracle of the Gated DeltaNet state in a verify pass (test infrastructure).

A ctypes view of ``gdn_state.c``, which states what is computed and the
passages it follows (Splash engine article, section on what one step reads;
qwen-spec page, the paragraph on the hybrid model and the figure after it).

* :func:`tree_out` -- each tree node's output from the shared state plus the
  gated delta-rule updates along its own path (one layer).
* :func:`commit` -- the state after the accepted path's updates (all layers).

All arithmetic is IEEE double; the inputs are fp32 arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import GDN_LIB_PATH, build


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


class GdnOracle:
    """ctypes view of one compiled copy of gdn_state.c."""

    def __init__(self, lib_path: str = GDN_LIB_PATH):
        if lib_path == GDN_LIB_PATH and not os.path.exists(lib_path):
            build(force=False)
        lib = ctypes.CDLL(lib_path)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.gdn_tree_out.argtypes = [P, I, I, I, I, I, P, P, P, P, P, P, P]
        lib.gdn_tree_out.restype = I
        lib.gdn_commit.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, I]
        lib.gdn_commit.restype = I
        self.lib = lib

    def tree_out(self, S0, q, k, v, alpha, beta, parent):
        """Outputs [M, H, dv] (float64) of one layer.

        S0 [H, dv, dk]; q, k [M, Hk, dk]; v [M, H, dv]; alpha, beta [M, H];
        parent [M] (-1: child of the context, else an earlier node)."""
        S0, q, k, v = _f32(S0), _f32(q), _f32(k), _f32(v)
        alpha, beta = _f32(alpha), _f32(beta)
        parent = np.ascontiguousarray(parent, dtype=np.int32)
        H, dv, dk = S0.shape
        M, Hk = k.shape[0], k.shape[1]
        if (q.shape != (M, Hk, dk) or k.shape != (M, Hk, dk)
                or v.shape != (M, H, dv) or alpha.shape != (M, H)
                or beta.shape != (M, H) or parent.shape != (M,)):
            raise ValueError("tree_out: inconsistent shapes")
        out = np.zeros((M, H, dv), dtype=np.float64)
        st = self.lib.gdn_tree_out(_p(S0), H, Hk, dv, dk, M, _p(q), _p(k),
                                   _p(v), _p(alpha), _p(beta), _p(parent),
                                   _p(out))
        if st != 0:
            raise ValueError(f"gdn_tree_out status {st}")
        return out

    def commit(self, S, k, v, alpha, beta, path):
        """State [L, H, dv, dk] (float64) after the accepted nodes' updates.

        S [L, H, dv, dk]; k [L, M, Hk, dk]; v [L, M, H, dv]; alpha, beta
        [L, M, H]; path: the accepted node indices, root first."""
        S = np.array(S, dtype=np.float64, order="C", copy=True)
        k, v = _f32(k), _f32(v)
        alpha, beta = _f32(alpha), _f32(beta)
        path = np.ascontiguousarray(path, dtype=np.int32).reshape(-1)
        L, H, dv, dk = S.shape
        M, Hk = k.shape[1], k.shape[2]
        if (k.shape != (L, M, Hk, dk) or v.shape != (L, M, H, dv)
                or alpha.shape != (L, M, H) or beta.shape != (L, M, H)):
            raise ValueError("commit: inconsistent shapes")
        st = self.lib.gdn_commit(_p(S), L, H, Hk, dv, dk, M, _p(k), _p(v),
                                 _p(alpha), _p(beta),
                                 _p(path) if path.size else None,
                                 int(path.size))
        if st != 0:
            raise ValueError(f"gdn_commit status {st}")
        return S


_default = None


def default() -> GdnOracle:
    global _default
    if _default is None:
        _default = GdnOracle()
    return _default


def tree_out(*a, **kw):
    return default().tree_out(*a, **kw)


def commit(*a, **kw):
    return default().commit(*a, **kw)
