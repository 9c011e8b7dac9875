"""CPU oracle of the verify step's sampling epilogue (test infrastructure).

A ctypes view of ``verify_sample.c``, which states what is computed and the
passages it follows (Splash engine article, section "Exact, up to top-32";
qwen-spec page, the fused sampling kernel and the sampling paragraph).

* :func:`topk` -- the top_k candidates of each row: larger logit first,
  equal logits by smaller token index.
* :func:`sample` -- target probabilities (temperature over the candidates,
  top-p prefix, renormalised), the accept test u q(d) < p(d) and the residual
  draw max(p - q, 0) at v, with the margin of each decision.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import SAMPLE_LIB_PATH, build

MAX_TOPK = 32
MAX_DRAFT = 16


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class SampleOracle:
    """ctypes view of one compiled copy of verify_sample.c."""

    def __init__(self, lib_path: str = SAMPLE_LIB_PATH):
        if lib_path == SAMPLE_LIB_PATH and not os.path.exists(lib_path):
            build(force=False)
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        lib.vs_topk.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                P, P]
        lib.vs_topk.restype = ctypes.c_int
        lib.vs_sample.argtypes = [P, P, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_double, ctypes.c_double, P, P, P,
                                  ctypes.c_int, P, P, P, P, P, P, P, P]
        lib.vs_sample.restype = ctypes.c_int
        self.lib = lib

    def topk(self, logits, k: int):
        """(index int32 [M, k], value float32 [M, k]) of each row of the
        fp32 logits [M, V]."""
        lg = np.ascontiguousarray(logits, dtype=np.float32)
        if lg.ndim != 2:
            raise ValueError("logits must be [M, V]")
        M, V = lg.shape
        idx = np.zeros((M, k), dtype=np.int32)
        val = np.zeros((M, k), dtype=np.float32)
        st = self.lib.vs_topk(_p(lg), M, V, k, _p(idx), _p(val))
        if st != 0:
            raise ValueError(f"vs_topk status {st}")
        return idx, val

    def sample(self, top_idx, top_val, T: float, top_p: float, draft_tok,
               draft_idx, draft_q, u, v) -> dict:
        """Steps 2-4 for rows whose candidates come from :meth:`topk`.
        draft_idx [M, kd] / draft_q [M, kd] are the draft's candidate tokens
        and probabilities (kd may be 0); u, v [M] uniforms in [0, 1)."""
        ti = np.ascontiguousarray(top_idx, dtype=np.int32)
        tv = np.ascontiguousarray(top_val, dtype=np.float32)
        M, k = ti.shape
        dt = np.ascontiguousarray(draft_tok, dtype=np.int32).reshape(M)
        di = np.ascontiguousarray(draft_idx, dtype=np.int32).reshape(M, -1)
        dq = np.ascontiguousarray(draft_q, dtype=np.float64).reshape(M, -1)
        kd = di.shape[1]
        uu = np.ascontiguousarray(u, dtype=np.float64).reshape(M)
        vv = np.ascontiguousarray(v, dtype=np.float64).reshape(M)
        out = {"p": np.zeros((M, k)), "greedy": np.zeros(M, dtype=np.int32),
               "accept": np.zeros(M, dtype=np.int32),
               "token": np.zeros(M, dtype=np.int32),
               "accept_margin": np.zeros(M), "draw_margin": np.zeros(M)}
        st = self.lib.vs_sample(
            _p(ti), _p(tv), M, k, float(T), float(top_p), _p(dt), _p(di),
            _p(dq), kd, _p(uu), _p(vv), _p(out["p"]), _p(out["greedy"]),
            _p(out["accept"]), _p(out["token"]), _p(out["accept_margin"]),
            _p(out["draw_margin"]))
        if st != 0:
            raise ValueError(f"vs_sample status {st}")
        return out


_default = None


def default() -> SampleOracle:
    global _default
    if _default is None:
        _default = SampleOracle()
    return _default


def topk(logits, k: int):
    return default().topk(logits, k)


def sample(top_idx, top_val, T: float, top_p: float, draft_tok, draft_idx,
           draft_q, u, v) -> dict:
    return default().sample(top_idx, top_val, T, top_p, draft_tok, draft_idx,
                            draft_q, u, v)
