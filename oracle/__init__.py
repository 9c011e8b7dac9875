"""CPU oracle for the group-affine Q4 verify GEMM (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it; the C source ``q4_oracle.c`` states what is computed
and which readings of the pages it takes.

Arrays are numpy arrays.  Activations are passed as raw bf16 bit patterns
(``uint16``), the packed weights as ``uint8`` bytes.

Functions and the passages they follow:

* :func:`packed_bytes` -- the packed size, 9 bytes per 16 weights (Splash
  engine article, section "The engine hard-codes the model", the
  ``q4PackedBytes`` listing and the sentence after it).
* :func:`dequant` -- w = scale * q + bias per group of 64 inputs (same
  section; the affine form scale/bias).
* :func:`gemm` -- y = x @ W^T with fp64 accumulation, plus sum |x*w| (Splash
  article, section "Why Apple silicon, and why not the M5": verify rows make
  decode an M x K x N GEMM; qwen-spec page, Notes: the matmul that multiplies
  all rows at once).
* :mod:`oracle.sample` -- the verify step's sampling epilogue: top-k
  candidates, target probabilities, the accept test and the residual draw
  (``verify_sample.c``).
* :mod:`oracle.gdn` -- the Gated DeltaNet state of a verify pass: each tree
  node's output from the shared state plus the updates along its path, and
  the commit of the accepted path (``gdn_state.c``).
* :mod:`oracle.attn` -- tree-verify attention over the paged int8 KV cache
  with the ancestor mask (``tree_attn.c``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "q4_oracle.c")
LIB_PATH = os.path.join(_HERE, "libq4oracle.so")

GROUP = 64
OK = 0
EINVAL = -1
EOVERFLOW = -3

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
             "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
             "-Werror"]


class OracleError(RuntimeError):
    pass


def compile_source(src: str, out: str, extra=()) -> str:
    """Compile a C oracle source into a shared library with gcc."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, *extra, "-o", tmp, src, "-lm"],
                   check=True)
    os.replace(tmp, out)
    return out


SAMPLE_SOURCE = os.path.join(_HERE, "verify_sample.c")
SAMPLE_LIB_PATH = os.path.join(_HERE, "libverifysample.so")
GDN_SOURCE = os.path.join(_HERE, "gdn_state.c")
GDN_LIB_PATH = os.path.join(_HERE, "libgdnstate.so")
ATTN_SOURCE = os.path.join(_HERE, "tree_attn.c")
ATTN_LIB_PATH = os.path.join(_HERE, "libtreeattn.so")


def build(force: bool = True) -> str:
    """Compile the oracles (plain IEEE arithmetic, no FMA contraction)."""
    if force or not os.path.exists(LIB_PATH):
        compile_source(SOURCE, LIB_PATH)
    if force or not os.path.exists(SAMPLE_LIB_PATH):
        compile_source(SAMPLE_SOURCE, SAMPLE_LIB_PATH)
    if force or not os.path.exists(GDN_LIB_PATH):
        compile_source(GDN_SOURCE, GDN_LIB_PATH)
    if force or not os.path.exists(ATTN_LIB_PATH):
        compile_source(ATTN_SOURCE, ATTN_LIB_PATH)
    return LIB_PATH


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, lib_path: str = LIB_PATH):
        if lib_path == LIB_PATH and not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(lib_path)
        i64, u64p = ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)
        lib.q4o_packed_bytes.argtypes = [i64, i64, u64p]
        lib.q4o_packed_bytes.restype = ctypes.c_int
        lib.q4o_dequant.argtypes = [ctypes.c_void_p, i64, i64, ctypes.c_void_p]
        lib.q4o_dequant.restype = ctypes.c_int
        lib.q4o_gemm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, i64,
                                 i64, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_int)]
        lib.q4o_gemm.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    @staticmethod
    def _check(status: int, what: str) -> None:
        if status != OK:
            raise OracleError(f"{what}: oracle status {status}")

    def packed_bytes_status(self, N: int, K: int) -> int:
        """Status code of the size function (for the error-path checks)."""
        out = ctypes.c_uint64(0)
        return int(self.lib.q4o_packed_bytes(int(N), int(K),
                                             ctypes.byref(out)))

    def packed_bytes(self, N: int, K: int) -> int:
        """Bytes of an N x K packed matrix (elements/16*9, overflow-checked)."""
        out = ctypes.c_uint64(0)
        self._check(self.lib.q4o_packed_bytes(int(N), int(K),
                                              ctypes.byref(out)),
                    f"packed_bytes({N}, {K})")
        return int(out.value)

    def _as_packed(self, W, N, K) -> np.ndarray:
        W = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1)
        want = self.packed_bytes(N, K)
        if W.size != want:
            raise OracleError(f"packed buffer has {W.size} bytes, expected "
                              f"{want} for {N}x{K}")
        return W

    def dequant(self, W, N: int, K: int) -> np.ndarray:
        """fp32 [N, K] dequantised weights of the packed buffer ``W``."""
        W = self._as_packed(W, N, K)
        out = np.empty((N, K), dtype=np.float32)
        self._check(self.lib.q4o_dequant(W.ctypes.data, int(N), int(K),
                                         out.ctypes.data), "dequant")
        return out

    def gemm(self, x_bits, W, N: int, K: int, threads: int = 0):
        """Return ``(y32, y64, a64, threads_used)`` for x (bf16 bits [M, K]).

        y64 is the fp64 sum in ascending k, a64 the fp64 sum of |x*w|, y32
        the fp32 rounding of y64; all three are [M, N].
        """
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        if x_bits.ndim != 2 or x_bits.shape[1] != K:
            raise OracleError(f"x must be [M, {K}] bf16 bits, got "
                              f"{x_bits.shape}")
        M = x_bits.shape[0]
        W = self._as_packed(W, N, K)
        y64 = np.empty((M, N), dtype=np.float64)
        a64 = np.empty((M, N), dtype=np.float64)
        y32 = np.empty((M, N), dtype=np.float32)
        used = ctypes.c_int(0)
        self._check(self.lib.q4o_gemm(x_bits.ctypes.data, W.ctypes.data,
                                      int(M), int(N), int(K), y64.ctypes.data,
                                      a64.ctypes.data, y32.ctypes.data,
                                      int(threads), ctypes.byref(used)),
                    "gemm")
        return y32, y64, a64, int(used.value)

    def gemm_status(self, M: int, N: int, K: int) -> int:
        """Status of the GEMM's argument checks, for shapes it rejects."""
        if M >= 1 and self.packed_bytes_status(N, K) == OK:
            raise ValueError("gemm_status is for shapes the oracle rejects")
        dummy_x = np.zeros(1, dtype=np.uint16)
        dummy_w = np.zeros(1, dtype=np.uint8)
        return int(self.lib.q4o_gemm(dummy_x.ctypes.data, dummy_w.ctypes.data,
                                     int(M), int(N), int(K), None, None, None,
                                     1, None))


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(LIB_PATH)
    return _default


def packed_bytes(N: int, K: int) -> int:
    return default().packed_bytes(N, K)


def packed_bytes_status(N: int, K: int) -> int:
    return default().packed_bytes_status(N, K)


def dequant(W, N: int, K: int) -> np.ndarray:
    return default().dequant(W, N, K)


def gemm(x_bits, W, N: int, K: int, threads: int = 0):
    return default().gemm(x_bits, W, N, K, threads)


def gemm_status(M: int, N: int, K: int) -> int:
    return default().gemm_status(M, N, K)
