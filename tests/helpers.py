"""Small helpers shared by the tests: exact arithmetic and buffer assembly.

Nothing here computes the method: the exact-rational helpers below are the
independent yardstick the oracle is checked against.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    """Parse a ``name = value | citation`` fixture into {name: value}."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, _, _cite = line.partition("|")
            key, _, val = lhs.partition("=")
            val = val.strip()
            out[key.strip()] = float(val) if "." in val else int(val)
    return out


def bf16_bits_of(values) -> np.ndarray:
    """bf16 bit patterns (RNE) of float values given as numpy/python floats."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_float(bits) -> np.ndarray:
    """float32 values of bf16 bit patterns (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def assemble(codes: np.ndarray, scale_bits: np.ndarray,
             bias_bits: np.ndarray) -> np.ndarray:
    """Planar packed buffer from code bytes [N, K/2] and bf16 bit planes
    [N, K/64]."""
    N, half = codes.shape
    K = 2 * half
    packed = torch.empty(synth.packed_size(N, K), dtype=torch.uint8)
    c, s, b = synth.planes(packed, N, K)
    c.copy_(torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)))
    s.view(torch.int16).copy_(torch.from_numpy(
        np.ascontiguousarray(scale_bits, dtype=np.uint16).view(np.int16)))
    b.view(torch.int16).copy_(torch.from_numpy(
        np.ascontiguousarray(bias_bits, dtype=np.uint16).view(np.int16)))
    return packed.numpy().copy()


def split_planes(packed: np.ndarray, N: int, K: int):
    """(codes u8 [N, K/2], scale bits u16 [N, K/64], bias bits u16 [N, K/64])."""
    t = torch.from_numpy(np.ascontiguousarray(packed, dtype=np.uint8))
    c, s, b = synth.planes(t, N, K)
    return (c.numpy().copy(), s.view(torch.int16).numpy().view(np.uint16).copy(),
            b.view(torch.int16).numpy().view(np.uint16).copy())


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Code bytes [N, K/2] from 4-bit codes [N, K]: even k in the low nibble
    (the reading of the byte order this build takes)."""
    q = np.asarray(q, dtype=np.uint8)
    assert q.max(initial=0) <= 15
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def frac(x) -> Fraction:
    return Fraction(float(x))


def round_f32(v: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even)."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum_exp = max(e - 23, -149)
    scaled = a / (Fraction(2) ** quantum_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** quantum_exp
    if val >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))


def tiled_from_planar(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Bytes of the tiled layout (records of 16 rows x 4 groups), restated
    from its definition: per record, two 1 KB blocks of 16 bytes per lane
    l = j + 16*kb (code bytes kb*8..kb*8+7 of group 2p, then of group 2p+1,
    of row j, each 4-byte word's nibbles reordered to inputs 0,2,4,6,1,3,5,7)
    and 16 bytes per row j of (scale, bias) for the 4 groups."""
    codes, s, b = split_planes(packed, N, K)
    T, Q = N // 16, K // 256
    # within each 4-byte word (inputs 0..7, input i in nibble i) reorder the
    # nibbles to inputs 0, 2, 4, 6, 1, 3, 5, 7
    q = np.empty((N, K), dtype=np.uint8)
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    q = q.reshape(N, K // 8, 8)[:, :, [0, 2, 4, 6, 1, 3, 5, 7]].reshape(N, K)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    c = codes.reshape(T, 16, Q, 4, 4, 8)          # tile, j, q, group, kb, 8
    out = np.empty((T, Q, 2304), dtype=np.uint8)
    for p in range(2):
        pair = np.concatenate([c[:, :, :, 2 * p], c[:, :, :, 2 * p + 1]],
                              axis=-1)              # tile, j, q, kb, 16
        out[:, :, 1024 * p:1024 * (p + 1)] = \
            pair.transpose(0, 2, 3, 1, 4).reshape(T, Q, 1024)
    sb = np.stack([s.reshape(T, 16, Q, 4), b.reshape(T, 16, Q, 4)], axis=-1)
    sb = sb.transpose(0, 2, 1, 3, 4).reshape(T, Q, 16 * 8)   # u16 values
    out[:, :, 2048:] = sb.astype("<u2").view(np.uint8).reshape(T, Q, 256)
    return out.reshape(-1)


# Tree-verify attention: per-element bound of the GPU outputs against the
# oracle, |o_gpu - o| <= ATTN_REL * absw + ATTN_ABS, absw = sum_p w_p |v_p|
# from the oracle.  Error sources of the kernel:
#  * the value product: each probability times its value scale, divided by a
#    power of two at or above the scales (so the product is at most 2^8), is
#    rounded to fp16 and meets the exact fp16 values: each term moves by a
#    relative 2^-11 at most (a term below fp16's normal range, 2^-14, by an
#    absolute 2^-25 of the same units instead: a weight 2^-14 below the
#    page's largest, which no score of the test caches comes near);
#  * the scores: bf16 x int8 products are exact; the MFMA adds them into an
#    fp32 accumulator in 8 steps of 32, so a score is off by at most
#    8 * 2^-24 * sum_d |q_d k_d| * k_scale * scale.  For the test caches
#    (|q| < 5, |k8| <= 127, k_scale <= 0.02, scale 1/16) that is below
#    2^-13.4, which moves each softmax weight by a relative 2^-12.4 at most;
#  * the exponentials, the fp32 sums and the merge of runs: near 2^-20.
# Together below 2^-11 + 2^-12 + 2^-14 of absw (under 2^-10).  The absolute
# term covers outputs whose absw is itself tiny.
ATTN_REL = 2.0 ** -11 + 2.0 ** -12 + 2.0 ** -14
ATTN_ABS = 1e-7


def attn_bound(absw: np.ndarray) -> np.ndarray:
    return ATTN_REL * absw + ATTN_ABS


def oracle_threads() -> int:
    """Threads for the CPU oracle: the CPUs this process may run on, at most
    16 (a one-GPU share of the test machine's host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))
