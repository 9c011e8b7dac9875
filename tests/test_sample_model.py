"""CPU model of the sampling row kernel's candidate merge (no GPU).

The row kernel merges S descending lists of 32 candidate keys (one per
workgroup of the fused LM head, or per slice of the standalone epilogue)
into the row's best 32 without reading every list: lane l of its wave reads
the first 4 keys of lists l, l + 64, ..; T, the 32nd largest lane maximum
of the heads, bounds the row's 32nd best key from below, and the keys read
that reach T are kept.  When some list's 4th key reaches T, T is raised to
the 32nd best kept key and the lists whose 4th key still reaches it are
read whole.  (Rows of at most 32 lists take a 16-wave exact merge
instead.)  The model restates those steps in numpy and checks, on random and on adversarial list sets, that the result is the
best 32 of all keys and that every count stays inside the kernel's LDS
areas (1024 kept lead keys and 8 lists read whole, 1248 kept keys in all).
"""
from __future__ import annotations

import numpy as np
import pytest

LIST = 32
LEAD = 4
MAX_LISTS = 512


def kth_largest(v, k):
    """The largest t with at least k of v at or above it (0 when fewer than
    k values are positive: keys are positive, 0 is none)."""
    s = np.sort(v)[::-1]
    return int(s[k - 1]) if len(s) >= k else 0


def row_merge(lists):
    S = lists.shape[0]
    assert 1 <= S <= MAX_LISTS
    if S <= LIST:
        # rows of at most 32 lists go to the 16-wave kernel, one key per
        # thread, whose sorting networks keep the exact best 32
        return best32(lists)
    padded = np.zeros((MAX_LISTS, LIST), dtype=np.uint64)
    padded[:S] = lists
    heads = padded[:, 0]
    per_lane = heads.reshape(MAX_LISTS // 64, 64)  # [i, lane] = list i*64+lane
    T = np.uint64(kth_largest(per_lane.max(axis=0), LIST))
    lead = padded[:, :LEAD]
    pool = lead[(lead != 0) & (lead >= T)]
    assert len(pool) <= LIST * (MAX_LISTS // 64) * LEAD
    if ((lead[:, -1] != 0) & (lead[:, -1] >= T)).any():
        # raise T to the 32nd best kept key; lists whose 4th key reaches it
        # are read whole
        ranked = np.sort(pool)[::-1]
        T = ranked[LIST - 1] if len(ranked) >= LIST else np.uint64(0)
        whole = np.nonzero((lead[:, -1] != 0) & (lead[:, -1] >= T))[0]
        assert len(whole) <= (8 if len(ranked) >= LIST else LIST - 1)
        rest = padded[whole, LEAD:].ravel()
        pool = np.concatenate([pool, rest[(rest != 0) & (rest >= T)]])
    assert len(pool) <= LIST * (MAX_LISTS // 64) * LEAD + 8 * (LIST - LEAD)
    out = np.zeros(LIST, dtype=np.uint64)
    best = np.sort(pool)[::-1][:LIST]
    out[:len(best)] = best
    return out


def best32(lists):
    keys = lists.ravel()
    keys = np.sort(keys[keys != 0])[::-1][:LIST]
    out = np.zeros(LIST, dtype=np.uint64)
    out[:len(keys)] = keys
    return out


def lists_from_columns(keys, S):
    """Split a row's distinct keys into S contiguous column ranges and keep
    each range's best 32, descending, zero-padded: what each workgroup or
    slice writes."""
    V = len(keys)
    out = np.zeros((S, LIST), dtype=np.uint64)
    for s in range(S):
        part = keys[V * s // S: V * (s + 1) // S]
        top = np.sort(part)[::-1][:LIST]
        out[s, :len(top)] = top
    return out


def keys_of(logit_rank, rng=None):
    """Distinct positive keys ordered as logit_rank (larger = better), with
    the column in the low bits as the kernel's key carries the token."""
    V = len(logit_rank)
    return (np.asarray(logit_rank, dtype=np.uint64) << np.uint64(32)) | \
        (np.uint64(0xFFFFFFFF) - np.arange(V, dtype=np.uint64))


@pytest.mark.parametrize("S", [33, 40, 64, 65, 255, 512])
@pytest.mark.parametrize("seed", [0, 1])
def test_random_rows(S, seed):
    rng = np.random.default_rng(seed)
    V = S * 600
    keys = keys_of(rng.integers(1, 1 << 20, size=V))
    lists = lists_from_columns(keys, S)
    assert np.array_equal(row_merge(lists), best32(lists))
    assert np.array_equal(best32(lists), np.sort(keys)[::-1][:LIST])


@pytest.mark.parametrize("S", [33, 64, 255, 512])
def test_adversarial_rows(S):
    V = S * 100
    cases = {
        # every list's keys above every later list's: the best 32 in one list
        "one list": np.arange(V, 0, -1),
        # equal logits: ties by token, the best 32 = tokens 0..31
        "ties": np.ones(V, dtype=np.int64),
        # each list holds exactly one of the best 32, at its head
        "spread": np.where(np.arange(V) % 100 == 0, 1 << 21, 1 + np.arange(V) % 7),
        # two lists' second keys beat every other list's head
        "seconds": np.concatenate([[1 << 22, (1 << 22) - 1] * 2,
                                   np.arange(V - 4) % 1000 + 1]),
    }
    for name, rank in cases.items():
        lists = lists_from_columns(keys_of(rank), S)
        assert np.array_equal(row_merge(lists), best32(lists)), name


def test_short_lists():
    """Fewer than 32 keys in every list and fewer than 32 lists with any
    (zero-padded lists, zero heads): every key is read."""
    rng = np.random.default_rng(3)
    lists = np.zeros((300, LIST), dtype=np.uint64)
    for s in rng.choice(300, size=20, replace=False):
        n = int(rng.integers(1, 5))
        lists[s, :n] = np.sort(rng.integers(1, 1 << 40, size=n).astype(np.uint64))[::-1]
    out = row_merge(lists)
    assert np.array_equal(out, best32(lists))
    assert (out[np.count_nonzero(lists):] == 0).all()


def test_most_lead_keys_kept():
    """Lists built so that lanes 1..31 hold 8 lists each whose every key is
    above lane 0's maximum (= T): about 1000 lead keys are kept, the deep
    path raises T, and at most 8 lists are read whole."""
    lists = np.zeros((MAX_LISTS, LIST), dtype=np.uint64)
    base = np.uint64(1 << 40)
    for g in range(MAX_LISTS):
        lane, i = g % 64, g // 64
        if lane == 0:
            top = 1000 + i  # lane 0's maximum is the 32nd largest lane maximum
        elif lane < 32:
            top = 1 << 30 | (lane * 8 + i) << 8
        else:
            top = 10 + i
        lists[g] = base + np.uint64(top) * np.uint64(64) - np.arange(LIST, dtype=np.uint64)
    T = kth_largest(lists[:, 0].reshape(8, 64).max(axis=0), LIST)
    lead = lists[:, :LEAD]
    assert ((lead >= np.uint64(T)).sum()) > 990
    assert np.array_equal(row_merge(lists), best32(lists))
