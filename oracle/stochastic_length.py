"""Stochastic length, the plain definition -- TEST INFRASTRUCTURE ONLY.

Stochastic length (the page "Generative recommenders / GRs" summary of
"Actions Speak Louder than Words", section 2.1; "行动胜于言语：万亿参数序列转导器
用于生成式推荐", section "2.1"): in training, a user history longer than a cap is
replaced by a random subsequence that keeps the events' order.  Reading taken
(the pages do not fix the sampler): each event j of sequence b gets a key
from a counter-based generator, Philox-4x64-10 with counter (j, b, step, 0)
and key (seed, 0x534c), first output word, top 32 bits; a sequence of L
events keeps the min(cap_b, L) events with the smallest (key, j), in
their original order.  Every subset of that size is equally likely.

Philox-4x64-10 is written from its published definition (Salmon, Moraes,
Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): ten
rounds of two 64x64->128-bit multiplications with fixed multipliers, the
high halves xor-ed with the other counter words and the key, the key bumped
by fixed Weyl constants between rounds.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
MASK64 = (1 << 64) - 1
DOMAIN = 0x534C


def philox4x64(counter, key, rounds: int = 10):
    """One Philox-4x64 block: 4 counter words, 2 key words -> 4 words (ints)."""
    x0, x1, x2, x3 = (int(c) & MASK64 for c in counter)
    k0, k1 = (int(k) & MASK64 for k in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + W0) & MASK64
            k1 = (k1 + W1) & MASK64
        p0 = M0 * x0
        p1 = M1 * x2
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def event_keys(L: int, b: int, seed: int, step: int) -> np.ndarray:
    """uint32 sort keys of events 0..L-1 of sequence b."""
    return np.array([philox4x64((j, b, step, 0), (seed, DOMAIN))[0] >> 32 for j in range(L)],
                    dtype=np.uint64)


def select_from_keys(u: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k smallest (key, index) pairs, ascending."""
    order = np.lexsort((np.arange(len(u)), u))     # by key, then index
    return np.sort(order[:k])


def select(offsets, caps, seed: int, step: int):
    """Kept source rows of every sequence, in order, and the packed offsets.

    offsets: [B+1] jagged input; caps: [B] (or one int) caps.  Returns
    (out_offsets int32 [B+1], out_index int64 [sum of kept] source rows).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    B = len(offsets) - 1
    caps = np.broadcast_to(np.asarray(caps, dtype=np.int64), (B,))
    out_off = np.zeros(B + 1, dtype=np.int64)
    idx = []
    for b in range(B):
        L = int(offsets[b + 1] - offsets[b])
        k = min(int(caps[b]), L)
        keep = np.arange(L) if k >= L else select_from_keys(event_keys(L, b, seed, step), k)
        idx.append(offsets[b] + keep)
        out_off[b + 1] = out_off[b] + len(keep)
    index = np.concatenate(idx) if idx else np.zeros(0, np.int64)
    return out_off.astype(np.int32), index.astype(np.int64)


def gather(x: np.ndarray, index: np.ndarray) -> np.ndarray:
    """Rows of x at the kept source rows, packed."""
    return np.asarray(x)[index]
