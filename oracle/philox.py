"""Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC 2011), written from its
published definition, and the dropout keep mask built from it.

TEST INFRASTRUCTURE ONLY: see the package docstring.

Philox4x32-R maps a 128-bit counter (c0, c1, c2, c3) and a 64-bit key (k0, k1)
to four 32-bit words by R rounds of
    (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2        (64-bit products)
    c <- (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)
with the key bumped by the Weyl constants (W0, W1) between rounds; the
multipliers M0 = 0xD2511F53, M1 = 0xCD9E8D57 and W0 = 0x9E3779B9 (golden
ratio), W1 = 0xBB67AE85 (sqrt(3) - 1) are the paper's.  R = 10 is the paper's
recommended round count.

The pages ("FlashAttention 원 논문 해부", sections "forward가 끝난 뒤 backward는
무엇을 저장하고 무엇을 다시 계산하는가" and "내부 구조와 실제 실행 흐름") fix only
the contract: the forward keeps the generator state, the backward regenerates
the same mask tile by tile.  They name no generator; this one is a reading.
"""
from __future__ import annotations

import numpy as np

M0, M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32(c0, c1, c2, c3, k0, k1, rounds: int = 10):
    """Vectorized Philox4x32-R: counters (arrays of any broadcastable shape) and a
    scalar key -> four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & MASK32 for x in np.broadcast_arrays(c0, c1, c2, c3)]
    k0, k1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for r in range(rounds):
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return [x.astype(np.uint32) for x in c]


def keep_threshold(p_drop: float) -> int:
    """Elements are kept iff their 16-bit uniform is below this value:
    round((1 - p_drop) * 2^16), so the keep probability is threshold / 2^16."""
    return int(round((1.0 - float(p_drop)) * 65536.0))


def uniforms16(head: int, n_q: int, n_k: int, seed: int, offset: int) -> np.ndarray:
    """uint16 [n_q, n_k]: the uniform of element (query i, key j) of attention head
    `head` (b * H + h).  Key j belongs to the 16-key group g = j // 16; the call
    with counter (i, 2 g + j % 2, head, offset) and key (seed low, seed high)
    gives eight 16-bit halves, low half first, word 0 first; key j takes half
    number (j % 16) // 2."""
    i = np.arange(n_q, dtype=np.uint64)[:, None]
    j = np.arange(n_k, dtype=np.uint64)[None, :]
    g = j // np.uint64(16)
    words = philox4x32(i, np.uint64(2) * g + j % np.uint64(2), np.uint64(head),
                       np.uint64(offset & 0xFFFFFFFF), seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    t = ((j % np.uint64(16)) // np.uint64(2)).astype(np.int64)   # half number 0..7
    stacked = np.stack(np.broadcast_arrays(*words), axis=-1)      # [n_q, n_k, 4]
    word = np.take_along_axis(stacked, np.broadcast_to(t // 2, stacked.shape[:2])[..., None],
                              axis=-1)[..., 0]
    return np.where(np.broadcast_to(t % 2, word.shape) == 0, word & 0xFFFF, word >> 16).astype(np.uint16)


def keep_mask(head: int, n_q: int, n_k: int, p_drop: float, seed: int, offset: int) -> np.ndarray:
    """Boolean [n_q, n_k]: element kept by dropout with probability p_drop."""
    return uniforms16(head, n_q, n_k, seed, offset).astype(np.int64) < keep_threshold(p_drop)
