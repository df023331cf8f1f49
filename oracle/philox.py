"""Counter-based random bits for attention dropout: Philox4x32-10 and the keep-bit layout.

TEST INFRASTRUCTURE ONLY.  The test suite is the only user; the product path has its own
generator kernel and this module shares no code with it.

Philox4x32-10 is restated from its published definition (Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): a 128-bit counter (c0, c1, c2, c3) and a
64-bit key (k0, k1) pass through ten rounds.  A round multiplies c0 and c2 by the two round
multipliers, keeping both halves of each 64-bit product, and mixes them with the other two
counter words and the key; the key is advanced by the two Weyl increments (from the golden ratio
and sqrt(3) - 1) before every round but the first.

Dropout (the "dropout_p" parameter of ffpa_attn_func on the ffpa-attn "API Reference" page, which
names SDPA-style attention dropout) keeps each attention weight independently with probability
1 - p and scales the kept ones by 1 / (1 - p).  The keep decisions of this library form a bitmask:

    keep[b, h, r, w]  (uint32, w < ceil(Nkv / 32)), bit i set  <=>  key 32 w + i is kept for query
                                                                    row r of batch b, query head h

and are drawn from Philox4x32-10 with key (seed mod 2^32, seed div 2^32) and, for row index
R = (b * Hq + h) * Nq + r, word w and block j < 8, the counter (8 w + j, R mod 2^32, R div 2^32,
offset).  Its four outputs u0..u3 decide keys 32 w + 4 j + i: kept iff u_i >= floor(p * 2^32).
Bits of keys at or past Nkv are 0.  This mapping is this library's own choice; the pages fix none.
"""
from __future__ import annotations

import numpy as np

_M0 = 0xD2511F53
_M1 = 0xCD9E8D57
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """One Philox4x32-10 block on Python integers: counter (4 words), key (2 words) -> 4 words."""
    c0, c1, c2, c3 = (int(x) & _MASK32 for x in counter)
    k0, k1 = (int(x) & _MASK32 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK32
            k1 = (k1 + _W1) & _MASK32
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & _MASK32, p1 & _MASK32, ((p0 >> 32) ^ c3 ^ k1) & _MASK32, p0 & _MASK32
    return c0, c1, c2, c3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """The same block on numpy uint64 arrays holding 32-bit values (element-wise over counters)."""
    m = np.uint64(_MASK32)
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & m for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & m
    k1 = np.asarray(k1, dtype=np.uint64) & m
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(_W0)) & m
            k1 = (k1 + np.uint64(_W1)) & m
        p0 = np.uint64(_M0) * c0  # < 2^64: exact in uint64
        p1 = np.uint64(_M1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0) & m, p1 & m, ((p0 >> np.uint64(32)) ^ c3 ^ k1) & m, p0 & m
    return c0, c1, c2, c3


def drop_threshold(p: float) -> int:
    """floor(p * 2^32) for the float32 value of p (0 <= p < 1): a draw below it drops the key."""
    p32 = float(np.float32(p))
    if not 0.0 <= p32 < 1.0:
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(p32 * 4294967296.0)


def dropout_keep_rows(rows, Nkv: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """Keep words [len(rows), ceil(Nkv / 32)] uint32 of the given row indices R = (b * Hq + h) * Nq + r."""
    W = (Nkv + 31) // 32
    thr = np.uint64(drop_threshold(p))
    R = np.asarray(rows, dtype=np.uint64)[:, None, None]
    w = np.arange(W, dtype=np.uint64)[None, :, None]
    j = np.arange(8, dtype=np.uint64)[None, None, :]
    shape = (R.shape[0], W, 8)
    c0 = np.broadcast_to(np.uint64(8) * w + j, shape)
    c1 = np.broadcast_to(R & np.uint64(_MASK32), shape)
    c2 = np.broadcast_to(R >> np.uint64(32), shape)
    c3 = np.full(shape, offset & _MASK32, dtype=np.uint64)
    u = philox4x32_10_np(c0, c1, c2, c3, seed & _MASK32, (seed >> 32) & _MASK32)
    keep = np.zeros((R.shape[0], W), dtype=np.uint64)
    for jj in range(8):
        for i in range(4):
            keep |= (u[i][:, :, jj] >= thr).astype(np.uint64) << np.uint64(4 * jj + i)
    # keys at or past Nkv are never kept
    valid = np.zeros(W, dtype=np.uint64)
    for key in range(Nkv):
        valid[key // 32] |= np.uint64(1) << np.uint64(key % 32)
    keep &= valid[None, :]
    return keep.astype(np.uint32)


def dropout_keep_bits(B: int, Hq: int, Nq: int, Nkv: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """Keep bitmask [B, Hq, Nq, ceil(Nkv / 32)] uint32 of the layout in the module docstring."""
    keep = dropout_keep_rows(np.arange(B * Hq * Nq), Nkv, p, seed, offset)
    return keep.reshape(B, Hq, Nq, keep.shape[-1])


# Planted-mistake switches of keep_matrix (tests of the pins only).
KEEP_FAULT_NONE = 0
KEEP_FAULT_BIT_REVERSED = 1   # key 32 w + i read from bit 31 - i
KEEP_FAULT_WORD_SHIFTED = 2   # key 32 w + i read from word w + 1 (the last word from word 0)


def keep_matrix(keep_bits: np.ndarray, Nkv: int, fault: int = KEEP_FAULT_NONE) -> np.ndarray:
    """Unpacks [..., W] keep words into a [..., Nkv] 0/1 float64 array (bit i of word w = key 32 w + i)."""
    kb = np.asarray(keep_bits, dtype=np.uint64)
    if fault == KEEP_FAULT_WORD_SHIFTED:
        kb = np.roll(kb, -1, axis=-1)
    shifts = np.arange(32, dtype=np.uint64)
    if fault == KEEP_FAULT_BIT_REVERSED:
        shifts = shifts[::-1].copy()
    bits = (kb[..., :, None] >> shifts) & np.uint64(1)
    return bits.reshape(*kb.shape[:-1], kb.shape[-1] * 32)[..., :Nkv].astype(np.float64)
