"""Philox4x32-10 counter-based generator and the stochastic-rounding stream map.

Test infrastructure only (see oracle/__init__.py).

Generator: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3" (SC'11), Philox4x32 with 10 rounds.  One round maps counter
(c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with the 32x32->64-bit products of the round multipliers M0 = 0xD2511F53 and
M1 = 0xCD9E8D57.  Between rounds the key is bumped by the Weyl constants
W0 = 0x9E3779B9, W1 = 0xBB67AE85 (mod 2**32), so round r (0-based) uses
(k0 + r*W0, k1 + r*W1).

Stream map (a reading: the NVFP4 pretraining post, "NVFP4 pretraining recipe"
ingredient 5, asks only for unbiased stochastic rounding on gradient
quantizers): for element (r, c) of a quantized output of shape [R', C'] in its
own orientation, idx = r*C' + c.  The Philox call with key = (seed lo, seed hi)
and counter = (lo(idx >> 3), hi(idx >> 3), offset, stream) yields four 32-bit
words, i.e. eight 16-bit halves; element idx takes half (idx & 7) of them:
word (idx & 7) >> 1, low half for even idx.  stream is 0 for rowwise outputs
and 1 for columnwise (transposed) outputs.
"""

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)

STREAM_ROW = 0
STREAM_COL = 1


def philox4x32_10(counter, key):
    """counter: 4 uint32 arrays (broadcastable); key: 2 uint32 scalars or arrays.

    Returns 4 uint32 arrays (the output words x0..x3)."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in counter)
    k0 = int(key[0]) & 0xFFFFFFFF
    k1 = int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        p0 = M0 * c0                      # < 2**64, exact in uint64
        p1 = M1 * c2
        n0 = (p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0)
        n1 = p1 & MASK32
        n2 = (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1)
        n3 = p0 & MASK32
        c0, c1, c2, c3 = n0, n1, n2, n3
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def sr_random16(idx, seed, offset, stream):
    """16-bit random word for each element index idx (uint64 array) under the
    stream map described in the module docstring."""
    idx = np.asarray(idx, dtype=np.uint64)
    grp = idx >> np.uint64(3)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    key = (seed & 0xFFFFFFFF, seed >> 32)
    ctr = (grp & MASK32, grp >> np.uint64(32),
           np.full(idx.shape, int(offset) & 0xFFFFFFFF, dtype=np.uint64),
           np.full(idx.shape, int(stream) & 0xFFFFFFFF, dtype=np.uint64))
    words = np.stack(philox4x32_10(ctr, key), axis=0)          # [4, ...]
    lane = (idx & np.uint64(7)).astype(np.int64)
    w = np.take_along_axis(words, (lane >> 1)[None, ...], axis=0)[0]
    half = (lane & 1).astype(np.uint32)
    return ((w >> (np.uint32(16) * half)) & np.uint32(0xFFFF)).astype(np.uint32)


def sr_random16_grid(rows, cols, seed, offset, stream, row_ids=None):
    """16-bit random words for a [rows, cols] output in its own orientation.

    row_ids (optional) gives the global row index of each of the `rows` rows
    when only a subset of the output's rows is being computed."""
    r = np.arange(rows, dtype=np.uint64) if row_ids is None else np.asarray(row_ids, dtype=np.uint64)
    idx = r[:, None] * np.uint64(cols) + np.arange(cols, dtype=np.uint64)[None, :]
    return sr_random16(idx, seed, offset, stream)
