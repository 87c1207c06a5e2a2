"""Philox-4x32-10 counter-based generator and the dropout keep-mask built on it
(test infrastructure).

The pages draw the dropout mask from a Bernoulli distribution ([TRAIN] Dropout
section) and require that sequence-parallel ranks draw different masks ([SP]
"Dropout 的 RNG 为什么要分域管理？" and its RNG-domain table).  Neither page
names a generator.  The library fixes one published counter-based generator
so that the kernel and this oracle can each implement it from its definition:

  Philox-4x32 with 10 rounds, from J. K. Salmon, M. A. Moraes, R. O. Dror,
  D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 (§4):
    one round maps counter (c0,c1,c2,c3) under key (k0,k1) to
      (hi(M1·c2) ^ c1 ^ k0,  lo(M1·c2),  hi(M0·c0) ^ c3 ^ k1,  lo(M0·c0))
    with M0 = 0xD2511F53, M1 = 0xCD9E8D57; the key is bumped by the Weyl
    constants (0x9E3779B9, 0xBB67AE85) between rounds.

Mask rule (the reading taken where the pages are silent; the same rule is
written independently in the HIP source): for element e of the row-major [s, h] activation (e = row·h + col,
over the whole sequence, so each sequence shard sees its own block of
counters), q = e // 4 and w = e % 4; u = word w of Philox(counter=(q mod 2³²,
q div 2³², 0, 0), key=(seed mod 2³², seed div 2³²)).  The element is dropped
iff u < floor(p·2³²); survivors are scaled by 1/(1−p).
"""

import math

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox-4x32-10.  Arguments are integer arrays (or scalars)
    holding 32-bit values; returns four uint64 arrays holding 32-bit words."""
    c0 = np.asarray(c0, dtype=np.uint64) & _MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & _MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & _MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & _MASK32
    k0 = np.uint64(int(k0) & _MASK32)
    k1 = np.uint64(int(k1) & _MASK32)
    m0, m1 = np.uint64(M0), np.uint64(M1)
    mask, sh = np.uint64(_MASK32), np.uint64(32)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + W0) & _MASK32)
            k1 = np.uint64((int(k1) + W1) & _MASK32)
        p0 = m0 * c0  # < 2^64: both factors < 2^32
        p1 = m1 * c2
        hi0, lo0 = p0 >> sh, p0 & mask
        hi1, lo1 = p1 >> sh, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def drop_threshold(p):
    """Integer threshold floor(p·2³²) for drop probability p in [0, 1)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(math.floor(p * 4294967296.0))


def uniform_words(e, seed):
    """The 32-bit draw for global element indices e (integer array)."""
    e = np.asarray(e, dtype=np.uint64)
    q = e >> np.uint64(2)
    w = (e & np.uint64(3)).astype(np.int64)
    r0, r1, r2, r3 = philox4x32_10(q & np.uint64(_MASK32), q >> np.uint64(32), 0, 0,
                                   seed & _MASK32, (seed >> 32) & _MASK32)
    words = np.stack([r0, r1, r2, r3], axis=0)
    return np.take_along_axis(words, w[None, ...], axis=0)[0]


def keep_mask(row0, rows, h, p, seed):
    """Boolean keep mask for rows [row0, row0+rows) of a row-major [*, h]
    activation.  True = kept."""
    e = (np.arange(row0, row0 + rows, dtype=np.uint64)[:, None] * np.uint64(h)
         + np.arange(h, dtype=np.uint64)[None, :])
    return uniform_words(e, seed) >= np.uint64(drop_threshold(p))
