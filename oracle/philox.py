"""Philox4x32-10 counter-based generator, written from its published
definition [P] (Salmon et al., SC'11, section on the Philox S-box).

Test infrastructure only (see the package docstring).

One round maps the counter (c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with M0 = 0xD2511F53, M1 = 0xCD9E8D57, and the key is advanced by the Weyl
constants (0x9E3779B9, 0xBB67AE85) between rounds; ten rounds in all.

The 64-bit seed of the method supplies the key: k0 = seed mod 2^32,
k1 = seed >> 32.  How the counter words are assigned to the draws of the
method is a reading of this library (the pages name no generator at all);
it is fixed in ``gauss.projections`` and ``hyperattn.sample_positions``.
"""

import numpy as np

MASK32 = 0xFFFFFFFF
M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Arguments are integers or numpy arrays
    (any integer dtype) holding values in [0, 2^32); returns four uint64
    arrays holding the 32-bit output words."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    k0 = np.uint64(int(k0) & MASK32)
    k1 = np.uint64(int(k1) & MASK32)
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    s32 = np.uint64(32)
    msk = np.uint64(MASK32)
    for rnd in range(10):
        if rnd > 0:
            k0 = np.uint64((int(k0) + W0) & MASK32)
            k1 = np.uint64((int(k1) + W1) & MASK32)
        p0 = m0 * c0          # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> s32, p0 & msk
        hi1, lo1 = p1 >> s32, p1 & msk
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox_words(seed, count, c1=0, c2=0, c3=0):
    """The first ``count`` 32-bit words of the stream with counters
    (j, c1, c2, c3), j = 0, 1, 2, ...; word i comes from counter j = i // 4,
    output word i % 4.  Returns a uint64 array of length ``count``."""
    seed = int(seed)
    nctr = (count + 3) // 4
    j = np.arange(nctr, dtype=np.uint64)
    w = philox4x32_10(j, c1, c2, c3, seed & MASK32, (seed >> 32) & MASK32)
    out = np.stack(w, axis=1).reshape(-1)
    return out[:count]
