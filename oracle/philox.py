"""Philox4x32-10, the counter-based random number generator of Salmon,
Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
(SC 2011), written from its published definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

A 128-bit counter (c0, c1, c2, c3) and a 64-bit key (k0, k1) map to four
32-bit outputs through 10 rounds.  One round multiplies c0 by 0xD2511F53 and
c2 by 0xCD9E8D57 into 64-bit products (hi:lo) and forms
(hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); the key is
advanced by the Weyl increments (0x9E3779B9, 0xBB67AE85) between rounds.
"""
import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)
_SH = np.uint64(32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised over numpy arrays (broadcast); returns four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _LO for x in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & _LO
    k1 = np.asarray(k1, dtype=np.uint64) & _LO
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _LO
            k1 = (k1 + _W1) & _LO
        p0 = c[0] * _M0          # < 2^64: exact in uint64
        p1 = c[2] * _M1
        c = [((p1 >> _SH) ^ c[1] ^ k0) & _LO, p1 & _LO,
             ((p0 >> _SH) ^ c[3] ^ k1) & _LO, p0 & _LO]
    return [x.astype(np.uint32) for x in c]


def uniform24(x):
    """A uint32 output as a uniform value in (0, 1): its top 24 bits plus
    one half, times 2^-24 (every value exact in float32 and never 0 or 1)."""
    return ((np.asarray(x, dtype=np.uint64) >> np.uint64(8)).astype(np.float64)
            + 0.5) * 2.0 ** -24
