"""Philox4x32-10 counter-based generator and the attention-dropout keep mask
(oracle side).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Philox4x32 is defined in J. K. Salmon, M. A. Moraes, R. O. Dror and
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011),
section 3.3: a 128-bit counter (four 32-bit words) and a 64-bit key (two
words); each of the 10 rounds multiplies words 0 and 2 by the constants
0xD2511F53 and 0xCD9E8D57 into 64-bit products, and the new words are
(hi(product of word 2) ^ word 1 ^ key 0, lo(product of word 2),
 hi(product of word 0) ^ word 3 ^ key 1, lo(product of word 0)).
Between rounds the key is bumped by the Weyl constants 0x9E3779B9 and
0xBB67AE85 (mod 2^32).  Written here with numpy uint64 arithmetic, vectorised
over counters.

Dropout mapping (the reading used by the library, see the dropout entry
points in include/gptattn.h): the pages fix only the drop probability p, so
the generator and the width of its draws are this library's choice.  For
head-problem n = b * H + h, query i and key j, the generator runs on counter
(j // 4, i // 2, n, stream) with key (seed & 0xffffffff, seed >> 32); the
draw x is the low 16 bits of output word j % 4 for even i and its high 16
bits for odd i.  The weight is kept iff x >= thr, thr = ceil(p * 2^16) (so it
is dropped with probability thr / 2^16), and a kept weight is scaled by the
inverse of the keep probability so realised, 2^16 / (2^16 - thr): over the
2^16 equally likely draws the scaled keep factor then averages to exactly 1
(dropout leaves the expected weights unchanged; with 1 / (1 - p) the
rounding of p * 2^16 up to thr would leave a bias of up to 2^-16 / (1 - p)).
"""

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds.  Counters are arrays (broadcast together)
    of values < 2^32; k0, k1 are Python ints < 2^32.  Returns four uint64
    arrays holding 32-bit words."""
    x = [np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3)]
    x = np.broadcast_arrays(*x)
    x = [a.copy() for a in x]
    ka, kb = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for r in range(10):
        if r:
            ka = (ka + W0) & 0xFFFFFFFF
            kb = (kb + W1) & 0xFFFFFFFF
        p0 = x[0] * M0          # < 2^64: both factors < 2^32
        p1 = x[2] * M1
        x = [(p1 >> np.uint64(32)) ^ x[1] ^ np.uint64(ka), p1 & MASK32,
             (p0 >> np.uint64(32)) ^ x[3] ^ np.uint64(kb), p0 & MASK32]
    return x


def threshold(p):
    """Drop threshold of the 16-bit draws for a float32 dropout probability
    p in [0, 1)."""
    p = float(np.float32(p))
    return min(int(np.ceil(p * 2.0 ** 16)), 2 ** 16) if p > 0 else 0


def keep_scale(p):
    """Factor of a kept weight: 2^16 / (2^16 - thr), the inverse of the keep
    probability the threshold realises (0 when every weight is dropped)."""
    thr = threshold(p)
    return 0.0 if thr >= 2 ** 16 else 2.0 ** 16 / (2 ** 16 - thr)


def keep_mask(n, Tq, Tk, p, seed, stream=0):
    """Boolean [Tq, Tk] keep mask of head-problem n."""
    if p <= 0:
        return np.ones((Tq, Tk), dtype=bool)
    i = np.arange(Tq, dtype=np.uint64)[:, None]
    j = np.arange(Tk, dtype=np.uint64)[None, :]
    words = philox4x32_10(j >> np.uint64(2), i >> np.uint64(1), np.uint64(n), np.uint64(stream),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    sel = (j & np.uint64(3)).astype(np.int64)
    w = np.choose(np.broadcast_to(sel, (Tq, Tk)), [np.broadcast_to(w, (Tq, Tk)) for w in words])
    x = (w >> (np.uint64(16) * (i & np.uint64(1)))) & np.uint64(0xFFFF)
    return x >= np.uint64(threshold(p))
