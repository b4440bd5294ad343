"""Random feature matrices drawn from a seed: plain float64 CPU reference.

TEST INFRASTRUCTURE.  Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import or call this module.  It shares no code with the library.

What it computes, and where that is defined
-------------------------------------------
"Rethinking Attention with Performers" (review page), section "제안 방법": the softmax
kernel is estimated with random features whose rows are made orthogonal (orthogonal
random features, ORF) to lower the estimator's variance.  Redrawing W from a seed on the
device needs random numbers that both sides can produce from the seed alone, so the
stream is a counter-based generator taken from its published definition:

* Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
  3", SC 2011): a 128-bit counter and a 64-bit key; ten rounds, each multiplying counter
  words 0 and 2 by the round constants 0xD2511F53 and 0xCD9E8D57 into 64-bit products and
  mixing the high halves with the other two words and the key, the key advanced by
  (0x9E3779B9, 0xBB67AE85) between rounds.  Pinned by the authors' known-answer vectors
  (tests/golden/philox4x32_10_kat.txt).
* Gaussians by the Box-Muller transform (Box and Muller, 1958) on two 53-bit uniforms.

The numbering (a reading; the pages fix no generator): Gaussian number e of the stream
fills G[h][b][i][j] (head h, block b of d rows, row i, column j) with
e = ((h * nblocks + b) * d + i) * d + j.  Pair p = e // 2 is one Philox call with counter
(p mod 2^32, p div 2^32, 0, 0) and key (seed mod 2^32, seed div 2^32), giving words
r0..r3; u1 = ((r1 r0 as a 64-bit number >> 11) + 1) / 2^53 in (0, 1],
u2 = (r3 r2 >> 11) / 2^53 in [0, 1), radius sqrt(-2 ln u1); an even e takes
radius cos(2 pi u2), an odd e radius sin(2 pi u2).

ORF (orthogonal): per block, modified Gram-Schmidt on the rows of G in row order, each
orthonormal row then scaled by the length of the same row of G (chi(d)-distributed, so
every row is marginally N(0, I_d)); i.i.d.: the rows of G as they are.  Rows past m in the
last block are dropped.
"""
from __future__ import annotations

import numpy as np

__all__ = ["philox4x32_10", "gaussian_stream", "draw_features"]

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 on arrays of counters: counter (c0, c1, c2, c3), key (k0, k1), each
    word an integer or uint array; returns the four 32-bit output words as uint64 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in counter]
    k0, k1 = (np.asarray(x, dtype=np.uint64) & _MASK for x in key)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_W0)) & _MASK
            k1 = (k1 + np.uint64(_W1)) & _MASK
        p0 = np.uint64(_M0) * c[0]  # < 2^64: no wrap-around
        p1 = np.uint64(_M1) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & _MASK, (p0 >> np.uint64(32)) ^ c[3] ^ k1, p0 & _MASK]
    return c


def gaussian_stream(seed, first, count):
    """Gaussian numbers first .. first+count-1 of the stream of `seed` (float64)."""
    seed = int(seed)
    e = np.arange(first, first + count, dtype=np.uint64)
    p = e >> np.uint64(1)
    r0, r1, r2, r3 = philox4x32_10((p & _MASK, p >> np.uint64(32), 0, 0),
                                   (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    a = ((r1 << np.uint64(32)) | r0) >> np.uint64(11)
    b = ((r3 << np.uint64(32)) | r2) >> np.uint64(11)
    u1 = (a.astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = b.astype(np.float64) * 2.0 ** -53
    radius = np.sqrt(-2.0 * np.log(u1))
    angle = 2.0 * np.pi * u2
    return np.where((e & np.uint64(1)) == 0, radius * np.cos(angle), radius * np.sin(angle))


def draw_features(heads_w, m, d, seed, orthogonal=True):
    """W of shape (heads_w, m, d), float64, drawn from `seed` as described above."""
    nblk = (m + d - 1) // d
    W = np.empty((heads_w, nblk * d, d))
    for h in range(heads_w):
        for b in range(nblk):
            g = gaussian_stream(seed, (h * nblk + b) * d * d, d * d).reshape(d, d)
            if not orthogonal:
                W[h, b * d:(b + 1) * d] = g
                continue
            q = g.copy()
            for i in range(d):
                for j in range(i):
                    q[i] = q[i] - np.dot(q[i], q[j]) * q[j]
                q[i] = q[i] / np.sqrt(np.dot(q[i], q[i]))
            W[h, b * d:(b + 1) * d] = q * np.sqrt(np.sum(g * g, axis=1))[:, None]
    return W[:, :m]
