"""Philox4x32-10 counter-based RNG and the per-element SR draw (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages only say that SR is on by default ([Lighthouse] §3.1); they name no
generator.  Reading taken: the random bits for element `idx` of a tensor come
from Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11), keyed by the 64-bit seed, so that the
draw depends only on (seed, stream, idx) and never on how the work is tiled.

Definition used here (written from the SC'11 description of the Philox
S-box/P-box round):

* key  = (seed mod 2^32, seed >> 32)
* ctr  = (g mod 2^32, g >> 32, stream, 0) with g = idx >> 3
* one round: multiply word 0 by M0 and word 2 by M1 (32x32->64 bit), then the
  new words are (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0))
* between rounds the key advances by the Weyl constants (W0, W1)
* M0 = 0xD2511F53, M1 = 0xCD9E8D57, W0 = 0x9E3779B9, W1 = 0xBB67AE85
* one call yields 4 x 32 bits = 8 draws of 16 bits: element idx takes word
  (idx >> 1) & 3 and its low (idx even) or high (idx odd) 16-bit half.

Streams: 0 = residual and vanilla activations, 1 = mean vector, 2 = weights.
Pinned against rocRAND's independent Philox4x32-10 engine in the tests.
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on arrays of counters; returns four uint32 arrays.

    c0..c3: uint32-valued arrays (broadcastable); k0, k1: Python ints.
    """
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = int(k0) & MASK32
    k1 = int(k1) & MASK32
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = c0 * np.uint64(M0)          # < 2^64, exact in uint64
        p1 = c2 * np.uint64(M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        n0 = hi1 ^ c1 ^ np.uint64(k0)
        n2 = hi0 ^ c3 ^ np.uint64(k1)
        c0, c1, c2, c3 = n0, lo1, n2, lo0
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def sr_draw16(seed, stream, idx):
    """16-bit uniform draw u in [0, 65536) for each logical element index.

    seed: 64-bit int; stream: small int; idx: integer array of element
    indices (row * cols + col of the tensor being quantized).
    """
    idx = np.asarray(idx, dtype=np.uint64)
    g = idx >> np.uint64(3)
    out = philox4x32_10(g & np.uint64(MASK32), g >> np.uint64(32),
                        np.uint64(stream), np.uint64(0),
                        seed & MASK32, (seed >> 32) & MASK32)
    words = np.stack(out, axis=-1)                       # (..., 4)
    w = ((idx >> np.uint64(1)) & np.uint64(3)).astype(np.intp)
    word = np.take_along_axis(words, w[..., None], axis=-1)[..., 0]
    half = (idx & np.uint64(1)).astype(np.uint32)
    return ((word >> (np.uint32(16) * half)) & np.uint32(0xFFFF)).astype(np.uint32)
