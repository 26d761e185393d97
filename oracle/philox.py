"""Philox4x32-10 and the dropout keep-mask built on it (fp64 oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages put dropout inside the fused attention operation (inferensys.com
glossary "FlashAttention", the paragraph on the single fused kernel: matrix
multiply, softmax, dropout and masking in one pass) but fix no random number
generator.  Reading taken here: the mask is drawn from the
counter-based generator Philox4x32-10 of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011), implemented from
that definition:

  state: four 32-bit counter words (c0, c1, c2, c3), key (k0, k1)
  one round, with M0 = 0xD2511F53 and M1 = 0xCD9E8D57:
      (hi0, lo0) = 64-bit product M0 * c0,  (hi1, lo1) = M1 * c2
      (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
  ten rounds; between consecutive rounds the key advances by the Weyl
  constants (k0 += 0x9E3779B9, k1 += 0xBB67AE85, modulo 2^32).

Dropout element (b, h, i, j) -- batch entry or packed sequence b, query head
h, query row i (inside its sequence), key j -- takes one 16-bit slot of a
call; one call serves eight keys of a row:

  counter = (2 * (j >> 4) + ((j >> 2) & 1), i, h, b),
  key     = (seed mod 2^32, seed >> 32),
  slot    = 4 * ((j >> 3) & 1) + (j & 3)   (0..7),
  u       = 16-bit half (slot & 1: 0 low, 1 high) of output word slot >> 1.

So the keys 16m + 4t + {0, 1, 2, 3, 8, 9, 10, 11} (t = 0, 1) share a call.
With T = floor(p * 2^16) (p in [0, 1)), a key is kept iff u >= T; the keep
probability is then exactly 1 - T / 2^16, and kept probabilities are scaled
by 2^16 / (2^16 - T), its inverse (1 / (1 - p) up to p's rounding to
multiples of 2^-16), so that the dropped output stays unbiased.  Pinned by
the generator's published known-answer vectors and by the statistics of the
mask (tests/oracle_pins.py).
"""

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10: counter words and key words as integer arrays
    (broadcast together), returns the four 32-bit output words (uint64 arrays
    holding values < 2^32)."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
        p0 = np.uint64(M0) * c[0]  # < 2^64: exact in uint64
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def drop_threshold(p):
    """16-bit threshold T = floor(p * 2^16): a key is dropped iff its slot < T."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(p * 65536.0)


def keep_scale(p):
    """Scale of the kept probabilities, 2^16 / (2^16 - T): the inverse of the
    exact keep probability."""
    return 65536.0 / (65536.0 - drop_threshold(p))


def slot_words(j):
    """(counter word c0, output word, half) of key j, as integer arrays."""
    j = np.asarray(j, dtype=np.int64)
    c0 = 2 * (j >> 4) + ((j >> 2) & 1)
    slot = 4 * ((j >> 3) & 1) + (j & 3)
    return c0, slot >> 1, slot & 1


def keep_mask(seed, b, h, rows, nk, p):
    """Boolean [len(rows), nk]: which keys query rows `rows` of (b, h) keep."""
    rows = np.asarray(rows, dtype=np.int64)
    c0, word, half = slot_words(np.arange(nk, dtype=np.int64))
    words = philox4x32_10(c0[None, :], rows[:, None], h, b,
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = word[None, :]
    u = np.select([w == 0, w == 1, w == 2, w == 3], words)
    u16 = (u >> (np.uint64(16) * half[None, :].astype(np.uint64))) & np.uint64(0xFFFF)
    return u16 >= np.uint64(drop_threshold(p))
