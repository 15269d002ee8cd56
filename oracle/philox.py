"""Counter-based random numbers for the dropout reference (Philox).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Philox-4xW-R as defined by Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11), section 3.3: a block of four W-bit
counter words (c0, c1, c2, c3) and a key (k0, k1) go through R rounds of

    (hi0, lo0) = M0 * c0        (full 2W-bit product, high and low halves)
    (hi1, lo1) = M1 * c2
    (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)

with the key bumped by the Weyl constants (k0 += W0, k1 += W1, mod 2^W)
between rounds. The multipliers and Weyl constants are the published ones;
R = 10 is the paper's recommended round count. One call maps a 128-bit
counter to 128 random bits; nothing is stateful, so any element of a random
stream can be computed on its own, which is what lets a tiled kernel and this
plain reference draw identical dropout masks.

The dropout stream (``dropout_keep``): the keep decision for score element
(bh, i, j) of head bh = b * Hq + hq uses the 16-bit half j mod 2 (0: low
bits, 1: high bits) of the 32-bit word i mod 4 of Philox-4x32-10 with counter
(floor(j / 2), floor(i / 4), bh, offset) and key (seed mod 2^32,
floor(seed / 2^32)); the element is kept when that half is
>= T = floor(p * 2^16). It is dropped with probability exactly T / 2^16
(``effective_p``), the value the kept weights are rescaled by.
"""

from __future__ import annotations

import numpy as np

CONSTANTS = {
    32: dict(M0=0xD2511F53, M1=0xCD9E8D57, W0=0x9E3779B9, W1=0xBB67AE85),
    64: dict(M0=0xD2E7470EE14C6C93, M1=0xCA5A826395121157,
             W0=0x9E3779B97F4A7C15, W1=0xBB67AE8584CAA73B),
}


def _mulhilo(a, b, width):
    """High and low W-bit halves of the 2W-bit product a * b (object arrays
    of Python ints, exact for any W)."""
    prod = a * b
    mask = (1 << width) - 1
    return prod >> width, prod & mask


def philox(counter, key, rounds=10, width=32):
    """Philox-4xW-R of a block of counters.

    counter: 4 arrays (or ints) of W-bit words, broadcast together; key: 2
    words. Returns 4 arrays of W-bit words (dtype uint32 for W = 32, uint64
    for W = 64).
    """
    const = CONSTANTS[width]
    mask = (1 << width) - 1
    shape = np.broadcast(*[np.asarray(x) for x in counter]).shape
    c = [np.broadcast_to(np.asarray(x, dtype=object), shape).copy() for x in counter]
    c = [np.vectorize(lambda v: int(v) & mask, otypes=[object])(x) if x.size else x for x in c]
    k0, k1 = int(key[0]) & mask, int(key[1]) & mask
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + const["W0"]) & mask
            k1 = (k1 + const["W1"]) & mask
        hi0, lo0 = _mulhilo(c[0], const["M0"], width)
        hi1, lo1 = _mulhilo(c[2], const["M1"], width)
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    dt = np.uint32 if width == 32 else np.uint64
    return [np.asarray(x, dtype=dt).reshape(shape) for x in c]


def philox4x32(counter, key, rounds=10):
    """Philox-4x32-R with numpy uint64 arithmetic (a 32 x 32-bit product fits
    in 64 bits): the same function as philox(..., width=32), vectorised."""
    const = CONSTANTS[32]
    m32 = np.uint64(0xFFFFFFFF)
    shape = np.broadcast(*[np.asarray(x) for x in counter]).shape
    c = [np.broadcast_to(np.asarray(x).astype(np.uint64) & m32, shape) for x in counter]
    k0, k1 = np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF)
    M0, M1 = np.uint64(const["M0"]), np.uint64(const["M1"])
    W0, W1 = np.uint64(const["W0"]), np.uint64(const["W1"])
    s32 = np.uint64(32)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + W0) & m32
            k1 = (k1 + W1) & m32
        p0 = c[0] * M0
        p1 = c[2] * M1
        c = [(p1 >> s32) ^ c[1] ^ k0, p1 & m32, (p0 >> s32) ^ c[3] ^ k1, p0 & m32]
    return [x.astype(np.uint32) for x in c]


def keep_threshold(p: float) -> int:
    """floor(p * 2^16): 16-bit values below it are dropped. p is taken as the
    exact value it has (callers pass the float32 the kernels see)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(np.floor(np.float64(p) * 65536.0)), 65535)


def effective_p(p: float) -> float:
    """The drop probability the stream realises: keep_threshold(p) / 2^16."""
    return keep_threshold(p) / 65536.0


def dropout_keep(bh: int, rows, cols, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean keep mask [len(rows), len(cols)] of head bh (see the module
    docstring for the stream layout)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    t = keep_threshold(p)
    if t == 0:
        return np.ones((rows.size, cols.size), dtype=bool)
    i = rows[:, None]
    j = cols[None, :]
    words = philox4x32((j // 2, i // 4, np.int64(bh), np.int64(offset)),
                       (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF), rounds=10)
    w = np.choose((i % 4) * np.ones_like(j), words).astype(np.uint64)
    half = (w >> (16 * (j % 2)).astype(np.uint64)) & np.uint64(0xFFFF)
    return half >= t
