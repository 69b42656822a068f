"""Philox4x64-10, the counter-based generator behind stochastic rounding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC 2011, the Philox-4x64 bijection with 10 rounds): a 256-bit counter
(x0, x1, x2, x3) and a 128-bit key (k0, k1); each round multiplies x0 and x2 by
the constants M0, M1 into 128-bit products (hi, lo) and sets
    (x0, x1, x2, x3) <- (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0),
then bumps the key by the Weyl constants W0, W1.  All arithmetic is modulo 2^64.

Stochastic rounding draws one 32-bit half-word per element: element at
position `pos` of output row `row` in stream `stream` (0 for a row-direction
output, 1 for a column-direction output) takes
    words = philox(counter=(pos >> 3, row, stream, 0), key=(seed, 0))
    w = words[(pos >> 1) & 3];  bits = high half of w if pos is odd, else low half
and its uniform is (bits >> 8) * 2^-24.
"""

from __future__ import annotations

import numpy as np

M0, M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
W0, W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
_MASK = (1 << 64) - 1


def philox4x64_scalar(ctr, key, rounds: int = 10) -> tuple[int, int, int, int]:
    """The bijection on Python integers, written as defined."""
    x0, x1, x2, x3 = (int(c) & _MASK for c in ctr)
    k0, k1 = (int(k) & _MASK for k in key)
    for _ in range(rounds):
        p0, p1 = M0 * x0, M1 * x2
        hi0, lo0 = p0 >> 64, p0 & _MASK
        hi1, lo1 = p1 >> 64, p1 & _MASK
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
        k0, k1 = (k0 + W0) & _MASK, (k1 + W1) & _MASK
    return x0, x1, x2, x3


def _mulhilo(a: np.ndarray, m: int) -> tuple[np.ndarray, np.ndarray]:
    """128-bit product of uint64 arrays with a constant, from 32-bit halves."""
    a = a.astype(np.uint64)
    lo32 = np.uint64(0xFFFFFFFF)
    al, ah = a & lo32, a >> np.uint64(32)
    ml, mh = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    ll, lh, hl, hh = al * ml, al * mh, ah * ml, ah * mh
    mid = (ll >> np.uint64(32)) + (lh & lo32) + (hl & lo32)
    lo = (ll & lo32) | ((mid & lo32) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64(c0, c1, c2, c3, k0, k1, rounds: int = 10) -> tuple[np.ndarray, ...]:
    """The same bijection on uint64 arrays (broadcast), modulo 2^64 throughout."""
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
        x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
        ka = np.uint64(int(k0) & _MASK)
        kb = np.uint64(int(k1) & _MASK)
        for _ in range(rounds):
            hi0, lo0 = _mulhilo(x0, M0)
            hi1, lo1 = _mulhilo(x2, M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ ka, lo1, hi0 ^ x3 ^ kb, lo0
            ka = ka + np.uint64(W0)
            kb = kb + np.uint64(W1)
    return x0, x1, x2, x3


def uniform24(rows: np.ndarray, pos: np.ndarray, stream: int, seed: int) -> np.ndarray:
    """24-bit integer uniforms (0 .. 2^24 - 1) of the elements at (rows, pos)."""
    rows = np.asarray(rows, dtype=np.uint64)
    pos = np.asarray(pos, dtype=np.uint64)
    rows, pos = np.broadcast_arrays(rows, pos)
    w = philox4x64(pos >> np.uint64(3), rows, np.uint64(stream), np.uint64(0), seed, 0)
    words = np.stack(w, axis=0)                                   # [4, ...]
    sel = ((pos >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(words, sel[None], axis=0)[0]
    half = np.where((pos & np.uint64(1)) == 1, word >> np.uint64(32), word & np.uint64(0xFFFFFFFF))
    return (half >> np.uint64(8)).astype(np.uint32)
