"""Philox4x32-10 counter-based random numbers, written from its published definition.

TEST INFRASTRUCTURE: part of the CPU oracle. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.

Source of the algorithm: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 (the Philox-4x32 S-box with
R = 10 rounds, multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key increments
0x9E3779B9 / 0xBB67AE85).

How the verify step draws its randoms (a reading: the pages say only that sampled output is
an exact sample of the target, mlx-dspark release v0.0.2, "Highlights" and release v0.1.0,
"Highlights", and that requests carry a seed; keying every draw by seed, sequence index and
absolute token position means no variate is reused within a generation):
  key      = (seed & 0xffffffff, seed >> 32)
  counter  = (block, position, sequence index b, tag)
  tag 0    : the acceptance uniform of a drafted position: block 0, words (w0, w1)
  tag 1    : the exponential variates of a categorical draw over token ids j: block j >> 1,
             words (w[2 (j & 1)], w[2 (j & 1) + 1])
Both are 64-bit uniforms on the open interval (0, 1), the midpoints of a 2^-64 grid:
  U = (hi * 2^32 + lo + 1/2) * 2^-64
so no variate is 0 or 1 (an exponential E = -ln U is then finite and positive, and no id
can take an infinite race key whatever its weight). In fp64, U is evaluated as
  ((double) hi + ((double) lo + 0.5) * 2^-32) * 2^-32          (one rounding, in the sum)
and E, near U = 1, through the complement c = 1 - U, which the same formula gives exactly
from the bitwise complements of the two words: E = -log1p(-c).
Everything here is vectorised numpy over uint64 lanes holding 32-bit values.
"""
import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)
_2M32 = 2.0 ** -32

TAG_ACCEPT = 0
TAG_RACE = 1


def _u32(x):
    return np.asarray(x, dtype=np.uint64) & _MASK


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """The Philox4x32-10 bijection on counters (c0..c3) under key (k0, k1).

    One round maps (c0, c1, c2, c3) to
      (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)),
    and the key is bumped by the Weyl constants between rounds (ten rounds, nine bumps).
    Inputs broadcast; returns four uint64 arrays holding 32-bit words.
    """
    c0, c1, c2, c3 = np.broadcast_arrays(*(_u32(v) for v in (c0, c1, c2, c3)))
    c0, c1, c2, c3 = (np.array(v, dtype=np.uint64) for v in (c0, c1, c2, c3))
    k0, k1 = _u32(k0), _u32(k1)
    p0, p1 = np.empty_like(c0), np.empty_like(c0)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        np.multiply(c0, _M0, out=p0)          # < 2^64: both factors < 2^32
        np.multiply(c2, _M1, out=p1)
        # (c0, c1, c2, c3) <- (hi(p1) ^ c1 ^ k0, lo(p1), hi(p0) ^ c3 ^ k1, lo(p0))
        np.right_shift(p1, _S32, out=c0)
        c0 ^= c1
        c0 ^= k0
        np.bitwise_and(p1, _MASK, out=c1)
        np.right_shift(p0, _S32, out=c2)
        c2 ^= c3
        c2 ^= k1
        np.bitwise_and(p0, _MASK, out=c3)
    return c0, c1, c2, c3


def _key(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def block_words(seed, b, position, tag, block):
    """The four 32-bit words of counter (block, position, b, tag) under the seed; `block`
    may be an array. Returns a [4, n] uint64 array."""
    k0, k1 = _key(seed)
    return np.stack(philox4x32_10(np.asarray(block, dtype=np.uint64),
                                  int(position) & 0xFFFFFFFF, int(b) & 0xFFFFFFFF,
                                  int(tag) & 0xFFFFFFFF, k0, k1))


def uniform64(hi, lo):
    """U = (hi 2^32 + lo + 1/2) 2^-64 in fp64, in (0, 1)."""
    hi = np.asarray(hi, dtype=np.uint64).astype(np.float64)
    lo = np.asarray(lo, dtype=np.uint64).astype(np.float64)
    return (hi + (lo + 0.5) * _2M32) * _2M32


def exponential64(hi, lo):
    """E = -ln U for the 64-bit uniform of (hi, lo): -ln U directly while U < 1/2 (hi below
    2^31), else -log1p(-c) with c = 1 - U formed from the complemented words."""
    hi = np.asarray(hi, dtype=np.uint64)
    lo = np.asarray(lo, dtype=np.uint64)
    u = uniform64(hi, lo)
    c = uniform64(hi ^ _MASK, lo ^ _MASK)          # 1 - U, exactly as the same formula
    low = hi < np.uint64(1 << 31)
    with np.errstate(divide="ignore"):
        return np.where(low, -np.log(u), -np.log1p(-c))


def race_words(seed, b, position, j):
    """(hi, lo) words of token ids j (array) in the tag-1 stream of (seed, b, position)."""
    j = np.asarray(j, dtype=np.uint64).ravel()
    if j.size == 0:
        return j.copy(), j.copy()
    blk = (j >> np.uint64(1)).astype(np.int64)
    b0, b1 = int(blk.min()), int(blk.max())
    w = block_words(seed, b, position, TAG_RACE, np.arange(b0, b1 + 1, dtype=np.uint64))
    idx = blk - b0
    odd = (j & np.uint64(1)).astype(bool)
    return (np.where(odd, w[2][idx], w[0][idx]), np.where(odd, w[3][idx], w[1][idx]))


def race_exponentials(seed, b, position, j):
    """E_j = -ln U_j, the standard exponentials of token ids j for the categorical draw of
    (seed, b, position), fp64, all finite and > 0."""
    return exponential64(*race_words(seed, b, position, j))


def acceptance_uniform(seed, b, position):
    """U in (0, 1) used to accept the draft at absolute token index `position`."""
    w = block_words(seed, b, position, TAG_ACCEPT, 0)
    return float(uniform64(w[0], w[1]))
