"""Philox4x32-10 counter-based random numbers, written from its published definition.

TEST INFRASTRUCTURE: part of the CPU oracle. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.

Source of the algorithm: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 (the Philox-4x32 S-box with
R = 10 rounds, multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key increments
0x9E3779B9 / 0xBB67AE85).

How the verify step draws its randoms (a reading: the pages say only that sampled output is
an exact sample of the target, mlx-dspark release v0.0.2, "Highlights", and that requests
carry a seed, release v0.1.0, "Highlights"; keying every draw by seed, sequence index and
absolute token position means no variate is reused within a generation):
  key      = (seed & 0xffffffff, seed >> 32)
  counter  = (j >> 2, position, sequence index b, tag)
  word     = j & 3 of the four output words
  tag 0    : the acceptance uniform of a drafted position (j = 0)
  tag 1    : the exponential-race variates of a categorical draw over token ids j
  U  = (word >> 8) * 2^-24          in [0, 1)   (acceptance)
  U' = ((word >> 8) + 1) * 2^-24    in (0, 1]   (race; E = -ln U')
Everything here is vectorised numpy over uint64 lanes holding 32-bit values.
"""
import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

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
    c0, c1, c2, c3 = (_u32(v) for v in (c0, c1, c2, c3))
    k0, k1 = _u32(k0), _u32(k1)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0          # < 2^64: both factors < 2^32
        p1 = _M1 * c2
        hi0, lo0 = p0 >> _S32, p0 & _MASK
        hi1, lo1 = p1 >> _S32, p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def _key(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def random_words(seed, b, position, tag, j):
    """32-bit word for token slot j (array) of stream (seed, b, position, tag)."""
    j = np.asarray(j, dtype=np.uint64)
    k0, k1 = _key(seed)
    words = philox4x32_10(j >> np.uint64(2), int(position) & 0xFFFFFFFF,
                          int(b) & 0xFFFFFFFF, int(tag) & 0xFFFFFFFF, k0, k1)
    sel = (j & np.uint64(3)).astype(np.int64)
    return np.choose(sel, words)


def acceptance_uniform(seed, b, position):
    """U in [0,1) used to accept the draft at absolute token index `position`."""
    w = int(random_words(seed, b, position, TAG_ACCEPT, np.uint64(0)))
    return (w >> 8) * 2.0 ** -24


def race_uniforms(seed, b, position, j):
    """U' in (0,1] for token ids j of the categorical draw at `position` (fp64)."""
    w = random_words(seed, b, position, TAG_RACE, j)
    return ((w >> np.uint64(8)).astype(np.float64) + 1.0) * 2.0 ** -24
