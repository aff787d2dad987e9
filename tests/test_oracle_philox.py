"""Pins for the oracle's Philox4x32-10 (oracle/philox.py).

* rocRAND's implementation of the same bijection, compiled from its ROCm header, must agree
  word for word on random and edge counters/keys (an independent implementation of the
  SC'11 definition);
* the published known-answer input (counter = key = 0) and the pi-digits input must agree
  with rocRAND too (checked through the same program, no stored values);
* the 64-bit uniforms and their exponentials: E = -ln U against a 40-digit decimal
  evaluation (both branches, the extremes of the grid: no E is 0 or infinite);
* the derived variates are exponential / uniform (KS, chi-square) and pairwise independent.
"""
import math
import os
import shutil
import subprocess
from decimal import Decimal, getcontext

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


@pytest.fixture(scope="module")
def rocrand_pin(tmp_path_factory):
    if not (shutil.which("g++") and os.path.exists(HEADER)):
        pytest.skip("g++ or the rocRAND header is missing")
    exe = str(tmp_path_factory.mktemp("pin") / "philox_pin")
    subprocess.run(["g++", "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    os.path.join(HERE, "pins", "rocrand_philox_pin.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(rows):
        text = "".join(" ".join(f"{int(v):08x}" for v in r) + "\n" for r in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
        return np.array([[int(w, 16) for w in line.split()]
                         for line in out.stdout.strip().splitlines()], dtype=np.uint64)
    return run


def test_bijection_matches_rocrand(rocrand_pin):
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 2 ** 32, size=(3000, 6), dtype=np.uint64)
    edge = np.array([[0, 0, 0, 0, 0, 0],
                     [0xFFFFFFFF] * 6,
                     [0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344, 0xA4093822, 0x299F31D0],
                     [1, 0, 0, 0, 0, 0], [0, 0, 0, 1, 0, 0], [0, 0, 0, 0, 0, 1]],
                    dtype=np.uint64)
    rows = np.concatenate([edge, rows])
    expect = rocrand_pin(rows)
    got = np.stack(philox.philox4x32_10(*[rows[:, i] for i in range(6)]), axis=1)
    assert np.array_equal(got, expect)


def test_stream_words_match_rocrand(rocrand_pin):
    """Race words of id j are words 2 (j & 1) and 2 (j & 1) + 1 of block (j >> 1, position,
    b, tag 1); the acceptance uniform takes words 0 and 1 of block (0, position, b, 0)."""
    seed = 0x0123456789ABCDEF
    j = np.arange(0, 4099, dtype=np.uint64)
    hi, lo = philox.race_words(seed, 5, 777, j)
    rows = [[int(x) >> 1, 777, 5, 1, seed & 0xFFFFFFFF, seed >> 32] for x in j]
    blocks = rocrand_pin(rows)
    sel = (j & 1).astype(np.int64) * 2
    assert np.array_equal(hi, blocks[np.arange(j.size), sel])
    assert np.array_equal(lo, blocks[np.arange(j.size), sel + 1])
    acc = rocrand_pin([[0, 99, 3, 0, seed & 0xFFFFFFFF, seed >> 32]])[0]
    u = philox.acceptance_uniform(seed, 3, 99)
    assert u == (float(acc[0]) + (float(acc[1]) + 0.5) * 2.0 ** -32) * 2.0 ** -32


def _exact_e(hi, lo):
    """-ln U for U = (hi 2^32 + lo + 1/2) 2^-64, in 40-digit decimal arithmetic."""
    getcontext().prec = 40
    u = (Decimal(int(hi)) * Decimal(2) ** 32 + Decimal(int(lo)) + Decimal("0.5")) / \
        Decimal(2) ** 64
    return -u.ln()


def test_exponentials_against_decimal_reference():
    """E = -ln U is within a few fp64 ulps of a 40-digit evaluation over random words and
    the extremes of both branches (U near 0, near 1/2 from both sides, near 1)."""
    rng = np.random.default_rng(3)
    m = 0xFFFFFFFF
    pairs = [(0, 0), (0, 1), (0, m), (1, 0), (m, m), (m, m - 1), (m, 0), (m - 1, m),
             (2 ** 31 - 1, m), (2 ** 31, 0), (2 ** 31, 1), (2 ** 31 - 1, m - 1)]
    pairs += [tuple(int(v) for v in rng.integers(0, 2 ** 32, size=2)) for _ in range(300)]
    pairs += [(m - int(d), int(rng.integers(0, 2 ** 32))) for d in range(40)]
    hi = np.array([p[0] for p in pairs], dtype=np.uint64)
    lo = np.array([p[1] for p in pairs], dtype=np.uint64)
    e = philox.exponential64(hi, lo)
    for k, (h, l_) in enumerate(pairs):
        ref = _exact_e(h, l_)
        assert abs(Decimal(float(e[k])) - ref) <= Decimal(4e-16) * ref, (h, l_, e[k], ref)
    # the extremes: U = 2^-65 gives 65 ln 2; U = 1 - 2^-65 gives 2^-65 (no zero, no infinity)
    assert philox.uniform64(0, 0) == 2.0 ** -65
    assert philox.exponential64(np.uint64(m), np.uint64(m)) == 2.0 ** -65
    assert abs(philox.exponential64(np.uint64(0), np.uint64(0)) - 65 * math.log(2)) < 1e-13


def test_uniforms_ranges_and_uniformity():
    e = philox.race_exponentials(3, 1, 10, np.arange(200000, dtype=np.uint64))
    assert np.all(np.isfinite(e)) and e.min() > 0.0
    assert stats.kstest(e, "expon").pvalue > 1e-4
    u = np.exp(-e)
    hist = np.histogram(u, bins=64, range=(0.0, 1.0))[0]
    assert stats.chisquare(hist).pvalue > 1e-4
    acc = np.array([philox.acceptance_uniform(11, 0, p) for p in range(20000)])
    assert acc.min() > 0.0 and acc.max() < 1.0
    assert stats.chisquare(np.histogram(acc, bins=32, range=(0, 1))[0]).pvalue > 1e-4


def test_pairwise_independence():
    u = np.exp(-philox.race_exponentials(9, 2, 3, np.arange(131072, dtype=np.uint64)))
    a, b = u[0::2], u[1::2]
    h = np.histogram2d(a, b, bins=8, range=[[0, 1], [0, 1]])[0].ravel()
    assert stats.chisquare(h).pvalue > 1e-4
    # distinct streams (positions, sequences, tags) are not copies of one another
    v = np.exp(-philox.race_exponentials(9, 2, 4, np.arange(4096, dtype=np.uint64)))
    w = np.exp(-philox.race_exponentials(9, 3, 3, np.arange(4096, dtype=np.uint64)))
    assert abs(np.corrcoef(u[:4096], v)[0, 1]) < 0.06
    assert abs(np.corrcoef(u[:4096], w)[0, 1]) < 0.06
