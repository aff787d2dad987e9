"""Pins for the oracle's Philox4x32-10 (oracle/philox.py).

* rocRAND's implementation of the same bijection, compiled from its ROCm header, must agree
  word for word on random and edge counters/keys (an independent implementation of the
  SC'11 definition);
* the published known-answer input (counter = key = 0) and the pi-digits input must agree
  with rocRAND too (checked through the same program, no stored values);
* the derived uniforms are uniform (chi-square) and pairwise independent.
"""
import os
import shutil
import subprocess

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
    """random_words picks word j&3 of the block (j>>2, position, b, tag) under the seed."""
    seed = 0x0123456789ABCDEF
    j = np.arange(0, 4099, dtype=np.uint64)
    got = philox.random_words(seed, 5, 777, philox.TAG_RACE, j)
    rows = [[int(x) >> 2, 777, 5, 1, seed & 0xFFFFFFFF, seed >> 32] for x in j]
    blocks = rocrand_pin(rows)
    assert np.array_equal(got, blocks[np.arange(j.size), (j & 3).astype(np.int64)])


def test_uniforms_ranges_and_uniformity():
    u = philox.race_uniforms(3, 1, 10, np.arange(200000, dtype=np.uint64))
    assert u.min() > 0.0 and u.max() <= 1.0
    hist = np.histogram(u, bins=64, range=(0.0, 1.0))[0]
    assert stats.chisquare(hist).pvalue > 1e-4
    acc = np.array([philox.acceptance_uniform(11, 0, p) for p in range(20000)])
    assert acc.min() >= 0.0 and acc.max() < 1.0
    assert stats.chisquare(np.histogram(acc, bins=32, range=(0, 1))[0]).pvalue > 1e-4


def test_pairwise_independence():
    u = philox.race_uniforms(9, 2, 3, np.arange(131072, dtype=np.uint64))
    a, b = u[0::2], u[1::2]
    h = np.histogram2d(a, b, bins=8, range=[[0, 1], [0, 1]])[0].ravel()
    assert stats.chisquare(h).pvalue > 1e-4
    # distinct streams (positions, sequences, tags) are not copies of one another
    v = philox.race_uniforms(9, 2, 4, np.arange(4096, dtype=np.uint64))
    w = philox.race_uniforms(9, 3, 3, np.arange(4096, dtype=np.uint64))
    assert abs(np.corrcoef(u[:4096], v)[0, 1]) < 0.06
    assert abs(np.corrcoef(u[:4096], w)[0, 1]) < 0.06
