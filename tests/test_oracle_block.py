"""Pins of the windowed block-attention oracle (CPU): a hand-worked example, closed forms,
and reductions of every window and mask form to the plain verify definition over a
shifted cache or a single row (which other pins tie to the mathematics)."""
import math

import numpy as np
import pytest

from oracle.attention import block_attention, block_visible_range, verify_attention


def _problem(seed, ctxs, rows, hq=4, hkv=2, d=16, s_max=None):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    s_max = s_max or max(c + r for c, r in zip(ctxs, rows)) + 3
    q = rng.standard_normal((int(cu[-1]), hq, d)).astype(np.float32)
    k = rng.standard_normal((len(ctxs), hkv, s_max, d)).astype(np.float32)
    v = rng.standard_normal((len(ctxs), hkv, s_max, d)).astype(np.float32)
    return q, k, v, cu, np.asarray(ctxs, dtype=np.int32), hq, hkv


def test_hand_worked_windows_and_masks():
    # one head, D = 1, scale 1, q = 1: the score of key t is k_t. Context keys 0, 1, block
    # keys 2, 3. Key 0 (score 5, value 100) would dominate any row that sees it.
    q = np.ones((2, 1, 1), dtype=np.float32)
    kc = np.array([5.0, 0.0, math.log(3.0), 0.0], dtype=np.float32).reshape(1, 1, 4, 1)
    vc = np.array([100.0, 4.0, 8.0, 12.0], dtype=np.float32).reshape(1, 1, 4, 1)
    cu, ctx = np.array([0, 2]), np.array([2])
    run = lambda **kw: block_attention(q, kc, vc, cu, ctx, 1, 1, scale=1.0, **kw)[:, 0, 0]
    # recent window of 1 context row: row 0 sees keys 1..2 (weights 1/4, 3/4 -> 7), row 1
    # keys 1..3 (1/5, 3/5, 1/5 -> 8)
    assert np.allclose(run(window=1), [7.0, 8.0], rtol=1e-6)
    # bidirectional: both rows see keys 1..3
    assert np.allclose(run(window=1, bidirectional=True), [8.0, 8.0], rtol=1e-6)
    # sliding window of 2 ending at each row: keys 1..2 (7) and 2..3 (3/4, 1/4 -> 9)
    assert np.allclose(run(window=2, sliding=True), [7.0, 9.0], rtol=1e-6)
    # key 0 (score 5, the others at most ln 3) dominates a row that sees it
    assert np.all(run() > 90.0)


def test_visible_ranges_by_hand():
    assert block_visible_range(10, 4, 0) == (0, 10)
    assert block_visible_range(10, 4, 3, bidirectional=True) == (0, 13)
    assert block_visible_range(10, 4, 2, window=4) == (6, 12)
    assert block_visible_range(10, 4, 2, window=4, sliding=True) == (9, 12)
    assert block_visible_range(3, 4, 1, window=8) == (0, 4)
    assert block_visible_range(3, 4, 1, window=8, sliding=True) == (0, 4)
    assert block_visible_range(10, 4, 0, window=1, sliding=True) == (10, 10)


def test_defaults_are_the_verify_definition():
    p = _problem(1, [0, 17, 40], [3, 1, 5])
    assert np.array_equal(block_attention(*p), verify_attention(*p))


def test_sliding_window_of_one_returns_own_value():
    q, k, v, cu, ctx, hq, hkv = _problem(2, [5, 30], [4, 2])
    out = block_attention(q, k, v, cu, ctx, hq, hkv, window=1, sliding=True)
    group = hq // hkv
    for b in range(2):
        for i in range(cu[b + 1] - cu[b]):
            for h in range(hq):
                assert np.array_equal(out[cu[b] + i, h], v[b, h // group, ctx[b] + i])


@pytest.mark.parametrize("window", [6, 25, 64])
def test_recent_window_is_verify_over_shifted_cache(window):
    q, k, v, cu, ctx, hq, hkv = _problem(3, [3, 20, 50], [2, 4, 6])
    got = block_attention(q, k, v, cu, ctx, hq, hkv, window=window)
    k2, v2 = np.zeros_like(k), np.zeros_like(v)
    ctx2 = ctx.copy()
    for b in range(len(ctx)):
        lo = max(0, int(ctx[b]) - window)
        n = k.shape[2] - lo
        k2[b, :, :n], v2[b, :, :n] = k[b, :, lo:], v[b, :, lo:]
        ctx2[b] = ctx[b] - lo
    assert np.array_equal(got, verify_attention(q, k2, v2, cu, ctx2, hq, hkv))


@pytest.mark.parametrize("bidirectional", [False, True])
@pytest.mark.parametrize("window", [1, 3, 16])
def test_each_row_is_one_verify_row(window, bidirectional):
    """Every row of every form equals a one-row verify problem: the query alone, over the
    cache shifted to its first visible key, with context up to its last visible key."""
    q, k, v, cu, ctx, hq, hkv = _problem(4, [0, 9, 33], [5, 3, 7])
    for sliding in (False, True):
        got = block_attention(q, k, v, cu, ctx, hq, hkv, window=window, sliding=sliding,
                              bidirectional=bidirectional)
        for b in range(len(ctx)):
            rows = int(cu[b + 1] - cu[b])
            for i in range(rows):
                lo, hi = block_visible_range(int(ctx[b]), rows, i, window, sliding,
                                             bidirectional)
                ref = verify_attention(q[cu[b] + i:cu[b] + i + 1], k[b:b + 1, :, lo:],
                                       v[b:b + 1, :, lo:], np.array([0, 1]),
                                       np.array([hi - lo]), hq, hkv)
                assert np.array_equal(got[cu[b] + i], ref[0]), (b, i, sliding)


def test_window_covering_everything_is_no_window():
    p = _problem(5, [7, 12], [3, 6])
    ref = block_attention(*p)
    assert np.array_equal(block_attention(*p, window=12), ref)
    assert np.array_equal(block_attention(*p, window=18, sliding=True), ref)
    refb = block_attention(*p, bidirectional=True)
    assert np.array_equal(block_attention(*p, window=40, bidirectional=True), refb)


def test_bidirectional_single_row_is_causal():
    p = _problem(6, [4, 0, 11], [1, 1, 1])
    assert np.array_equal(block_attention(*p, bidirectional=True), block_attention(*p))
