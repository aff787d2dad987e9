"""Pins for the oracle's verify attention (oracle/attention.py).

* torch's CPU scaled_dot_product_attention in fp64, with an explicit boolean causal mask and
  K/V tiled to one head per query head (repeat per group) -- a library routine, and the
  pages' statement that native-GQA attention equals explicit K/V tiling (mlx-dspark
  Changelog [0.3.1], "Fixed" and "Added");
* closed forms: a single visible key returns its value; constant values return that
  constant; identical keys return the mean of the visible values;
* causality: changing keys/values a row may not see leaves that row bit-identical;
* row isolation (Changelog [0.3.0], "Added": rows never influence each other).
"""
import math

import numpy as np
import torch

from oracle.attention import verify_attention


def _case(rng, ctx, rows, hq=4, hkv=2, d=16, s_max=None):
    batch = len(ctx)
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    s_max = s_max or int(max(c + r for c, r in zip(ctx, rows))) + 3
    q = rng.standard_normal((cu[-1], hq, d))
    k = rng.standard_normal((batch, hkv, s_max, d))
    v = rng.standard_normal((batch, hkv, s_max, d))
    return q, k, v, cu, np.asarray(ctx)


def _torch_reference(q, k, v, cu, ctx, hq, hkv):
    """fp64 SDPA per sequence with tiled K/V and an explicit [rows, keys] mask."""
    out = np.zeros(q.shape)
    group = hq // hkv
    for b in range(len(ctx)):
        r0, r1 = cu[b], cu[b + 1]
        n_all = ctx[b] + (r1 - r0)
        qq = torch.tensor(q[r0:r1]).permute(1, 0, 2)                        # [Hq, R, D]
        kk = torch.tensor(k[b, :, :n_all]).repeat_interleave(group, dim=0)  # [Hq, n, D]
        vv = torch.tensor(v[b, :, :n_all]).repeat_interleave(group, dim=0)
        mask = torch.zeros(r1 - r0, n_all, dtype=torch.bool)
        for i in range(r1 - r0):
            mask[i, :ctx[b] + i + 1] = True
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        out[r0:r1] = o.permute(1, 0, 2).numpy()
    return out


def test_matches_torch_sdpa_with_tiled_kv():
    rng = np.random.default_rng(0)
    for ctx, rows, hq, hkv, d in [([5, 0, 17], [3, 1, 6], 4, 2, 16),
                                  ([40], [9], 6, 1, 8),
                                  ([3, 9], [2, 4], 8, 8, 32)]:
        q, k, v, cu, c = _case(rng, ctx, rows, hq, hkv, d)
        got = verify_attention(q, k, v, cu, c, hq, hkv)
        ref = _torch_reference(q, k, v, cu, c, hq, hkv)
        np.testing.assert_allclose(got, ref, rtol=2e-6, atol=2e-6)


def test_default_and_explicit_scale():
    rng = np.random.default_rng(1)
    q, k, v, cu, c = _case(rng, [7], [3], 2, 1, 64)
    a = verify_attention(q, k, v, cu, c, 2, 1)
    b = verify_attention(q, k, v, cu, c, 2, 1, scale=1.0 / math.sqrt(64))
    assert np.array_equal(a, b)
    c2 = verify_attention(q * 2.0, k, v, cu, c, 2, 1, scale=0.5 / math.sqrt(64))
    assert np.allclose(a, c2, atol=1e-6)


def test_closed_forms():
    rng = np.random.default_rng(2)
    # ctx 0: row 0 sees exactly one key -> its value
    q, k, v, cu, c = _case(rng, [0], [4], 4, 2, 8)
    out = verify_attention(q, k, v, cu, c, 4, 2)
    for h in range(4):
        assert np.allclose(out[0, h], v[0, h // 2, 0].astype(np.float32), atol=1e-7)
    # constant values -> that constant
    v_const = np.full_like(v, 0.375)
    out = verify_attention(q, k, v_const, cu, c, 4, 2)
    assert np.allclose(out, 0.375, atol=1e-7)
    # identical keys -> uniform weights -> mean of the visible values
    k_same = np.broadcast_to(k[:, :, :1], k.shape).copy()
    out = verify_attention(q, k_same, v, cu, c, 4, 2)
    for i in range(4):
        for h in range(4):
            mean = v[0, h // 2, :i + 1].mean(axis=0)
            assert np.allclose(out[i, h], mean, atol=1e-6)


def test_causality_and_poison():
    rng = np.random.default_rng(3)
    q, k, v, cu, c = _case(rng, [11, 4], [5, 3], 4, 2, 16, s_max=40)
    base = verify_attention(q, k, v, cu, c, 4, 2)
    for b, (ctx, rows) in enumerate([(11, 5), (4, 3)]):
        for i in range(rows):
            k2, v2 = k.copy(), v.copy()
            k2[b, :, ctx + i + 1:] = np.nan       # unseen keys, incl. later drafts + tail
            v2[b, :, ctx + i + 1:] = np.nan
            out = verify_attention(q, k2, v2, cu, c, 4, 2)
            r = cu[b] + i
            assert np.array_equal(out[r], base[r])


def test_row_isolation():
    rng = np.random.default_rng(4)
    q, k, v, cu, c = _case(rng, [6], [3], 4, 2, 16)
    q2 = np.concatenate([q, q, q])
    k2 = np.concatenate([k, k, k])
    v2 = np.concatenate([v, v, v])
    cu2 = np.array([0, 3, 6, 9])
    out = verify_attention(q2, k2, v2, cu2, np.array([6, 6, 6]), 4, 2)
    single = verify_attention(q, k, v, cu, c, 4, 2)
    for b in range(3):
        assert np.array_equal(out[3 * b:3 * b + 3], single)
