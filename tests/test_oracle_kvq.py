"""Pins of the quantized-K/V attention oracle (CPU): the dequantization against values
worked by hand and against exact reconstructions, and attention over a cache that
quantizes losslessly against the unquantized definition."""
import numpy as np
import pytest

from oracle.attention import dequantize_kv, verify_attention, verify_attention_kvq
from verify_step_attention_amd import workloads as wl


def _sb(scale, bias, groups):
    sb = np.zeros((groups, 2), dtype=np.float16)
    sb[:, 0] = scale
    sb[:, 1] = bias
    return sb


def test_dequantize_8bit_by_hand():
    codes = np.zeros(64, dtype=np.uint8)
    codes[:4] = [0, 1, 128, 255]
    out = dequantize_kv(codes[None], _sb(0.5, -1.0, 1)[None], 8)[0]
    assert out[:4].tolist() == [-1.0, -0.5, 63.0, 126.5]
    assert np.all(out[4:] == -1.0)


def test_dequantize_4bit_nibble_order_by_hand():
    codes = np.zeros(32, dtype=np.uint8)          # 64 elements
    codes[0] = 0xA3                               # element 0 = 3 (low), element 1 = 10 (high)
    codes[31] = 0x0F                              # element 62 = 15, element 63 = 0
    out = dequantize_kv(codes[None], _sb(0.25, 2.0, 1)[None], 4)[0]
    assert out[0] == 2.75 and out[1] == 4.5
    assert out[62] == 5.75 and out[63] == 2.0
    assert np.all(out[2:62] == 2.0)


def test_dequantize_uses_each_groups_own_scale():
    codes = np.full((1, 128), 2, dtype=np.uint8)
    sb = np.array([[[1.0, 0.0], [-3.0, 10.0]]], dtype=np.float16)
    out = dequantize_kv(codes, sb, 8)[0]
    assert np.all(out[:64] == 2.0) and np.all(out[64:] == 4.0)


@pytest.mark.parametrize("bits", [8, 4])
def test_exact_levels_round_trip(bits):
    """Values that sit exactly on a group's levels quantize and dequantize to themselves."""
    rng = np.random.default_rng(7)
    qmax = (1 << bits) - 1
    shape = (2, 3, 5, 128)
    scale = np.float16(0.125)
    bias = rng.integers(-8, 8, size=shape[:-1] + (2,)).astype(np.float16)
    codes = rng.integers(0, qmax + 1, size=shape).astype(np.int64)
    codes[..., 0] = 0
    codes[..., 64] = 0                            # every group spans 0 .. qmax
    codes[..., 1] = qmax
    codes[..., 65] = qmax
    x = (np.float64(scale) * codes +
         np.repeat(bias.astype(np.float64), 64, axis=-1)).astype(np.float32)
    c, sb = wl.quantize_kv(x, bits)
    assert np.all(sb[..., 0] == scale)
    assert np.array_equal(dequantize_kv(c, sb, bits), x.astype(np.float64))


def test_attention_over_lossless_cache_equals_definition():
    rng = np.random.default_rng(11)
    hq, hkv, d, s_max = 4, 2, 128, 96
    ctx = np.array([40, 70], dtype=np.int32)
    cu = np.array([0, 3, 5], dtype=np.int32)
    q = rng.standard_normal((5, hq, d)).astype(np.float32)
    lv = rng.integers(0, 256, size=(2, hkv, s_max, d))
    lv[..., 0] = 0
    lv[..., 64] = 0
    lv[..., 1] = 255
    lv[..., 65] = 255
    k = (0.03125 * lv - 4.0).astype(np.float32)
    v = (0.0625 * rng.permutation(lv.ravel()).reshape(lv.shape) - 8.0).astype(np.float32)
    v[..., 0] = -8.0
    v[..., 64] = -8.0
    v[..., 1] = 0.0625 * 255 - 8.0
    v[..., 65] = 0.0625 * 255 - 8.0
    kc, ks = wl.quantize_kv(k, 8)
    vc, vs = wl.quantize_kv(v, 8)
    got = verify_attention_kvq(q, kc, ks, vc, vs, 8, cu, ctx, hq, hkv)
    ref = verify_attention(q, k, v, cu, ctx, hq, hkv)
    assert np.array_equal(got, ref)


def test_quantization_error_bound_of_generator():
    """The generator's codes sit within half a level (plus the fp16 rounding of scale and
    bias) of the values they stand for."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    for bits in (8, 4):
        c, sb = wl.quantize_kv(x, bits)
        err = np.abs(dequantize_kv(c, sb, bits) - x)
        step = np.repeat(sb[..., 0].astype(np.float64), 64, axis=-1)
        assert np.all(err <= 0.5 * step * (1 + 2 ** -9) + 4 * 2 ** -11 * np.abs(x) + 1e-3)


def test_poison_groups_dequantize_to_nan():
    x = np.zeros((2, 128), dtype=np.float32)
    x[1, :] = np.nan
    c, sb = wl.quantize_kv(x, 8)
    out = dequantize_kv(c, sb, 8)
    assert np.isfinite(out[0]).all() and np.isnan(out[1]).all()
