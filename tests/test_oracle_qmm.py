"""Pins of the small-M quantized matmul oracle (CPU): a product worked by hand, and weights
that quantize losslessly against the plain matrix product."""
import numpy as np

from oracle.qmm import small_m_qmm
from verify_step_attention_amd import workloads as wl


def test_by_hand_two_groups_both_widths():
    # N = 1 output, K = 128 (two groups). Group 0: scale 0.5, bias -1; group 1: scale 2,
    # bias 3. Codes: k = 0 -> 4, k = 64 -> 1, k = 127 -> 5, every other code 0.
    c = np.zeros(128, dtype=np.int64)
    c[0], c[64], c[127] = 4, 1, 5
    sb = np.array([[[0.5, -1.0], [2.0, 3.0]]], dtype=np.float16)
    x = np.zeros((2, 128), dtype=np.float32)
    x[0, 0], x[0, 64], x[0, 127] = 1.0, 1.0, 1.0          # picks w[0], w[64], w[127]
    x[1, :] = 1.0                                         # sums every weight
    # w[0] = 1, w[64] = 5, w[127] = 13, other group-0 weights -1, other group-1 weights 3
    want = np.array([[1.0 + 5.0 + 13.0], [1.0 + 63 * -1.0 + 5.0 + 13.0 + 62 * 3.0]])
    codes8 = c.astype(np.uint8)[None]
    codes4 = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)[None]
    assert np.array_equal(small_m_qmm(x, codes8, sb, 8), want.astype(np.float32))
    assert np.array_equal(small_m_qmm(x, codes4, sb, 4), want.astype(np.float32))


def test_lossless_weights_equal_plain_product():
    rng = np.random.default_rng(5)
    for bits in (8, 4):
        qmax = (1 << bits) - 1
        n, k, m = 24, 256, 7
        lv = rng.integers(0, qmax + 1, size=(n, k))
        lv[:, 0::64] = 0
        lv[:, 1::64] = qmax                                # every group spans 0 .. qmax
        w = (0.0625 * lv - 2.0).astype(np.float32)
        codes, sb = wl.quantize_kv(w, bits)
        x = wl.bf16_to_f32(wl.bf16_bits(rng.standard_normal((m, k)).astype(np.float32)))
        got = small_m_qmm(x, codes, sb, bits)
        ref = (x.astype(np.float64) @ w.astype(np.float64).T).astype(np.float32)
        assert np.array_equal(got, ref)
