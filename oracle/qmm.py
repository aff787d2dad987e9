"""The few-row quantized matmul of the verify forward, written out as its definition (CPU,
fp64).

TEST INFRASTRUCTURE: part of the CPU oracle. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.

What is computed (mlx-dspark Changelog [0.20.0] "Changed": a small-M verify matmul kernel
for the few rows of a verify, widths 5-16 at 4-bit and 6-16 at 8-bit, computing the
quantized matmul with the weights as the matrix operand shared by every row; the weights
are affine-quantized in groups of 64 along the input dimension, [0.12.0] "Changed": the
earlier small-M kernel runs on 4-bit and 8-bit gs64 weights):

    y[m][n] = sum_k x[m][k] * w[n][k],   w[n][k] = scale[n][g] * code[n][k] + bias[n][g],
    g = k // 64,

for M <= 16 rows x, N output features and K inputs. The weight layout is the one the
quantized K/V cache uses here (the pages give no byte layout for either):
  x      [M, K]            bf16 (widened exactly)
  codes  [N, K * bits / 8] uint8 (8 bits: one per element; 4 bits: element 2i in the low
                           nibble of byte i)
  sb     [N, K / 64, 2]    fp16 (scale, bias)
  y      [M, N]            float32: the fp64 sum rounded once.
"""
import numpy as np

from .attention import dequantize_kv


def small_m_qmm(x, codes, sb, bits):
    x = np.asarray(x, dtype=np.float64)
    w = dequantize_kv(codes, sb, bits)                 # [N, K] exact values in fp64
    if x.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [M, K] with K the weights' input dimension")
    return (x @ w.T).astype(np.float32)
