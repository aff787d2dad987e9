"""Verify attention, written out as its plain definition (CPU, fp64).

TEST INFRASTRUCTURE: part of the CPU oracle. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.

What is computed (mlx-dspark Changelog, [0.20.0] "Added": the multi-row decode-attention
kernel serves verify widths over the whole KV cache, every GQA head x query row of a KV
head reads the same keys; [0.3.1] "Fixed": n_kv-head K/V passed straight to attention is
identical to tiling K/V per query head):

  For sequence b with ctx_b cached tokens and R_b = K_b + 1 verify rows (the anchor and
  the K_b drafts, whose K/V the caller has already written at positions ctx_b .. ctx_b+K_b),
  verify row i and query head h:
      g = h // (Hq / Hkv)                        (contiguous head groups, as K/V tiling
                                                  with repeat-per-group implies)
      n = ctx_b + i + 1                          (causal: row i sees the cache, the anchor
                                                  and drafts up to and including its own)
      s_t = scale * <q, k_{g,t}>   for t < n     (scale = 1/sqrt(D) unless given)
      o   = sum_t softmax(s)_t v_{g,t}
  Inputs are widened exactly to fp64 (bf16 and fp32 are subsets of fp64); every product,
  sum and exponential is fp64; the result is rounded once to fp32.

Layouts (row-major):
  q        [total_rows, Hq, D]        rows of sequence b are cu_rows[b] .. cu_rows[b+1]-1
  k_cache  [B, Hkv, S_max, D]         v_cache the same
  ctx_lens [B]                        tokens cached before the block
  cu_rows  [B+1]                      prefix sums of R_b
  returns  [total_rows, Hq, D] float32
"""
import math

import numpy as np


def verify_attention(q, k_cache, v_cache, cu_rows, ctx_lens, num_q_heads, num_kv_heads,
                     scale=None):
    q = np.asarray(q)
    total_rows, hq, d = q.shape
    assert hq == num_q_heads and num_q_heads % num_kv_heads == 0
    group = num_q_heads // num_kv_heads
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((total_rows, hq, d), dtype=np.float32)
    batch = len(ctx_lens)
    for b in range(batch):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        ctx = int(ctx_lens[b])
        for i in range(r1 - r0):
            n = ctx + i + 1
            for g in range(num_kv_heads):
                keys = np.asarray(k_cache[b, g, :n], dtype=np.float64)      # [n, D]
                vals = np.asarray(v_cache[b, g, :n], dtype=np.float64)      # [n, D]
                heads = slice(g * group, (g + 1) * group)
                qg = np.asarray(q[r0 + i, heads], dtype=np.float64)          # [G, D]
                s = scale * (qg @ keys.T)                                    # [G, n]
                w = np.exp(s - s.max(axis=1, keepdims=True))
                out[r0 + i, heads] = ((w @ vals) / w.sum(axis=1, keepdims=True)).astype(
                    np.float32)
    return out
