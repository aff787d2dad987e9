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


# ------------------------------------------------------------- a drafter's block, windowed
# The same multi-row attention also serves a drafter's block over its context (Changelog
# [0.20.0] "Added"). Around it the pages give: the drafter's context K/V lives in one buffer
# with the block written into its tail ([0.20.0] "Changed"), i.e. the block's keys sit right
# after the context, as in verify; the drafter attends only the last N context rows
# (--drafter-window N, 0 = the whole context), while heads with a trained sliding window
# keep theirs ([0.20.0] "Changed"); DFlash-lineage heads are causal inside the block (a row
# never sees later block positions) and DeepSpec-native heads are bidirectional there
# ([0.8.1] "Changed"). The reading used here, for block row i at position p = ctx_b + i:
#   first visible key  lo_i = 0                          no window (window = 0)
#                           = max(0, ctx_b - window)     recent window of context rows
#                           = max(0, p - window + 1)     sliding window ending at p
#   last visible key   hi_i = p                          causal block
#                           = ctx_b + R_b - 1            bidirectional block
# and row i attends keys lo_i .. hi_i (never empty: lo_i <= p <= hi_i).


def block_visible_range(ctx, rows, i, window=0, sliding=False, bidirectional=False):
    """(lo, hi): the keys row i of a block of `rows` rows after `ctx` context keys sees."""
    p = ctx + i
    if window == 0:
        lo = 0
    elif sliding:
        lo = max(0, p - window + 1)
    else:
        lo = max(0, ctx - window)
    hi = ctx + rows - 1 if bidirectional else p
    return lo, hi


def block_attention(q, k_cache, v_cache, cu_rows, ctx_lens, num_q_heads, num_kv_heads,
                    scale=None, window=0, sliding=False, bidirectional=False):
    """Attention of each sequence's block rows over keys lo_i .. hi_i (above), in fp64,
    rounded once to fp32. window = 0, causal: the verify definition."""
    q = np.asarray(q)
    total_rows, hq, d = q.shape
    assert hq == num_q_heads and num_q_heads % num_kv_heads == 0 and window >= 0
    assert not (sliding and window == 0)
    group = num_q_heads // num_kv_heads
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((total_rows, hq, d), dtype=np.float32)
    for b in range(len(ctx_lens)):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        ctx = int(ctx_lens[b])
        for i in range(r1 - r0):
            lo, hi = block_visible_range(ctx, r1 - r0, i, window, sliding, bidirectional)
            for g in range(num_kv_heads):
                keys = np.asarray(k_cache[b, g, lo:hi + 1], dtype=np.float64)
                vals = np.asarray(v_cache[b, g, lo:hi + 1], dtype=np.float64)
                heads = slice(g * group, (g + 1) * group)
                qg = np.asarray(q[r0 + i, heads], dtype=np.float64)
                s = scale * (qg @ keys.T)
                w = np.exp(s - s.max(axis=1, keepdims=True))
                out[r0 + i, heads] = ((w @ vals) / w.sum(axis=1, keepdims=True)).astype(
                    np.float32)
    return out


# ---------------------------------------------------------------------- quantized K/V cache
# The pages' --kv-bits 4|8 option keeps the target's K/V cache quantized from token 0
# (mlx-dspark Changelog [0.3.0] "Added": KV-cache quantization; [0.13.1]: 8 bits halve and
# 4 bits quarter the per-token cache). They do not give the format; the reading used here
# is affine quantization in groups of 64 consecutive head dimensions, the grouping the pages
# name for weights:
#   value = scale * code + bias,   code unsigned (8 bits: 0..255, 4 bits: 0..15),
#   one (scale, bias) pair of fp16 per group.
# Layouts (row-major):
#   codes  [B, Hkv, S_max, D]       uint8 (8 bits)
#          [B, Hkv, S_max, D / 2]   uint8 (4 bits: element 2i in the low nibble, 2i + 1 in
#                                   the high nibble)
#   sb     [B, Hkv, S_max, D / 64, 2]  float16 (scale, bias)
# Attention over a quantized cache is the definition above applied to the dequantized
# values, each computed exactly in fp64 (an fp16 times an integer below 2^8, plus an fp16).

KV_GROUP = 64


def dequantize_kv(codes, sb, bits):
    """Quantized cache -> float64 [B, Hkv, S, D] (the exact values scale * code + bias)."""
    codes = np.asarray(codes, dtype=np.uint8)
    sb = np.asarray(sb, dtype=np.float16)
    if bits == 8:
        c = codes.astype(np.float64)
    elif bits == 4:
        lo = (codes & 0x0F).astype(np.float64)
        hi = (codes >> 4).astype(np.float64)
        c = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    else:
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    d = c.shape[-1]
    assert d % KV_GROUP == 0 and sb.shape[-2:] == (d // KV_GROUP, 2)
    scale = np.repeat(sb[..., 0].astype(np.float64), KV_GROUP, axis=-1)
    bias = np.repeat(sb[..., 1].astype(np.float64), KV_GROUP, axis=-1)
    return scale * c + bias


def verify_attention_kvq(q, k_codes, k_sb, v_codes, v_sb, bits, cu_rows, ctx_lens,
                         num_q_heads, num_kv_heads, scale=None):
    """Verify attention over a quantized K/V cache: the same definition on the dequantized
    keys and values."""
    return verify_attention(q, dequantize_kv(k_codes, k_sb, bits),
                            dequantize_kv(v_codes, v_sb, bits), cu_rows, ctx_lens,
                            num_q_heads, num_kv_heads, scale=scale)
