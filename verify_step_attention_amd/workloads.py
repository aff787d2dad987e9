"""Seeded synthetic inputs for the verify step (shared by tests, the smoke check and the
benchmark). This module holds no part of the verify arithmetic: it only draws inputs with
the shapes, dtypes and value distributions of the workloads below.

Workloads (shapes of the verify step as the mlx-dspark pages exercise it: Qwen3-class
GQA targets, 151936/262144-token vocabularies, verify widths of a few rows, contexts up to
32k, batched continuous verify; Changelog [0.20.0], [0.2.0], release v0.2.0):

  tiny                 B=1, K=2, Hq/Hkv 8/2, D=64, ctx 128, fp32 Q/K/V; V=1024,
                       target ~N(0, sd 2)
  qwen3_4b             B=1, K=4, 32/8, D=128, ctx 4096, bf16; V=151936, target ~N(0, sd 3)
                       with 20 random ids boosted by +8; T=0.7, top_k=20, top_p=0.8
  batched              B=4, K_b ~U{2..7}, ctx_b ~U{750..8192}, 32/8, D=128, bf16; V=151936,
                       ~N(0, sd 3); presence 0.5 / frequency 0.3 from count histograms of
                       U{0..2048} prior ids ~ Zipf(1.1) over a permuted vocabulary; even b
                       greedy, odd b T=0.8
  long                 B=1, K=8, 48/8, D=128, ctx 32768, bf16; V=262144, ~N(0, sd 3) plus
                       8/r for the token of rank r in a seeded permutation; T=1.0, top_k=64,
                       top_p=0.95
  swarm                B=16, K=4, ctx_b ~U{2048..16384}, 32/8, D=128, bf16; V=151936,
                       ~N(0, sd 3); T=0.6, top_k=20, top_p=0.95, penalties 0.5/0.3,
                       chosen logprob + top 5
  verify_b4k4_ctx8192  B=4, K=4, ctx 8192, 32/8, D=128, bf16; V=151936 ~N(0, sd 3);
                       penalties 0.5/0.3 with counts as in `batched`; b=0,2 greedy,
                       b=1,3 T=0.8; no top-k / top-p

Common recipe: Q, K, V ~N(0,1) (bf16 rounded to nearest even where bf16); K/V slots past
each sequence's ctx_b + R_b are NaN (poison that catches out-of-range reads); draft row t
of a sequence = target row t-1 + N(0, sd 0.5) (the draft predicts the slot target row t-1
decides); positions[b] = ctx_b + 1; verify seed 0. Draft tokens default to a stand-in
greedy drafter (argmax of each draft row); tests that need drafts distributed as the
truncated draft distribution replace them.
"""
from dataclasses import dataclass, field, replace

import numpy as np

F32, BF16 = 0, 1


def bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even, NaN kept quiet."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(np.asarray(x, dtype=np.float32)), np.uint16(0x7FC0), rounded)


def bf16_to_f32(bits):
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


@dataclass
class Params:
    """One sequence's sampling parameters, field order of the library's row struct."""
    temperature: float = 0.0
    top_k: int = 0
    top_p: float = 1.0
    presence_penalty: float = 0.0
    frequency_penalty: float = 0.0
    logprobs: int = 0
    top_logprobs: int = 0


@dataclass
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: int                       # F32 or BF16 (Q, K, V)
    vocab: int
    ctx_lens: np.ndarray             # [B] int32
    cu_rows: np.ndarray              # [B+1] int32
    s_max: int
    q: np.ndarray                    # [T, Hq, D]  float32 or bf16 bits (uint16)
    k_cache: np.ndarray              # [B, Hkv, S_max, D]
    v_cache: np.ndarray
    target_logits: np.ndarray        # [T, V] float32
    draft_logits: np.ndarray         # [T-B, V] float32
    draft_tokens: np.ndarray         # [T-B] int32
    token_counts: object             # [B, V] int32 or None
    params: list                     # [B] Params
    positions: np.ndarray            # [B] int32
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def total_rows(self):
        return int(self.cu_rows[-1])

    @property
    def max_rows(self):
        return int(np.diff(self.cu_rows).max())

    @property
    def max_kv_len(self):
        return int((self.ctx_lens + np.diff(self.cu_rows)).max())

    def q_f32(self):
        return self.q if self.dtype == F32 else bf16_to_f32(self.q)

    def kv_f32(self):
        if self.dtype == F32:
            return self.k_cache, self.v_cache
        return bf16_to_f32(self.k_cache), bf16_to_f32(self.v_cache)

    def with_params(self, params):
        return replace(self, params=list(params))


_SPECS = {
    # name: (rng id, B, K spec, ctx spec, Hq, Hkv, D, dtype, V)
    "verify_b4k4_ctx8192": (1000, 4, 4, 8192, 32, 8, 128, BF16, 151936),
    "tiny": (1001, 1, 2, 128, 8, 2, 64, F32, 1024),
    "qwen3_4b": (1002, 1, 4, 4096, 32, 8, 128, BF16, 151936),
    "batched": (1003, 4, (2, 7), (750, 8192), 32, 8, 128, BF16, 151936),
    "long": (1004, 1, 8, 32768, 48, 8, 128, BF16, 262144),
    "swarm": (1005, 16, 4, (2048, 16384), 32, 8, 128, BF16, 151936),
    # a drafter's block of 8 rows over a 32k context (attention only; tiny vocabulary)
    "drafter_b4r8_ctx32768": (1006, 4, 7, 32768, 32, 8, 128, BF16, 1024),
}

WORKLOAD_NAMES = tuple(_SPECS)


def _draw(rng, spec, batch):
    if isinstance(spec, tuple):
        return rng.integers(spec[0], spec[1] + 1, size=batch)
    return np.full(batch, spec)


def _zipf_counts(rng, batch, vocab):
    perm = rng.permutation(vocab)
    counts = np.zeros((batch, vocab), dtype=np.int32)
    for b in range(batch):
        n = int(rng.integers(0, 2049))
        ranks = (rng.zipf(1.1, size=n) - 1) % vocab
        np.add.at(counts[b], perm[ranks], 1)
    return counts


def _default_params(name, batch):
    if name in ("tiny", "drafter_b4r8_ctx32768"):
        return [Params()] * batch
    if name == "qwen3_4b":
        return [Params(temperature=0.7, top_k=20, top_p=0.8)]
    if name in ("batched", "verify_b4k4_ctx8192"):
        return [Params(presence_penalty=0.5, frequency_penalty=0.3) if b % 2 == 0 else
                Params(temperature=0.8, presence_penalty=0.5, frequency_penalty=0.3)
                for b in range(batch)]
    if name == "long":
        return [Params(temperature=1.0, top_k=64, top_p=0.95)]
    if name == "swarm":
        return [Params(temperature=0.6, top_k=20, top_p=0.95, presence_penalty=0.5,
                       frequency_penalty=0.3, logprobs=1, top_logprobs=5)
                for _ in range(batch)]
    raise KeyError(name)


def quantize_kv(x, bits, group=64):
    """Input generator for the quantized K/V cache format: float32 [..., D] -> (codes uint8,
    (scale, bias) float16 pairs [..., D / group, 2]). Per group of `group` dimensions:
    bias = fp16(min), scale = fp16((max - min) / (2^bits - 1)), code = the nearest level,
    clamped; 4-bit codes pack two to a byte, element 2i in the low nibble. A group holding
    NaN (poison past a sequence's keys) gets codes of all ones and NaN scale and bias."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    assert d % group == 0 and bits in (4, 8)
    g = x.reshape(x.shape[:-1] + (d // group, group))
    lo = np.nanmin(np.where(np.isnan(g), np.inf, g), axis=-1)
    hi = np.nanmax(np.where(np.isnan(g), -np.inf, g), axis=-1)
    bad = np.isnan(g).any(axis=-1)
    lo = np.where(bad, 0.0, lo)
    hi = np.where(bad, 0.0, hi)
    qmax = (1 << bits) - 1
    scale = ((hi - lo) / qmax).astype(np.float16)
    bias = lo.astype(np.float16)
    s32 = scale.astype(np.float32)[..., None]
    b32 = bias.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(s32 > 0, np.rint((g - b32) / s32), 0.0)
    c = np.clip(np.nan_to_num(c), 0, qmax).astype(np.uint8)
    c = np.where(bad[..., None], np.uint8(qmax), c).reshape(x.shape)
    sb = np.stack([scale, bias], axis=-1)
    sb[bad] = np.float16(np.nan)
    if bits == 4:
        c = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(c), np.ascontiguousarray(sb)


@dataclass
class KvQuant:
    """A workload's K/V cache in the quantized format (see quantize_kv)."""
    bits: int
    k_codes: np.ndarray
    k_sb: np.ndarray
    v_codes: np.ndarray
    v_sb: np.ndarray


def quantized_cache(w, bits):
    """The workload's K/V cache (its bf16 or fp32 values, NaN past each sequence's keys)
    in the quantized format."""
    k, v = w.kv_f32()
    kc, ks = quantize_kv(k, bits)
    vc, vs = quantize_kv(v, bits)
    return KvQuant(bits=bits, k_codes=kc, k_sb=ks, v_codes=vc, v_sb=vs)


def make_workload(name, *, batch=None, drafts=None, ctx=None, vocab=None, with_kv=True,
                  seed_offset=0):
    """Build the named workload. Overrides (batch, drafts per sequence, context, vocab)
    give scaled variants with the same distributions; `with_kv=False` skips the KV cache
    (for sampling-only uses)."""
    rid, b0, kspec, cspec, hq, hkv, d, dtype, v0 = _SPECS[name]
    rng = np.random.default_rng(rid + seed_offset)
    batch = b0 if batch is None else batch
    kspec = kspec if drafts is None else drafts
    cspec = cspec if ctx is None else ctx
    vocab = v0 if vocab is None else vocab
    k_per = _draw(rng, kspec, batch).astype(np.int32)
    ctx_lens = _draw(rng, cspec, batch).astype(np.int32)
    rows = k_per + 1
    cu_rows = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    total = int(cu_rows[-1])
    kv_len = ctx_lens + rows
    s_max = int(-(-int(kv_len.max() + 8) // 64) * 64)

    # attention operands
    qf = rng.standard_normal((total, hq, d), dtype=np.float32)
    if with_kv:
        kf = rng.standard_normal((batch, hkv, s_max, d), dtype=np.float32)
        vf = rng.standard_normal((batch, hkv, s_max, d), dtype=np.float32)
        for b in range(batch):
            kf[b, :, kv_len[b]:] = np.nan
            vf[b, :, kv_len[b]:] = np.nan
    else:
        kf = vf = np.zeros((batch, hkv, 0, d), dtype=np.float32)
    if dtype == BF16:
        q, k_cache, v_cache = bf16_bits(qf), bf16_bits(kf), bf16_bits(vf)
    else:
        q, k_cache, v_cache = qf, kf, vf

    # logits
    sd = 2.0 if name == "tiny" else 3.0
    target = (sd * rng.standard_normal((total, vocab), dtype=np.float32)).astype(np.float32)
    if name == "qwen3_4b":
        for r in range(total):
            target[r, rng.choice(vocab, size=min(20, vocab), replace=False)] += 8.0
    if name == "long":
        perm = rng.permutation(vocab)
        boost = np.zeros(vocab, dtype=np.float32)
        boost[perm] = (8.0 / np.arange(1, vocab + 1)).astype(np.float32)
        target += boost[None, :]
    draft = np.empty((total - batch, vocab), dtype=np.float32)
    for b in range(batch):
        for t in range(1, int(rows[b])):
            draft[cu_rows[b] - b + t - 1] = target[cu_rows[b] + t - 1] + (
                0.5 * rng.standard_normal(vocab, dtype=np.float32))
    draft_tokens = np.argmax(draft, axis=1).astype(np.int32) if total > batch else \
        np.zeros(0, dtype=np.int32)
    params = _default_params(name, batch)
    counts = None
    if any(p.presence_penalty or p.frequency_penalty for p in params):
        counts = _zipf_counts(rng, batch, vocab)
    positions = (ctx_lens + 1).astype(np.int32)
    return Workload(name=name, batch=batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    dtype=dtype, vocab=vocab, ctx_lens=ctx_lens, cu_rows=cu_rows,
                    s_max=s_max, q=q, k_cache=k_cache, v_cache=v_cache,
                    target_logits=target, draft_logits=draft, draft_tokens=draft_tokens,
                    token_counts=counts, params=params, positions=positions, seed=0)


def device_tensors(w, device="cuda", with_kv=True):
    """Copy a workload to the GPU as torch tensors (bf16 inputs keep their bit patterns)."""
    import torch

    def t(x, dtype=None):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device) if dtype is None else \
            torch.from_numpy(np.ascontiguousarray(x)).to(device).view(dtype)

    out = {}
    if w.q is None:
        with_kv = False
    elif w.dtype == BF16:
        out["q"] = t(w.q.view(np.int16), torch.bfloat16)
        if with_kv:
            out["k_cache"] = t(w.k_cache.view(np.int16), torch.bfloat16)
            out["v_cache"] = t(w.v_cache.view(np.int16), torch.bfloat16)
    else:
        out["q"] = t(w.q)
        if with_kv:
            out["k_cache"] = t(w.k_cache)
            out["v_cache"] = t(w.v_cache)
    out["cu_rows"] = t(w.cu_rows.astype(np.int32))
    out["ctx_lens"] = t(w.ctx_lens.astype(np.int32))
    out["target_logits"] = t(w.target_logits)
    out["draft_logits"] = (t(w.draft_logits) if w.draft_logits is not None and w.draft_logits.size
                           else None)
    out["draft_tokens"] = t(w.draft_tokens.astype(np.int32)) if w.draft_tokens.size else None
    out["token_counts"] = None if w.token_counts is None else t(w.token_counts.astype(np.int32))
    out["positions"] = t(w.positions.astype(np.int32))
    return out
