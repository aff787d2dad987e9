"""GPU parity of verify_attention against the CPU oracle (elementwise,
|gpu - oracle| <= 1e-3 + 2e-3 |oracle|), through the C ABI."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_step_attention_amd as vsa  # noqa: E402
from verify_step_attention_amd import workloads as wl  # noqa: E402
from gpu_helpers import (attention_gpu, attention_oracle, assert_attention_close,  # noqa: E402
                         compare_sample, q_distributed_drafts, sample_gpu, sample_oracle)


def _log(msg):
    print(msg, flush=True)


FLAGS = [0, vsa.ATTN_DYNAMIC_SPLITS]


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("name", ["tiny", "qwen3_4b", "batched", "verify_b4k4_ctx8192",
                                  "long", "swarm"])
def test_workload_parity(name, flags):
    _log(f"attention parity: workload {name} flags {flags}")
    w = wl.make_workload(name)
    got, err = attention_gpu(w, flags=flags)
    assert err == 0
    assert_attention_close(got, attention_oracle(w))


@pytest.mark.parametrize("case", [
    # (Hq, Hkv, D, dtype, ctx list, drafts list, max_kv_len override)
    (32, 8, 128, wl.BF16, [0, 1, 127, 128], [0, 3, 4, 31], None),      # ctx 0, K=0, K=31
    (8, 8, 64, wl.BF16, [300, 5], [2, 6], 4096),                        # D=64, MHA, empty splits
    (64, 8, 128, wl.BF16, [700], [15], None),                           # 128 columns (4 blocks)
    (48, 8, 128, wl.BF16, [1000, 2000], [8, 2], None),                  # 2 column blocks
    (16, 2, 64, wl.F32, [333, 40], [3, 9], None),                       # fp32, ragged
    (32, 8, 128, wl.BF16, [5], [4], 8192),                              # mostly empty splits
])
@pytest.mark.parametrize("flags", FLAGS)
def test_edge_shapes(case, flags):
    hq, hkv, d, dtype, ctxs, drafts, mkv = case
    _log(f"attention edge case {case} flags {flags}")
    w = _custom(hq, hkv, d, dtype, ctxs, drafts)
    if mkv is not None:
        mkv = min(mkv, w.s_max)
    got, err = attention_gpu(w, max_kv_len=mkv, flags=flags)
    assert err == 0
    assert_attention_close(got, attention_oracle(w))


def _custom(hq, hkv, d, dtype, ctxs, drafts, seed=5):
    rng = np.random.default_rng(seed)
    batch = len(ctxs)
    rows = np.array(drafts) + 1
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    kv_len = np.array(ctxs) + rows
    s_max = int(-(-int(kv_len.max() + 8) // 64) * 64)
    s_max = max(s_max, 4096 + 64) if max(ctxs) < 400 else s_max
    qf = rng.standard_normal((cu[-1], hq, d), dtype=np.float32)
    kf = rng.standard_normal((batch, hkv, s_max, d), dtype=np.float32)
    vf = rng.standard_normal((batch, hkv, s_max, d), dtype=np.float32)
    for b in range(batch):
        kf[b, :, kv_len[b]:] = np.nan
        vf[b, :, kv_len[b]:] = np.nan
    if dtype == wl.BF16:
        q, k, v = wl.bf16_bits(qf), wl.bf16_bits(kf), wl.bf16_bits(vf)
    else:
        q, k, v = qf, kf, vf
    z = np.zeros((cu[-1], 4), np.float32)
    return wl.Workload(name="custom", batch=batch, num_q_heads=hq, num_kv_heads=hkv,
                       head_dim=d, dtype=dtype, vocab=4, ctx_lens=np.array(ctxs, np.int32),
                       cu_rows=cu, s_max=s_max, q=q, k_cache=k, v_cache=v, target_logits=z,
                       draft_logits=z[:cu[-1] - batch], draft_tokens=np.zeros(cu[-1] - batch,
                                                                             np.int32),
                       token_counts=None, params=[wl.Params()] * batch,
                       positions=np.array(ctxs, np.int32) + 1)


def test_batch_invariance_and_workspace_reuse():
    """Identical sequences give identical rows (row isolation), and a workspace reused by a
    second call gives the same bits (counters were returned to zero)."""
    w1 = _custom(32, 8, 128, wl.BF16, [3000], [4])
    rep = _custom(32, 8, 128, wl.BF16, [3000], [4])
    for f in ("q", "k_cache", "v_cache"):
        setattr(rep, f, np.concatenate([getattr(w1, f)] * 3))
    rep.batch = 3
    rep.ctx_lens = np.array([3000] * 3, np.int32)
    rep.cu_rows = np.array([0, 5, 10, 15], np.int32)
    a, _ = attention_gpu(rep)
    for b in range(1, 3):
        assert np.array_equal(a[5 * b:5 * b + 5], a[0:5])
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    x, _ = attention_gpu(w1, workspace=ws)
    y, _ = attention_gpu(w1, workspace=ws)
    assert np.array_equal(x, y)


def test_dynamic_splits_reuse_workspace():
    """Dynamic splits: the tile counters return to zero, so calls that reuse one workspace
    (different sequences in between) all cover every key; results agree up to rounding."""
    _log("attention dynamic splits: workspace reuse")
    a = wl.make_workload("batched")
    b = wl.make_workload("qwen3_4b")
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    ref_a, ref_b = attention_oracle(a), attention_oracle(b)
    first = None
    for rep in range(3):
        x, err = attention_gpu(a, workspace=ws, flags=vsa.ATTN_DYNAMIC_SPLITS)
        assert err == 0
        assert_attention_close(x, ref_a)
        if first is None:
            first = x
        assert np.allclose(x, first, rtol=1e-5, atol=1e-6)
        y, err = attention_gpu(b, workspace=ws, flags=vsa.ATTN_DYNAMIC_SPLITS)
        assert err == 0
        assert_attention_close(y, ref_b)


def test_shared_workspace_across_shapes_and_calls():
    """One workspace serves calls of different shapes and different functions in stream
    order: a call over more (sequence, KV head) units than the previous one must still find
    its tile counters at zero, and a sampling call in between must not disturb them."""
    _log("shared workspace: 8 units, 96 units, sampling, 8 units, 96 units")
    small = wl.make_workload("qwen3_4b", ctx=300)                  # 8 units
    big = wl.make_workload("batched", batch=12, ctx=(200, 700))    # 96 units
    samp = wl.make_workload("batched", with_kv=False, vocab=8192)
    samp.draft_tokens = q_distributed_drafts(samp)
    sizes = [vsa.verify_attention_workspace_size(w.batch, w.num_q_heads, w.num_kv_heads,
                                                 w.head_dim, w.max_rows, w.max_kv_len)
             for w in (small, big)]
    sizes.append(vsa.verify_sample_accept_workspace_size(samp.batch, samp.total_rows,
                                                         samp.vocab, samp.max_rows, 0, 0))
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device="cuda")
    ref_s, ref_b = attention_oracle(small), attention_oracle(big)
    want = sample_oracle(samp, seed=0)
    for rep in range(2):
        x, err = attention_gpu(small, workspace=ws, flags=vsa.ATTN_DYNAMIC_SPLITS)
        assert err == 0
        assert_attention_close(x, ref_s)
        y, err = attention_gpu(big, workspace=ws, flags=vsa.ATTN_DYNAMIC_SPLITS)
        assert err == 0
        assert_attention_close(y, ref_b)
        got = sample_gpu(samp, seed=0, workspace=ws)
        assert got["err"] == 0
        compare_sample(samp, got, want)


def test_units_past_the_counter_region():
    """More (sequence, KV head) units than the workspace's counter region holds: the rest of
    the tile counters live in the call's own area, cleared first; dynamic splits still cover
    every key, twice in a row on one workspace."""
    _log("attention: 2100 x 8 units, dynamic splits")
    rng = np.random.default_rng(9)
    batch, hkv, hq, d = 2100, 8, 8, 64
    ctxs = rng.integers(0, 100, size=batch)
    drafts = rng.integers(0, 3, size=batch)
    w = _custom_small(hq, hkv, d, ctxs, drafts, rng)
    ref = attention_oracle(w)
    size = vsa.verify_attention_workspace_size(batch, hq, hkv, d, w.max_rows, w.max_kv_len)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        x, err = attention_gpu(w, workspace=ws, flags=vsa.ATTN_DYNAMIC_SPLITS)
        assert err == 0
        assert_attention_close(x, ref)


def _custom_small(hq, hkv, d, ctxs, drafts, rng):
    batch = len(ctxs)
    rows = np.asarray(drafts) + 1
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    kv_len = np.asarray(ctxs) + rows
    s_max = int(-(-int(kv_len.max() + 8) // 64) * 64)
    qf = rng.standard_normal((cu[-1], hq, d), dtype=np.float32)
    kf = rng.standard_normal((batch, hkv, s_max, d), dtype=np.float32)
    vf = rng.standard_normal((batch, hkv, s_max, d), dtype=np.float32)
    for b in range(batch):
        kf[b, :, kv_len[b]:] = np.nan
        vf[b, :, kv_len[b]:] = np.nan
    z = np.zeros((cu[-1], 4), np.float32)
    return wl.Workload(name="custom", batch=batch, num_q_heads=hq, num_kv_heads=hkv,
                       head_dim=d, dtype=wl.BF16, vocab=4,
                       ctx_lens=np.asarray(ctxs, np.int32), cu_rows=cu, s_max=s_max,
                       q=wl.bf16_bits(qf), k_cache=wl.bf16_bits(kf), v_cache=wl.bf16_bits(vf),
                       target_logits=z, draft_logits=z[:cu[-1] - batch],
                       draft_tokens=np.zeros(cu[-1] - batch, np.int32), token_counts=None,
                       params=[wl.Params()] * batch,
                       positions=np.asarray(ctxs, np.int32) + 1)


def test_device_error_word_on_bad_context():
    w = _custom(8, 2, 64, wl.BF16, [100], [2])
    w.ctx_lens = np.array([w.s_max], np.int32)          # ctx + R beyond S_max: clamped
    _, err = attention_gpu(w, max_kv_len=w.s_max)
    assert err & 0x01
