"""GPU parity of verify_sample_accept against the CPU oracle, through the C ABI.

Bar: top-k thresholds and kept-set sizes bit-exact; accepted lengths and emitted tokens
equal to the oracle's fp64 decisions, or, for a sequence with a decision inside the GPU's
stated arithmetic error (the oracle's exception points), equal to one of the outcomes the
oracle admits there; logprobs within 2e-5."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from verify_step_attention_amd import workloads as wl  # noqa: E402
from gpu_helpers import (compare_sample, q_distributed_drafts, sample_gpu,  # noqa: E402
                         sample_oracle)


def _log(msg):
    print(msg, flush=True)


def _run(w, seed=0, expect_err=0, max_top_k=None, onehot=False):
    gpu = sample_gpu(w, seed=seed, max_top_k=max_top_k, onehot=onehot)
    assert gpu["err"] == expect_err, hex(gpu["err"])
    ora = sample_oracle(w, seed=seed, onehot=onehot)
    flagged = compare_sample(w, gpu, ora)
    return gpu, ora, flagged


@pytest.mark.parametrize("name", ["tiny", "qwen3_4b", "batched", "verify_b4k4_ctx8192",
                                  "long", "swarm"])
def test_workload_parity(name):
    _log(f"sample parity: workload {name}")
    w = wl.make_workload(name, with_kv=False)
    w.draft_tokens = q_distributed_drafts(w)
    _, _, flagged = _run(w)
    _log(f"  flagged sequences (compared against admissible outcomes): {flagged}")


def test_tiny_sampled_variant():
    w = wl.make_workload("tiny", with_kv=False)
    w = w.with_params([wl.Params(temperature=1.0)])
    for off in range(6):
        w2 = wl.make_workload("tiny", with_kv=False, seed_offset=off)
        w2 = w2.with_params([wl.Params(temperature=1.0)])
        w2.draft_tokens = q_distributed_drafts(w2)
        _log(f"tiny T=1.0 offset {off}")
        _run(w2, seed=off)


def _mixed_batch(batch, vocab, seed, kmax=7, nucleus=False):
    """Many sequences with every parameter combination, ragged K, random counts; with
    `nucleus`, also sequences with a nucleus and no top-k."""
    rng = np.random.default_rng(seed)
    k_per = rng.integers(0, kmax + 1, size=batch)
    rows = k_per + 1
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    t = int(cu[-1])
    target = (3.0 * rng.standard_normal((t, vocab))).astype(np.float32)
    draft = np.empty((t - batch, vocab), np.float32)
    for b in range(batch):
        for s in range(1, rows[b]):
            draft[cu[b] - b + s - 1] = target[cu[b] + s - 1] + 0.5 * rng.standard_normal(vocab)
    counts = rng.integers(0, 3, size=(batch, vocab)).astype(np.int32) * \
        (rng.random((batch, vocab)) < 0.02)
    params = []
    for b in range(batch):
        kind = b % (8 if nucleus else 6)       # kinds 6, 7: a nucleus without top-k
        temp = [0.0, 0.8, 1.0, 0.6, 1.3, 0.7, 0.9, 0.7][kind]
        top_k = [0, 0, 20, 5, 64, 40, 0, 0][kind]
        top_p = [1.0, 1.0, 0.8, 0.95, 1.0, 0.9, 0.9, 0.5][kind]
        pen = b % 4 == 1
        params.append(wl.Params(temperature=temp, top_k=top_k, top_p=top_p,
                                presence_penalty=0.5 if pen else 0.0,
                                frequency_penalty=0.3 if pen else 0.0,
                                logprobs=int(b % 3 == 0), top_logprobs=[0, 5, 3][b % 3]))
    w = wl.Workload(name="mixed", batch=batch, num_q_heads=1, num_kv_heads=1, head_dim=64,
                    dtype=wl.BF16, vocab=vocab, ctx_lens=np.full(batch, 10, np.int32),
                    cu_rows=cu, s_max=0, q=None, k_cache=None, v_cache=None,
                    target_logits=target, draft_logits=draft,
                    draft_tokens=np.zeros(t - batch, np.int32), token_counts=counts.astype(np.int32),
                    params=params, positions=rng.integers(0, 100000, size=batch).astype(np.int32),
                    seed=0)
    w.draft_tokens = q_distributed_drafts(w, seed=seed + 1)
    return w


def test_large_mixed_batch_exception_rate():
    """1200 sequences with mixed parameters; flagged sequences under 0.1%."""
    w = _mixed_batch(1200, 3000, 21)
    _log("mixed batch: 1200 sequences, V=3000")
    _, _, flagged = _run(w, seed=5)
    _log(f"  flagged {flagged} of {w.batch}")
    assert flagged / w.batch < 1e-3


def test_odd_vocab_scalar_path_and_ties():
    """V not a multiple of 4 (scalar loads), integer logits with ties at the top-k
    threshold and at the greedy argmax."""
    rng = np.random.default_rng(3)
    w = _mixed_batch(60, 37, 9, kmax=4, nucleus=True)
    w.target_logits = rng.integers(-3, 4, size=w.target_logits.shape).astype(np.float32)
    w.draft_logits = rng.integers(-3, 4, size=w.draft_logits.shape).astype(np.float32)
    w.draft_tokens = q_distributed_drafts(w, seed=4)
    _log("odd vocab 37 with ties")
    _run(w, seed=1)


def test_edge_cases_k0_and_small_vocab():
    for vocab in (1, 2, 5, 8, 2048, 2049, 4096 + 3):
        w = _mixed_batch(24, vocab, 100 + vocab, kmax=3, nucleus=True)
        for p in w.params:
            p.top_k = min(p.top_k, vocab)          # top_k = V: a nucleus without top-k
            p.top_logprobs = min(p.top_logprobs, 5)
        _log(f"small vocab {vocab}")
        _run(w, seed=vocab)


def test_nucleus_mixed_batch():
    """600 sequences, V=3000, every parameter kind including nuclei without top-k."""
    w = _mixed_batch(600, 3000, 23, nucleus=True)
    _log("mixed batch with nuclei: 600 sequences, V=3000")
    _, _, flagged = _run(w, seed=6)
    _log(f"  flagged {flagged} of {w.batch}")


@pytest.mark.parametrize("temp,top_p,pen", [(0.7, 0.8, False), (0.5, 0.9, True),
                                              (0.6, 0.3, True), (1.0, 0.95, True)])
def test_nucleus_without_top_k(temp, top_p, pen):
    """top_p < 1 and no top-k over the full 151936 vocabulary: the GPU's weighted selection
    gives the full-sort nucleus (kept counts exact), acceptance and draws equal. At T=1.0,
    top_p=0.95 the ids near the cutoff carry ~4e-6 each, so most rows sit inside even the
    tighter margin and are counted, not compared."""
    w = wl.make_workload("verify_b4k4_ctx8192", with_kv=False, seed_offset=int(top_p * 100))
    w = w.with_params([wl.Params(temperature=temp, top_p=top_p,
                                 presence_penalty=0.5 if pen else 0.0,
                                 frequency_penalty=0.3 if pen else 0.0,
                                 logprobs=1)] * w.batch)
    w.draft_tokens = q_distributed_drafts(w)
    _log(f"nucleus without top-k: T={temp} top_p={top_p} penalties={pen}")
    gpu, _, flagged = _run(w, seed=3, max_top_k=1)
    _log(f"  flagged {flagged} of {w.batch} (compared against admissible outcomes)")
    kept = gpu["diag_kept"]
    assert (kept[:, 0] == w.vocab).all() and (kept[:, 1] > 0).all()


def test_nucleus_without_top_k_heavy_ties():
    """Integer logits over the full vocabulary: tens of thousands of ids share the crossing
    value (more than the selection's list holds), all kept or all dropped together."""
    w = wl.make_workload("verify_b4k4_ctx8192", with_kv=False, seed_offset=7)
    rng = np.random.default_rng(8)
    w.target_logits = rng.integers(-3, 4, size=w.target_logits.shape).astype(np.float32)
    w.draft_logits = rng.integers(-3, 4, size=w.draft_logits.shape).astype(np.float32)
    w = w.with_params([wl.Params(temperature=1.0, top_p=0.7)] * w.batch)
    w.draft_tokens = q_distributed_drafts(w)
    _log("nucleus without top-k: integer logits")
    _run(w, seed=4, max_top_k=1)


def test_nucleus_without_top_k_needs_the_truncation_pipeline():
    """With max_top_k = 0 the caller promised no truncation: a nucleus row is refused
    (parameter error bit) and the sequence decodes greedily."""
    w = wl.make_workload("tiny", with_kv=False)
    w = w.with_params([wl.Params(temperature=1.0, top_p=0.9)])
    w.draft_tokens = q_distributed_drafts(w)
    gpu = sample_gpu(w, seed=0, max_top_k=0)
    assert gpu["err"] & 0x04


def test_invalid_inputs_set_error_bits():
    w = _mixed_batch(12, 64, 7, kmax=3)
    w.draft_tokens = w.draft_tokens.copy()
    if w.draft_tokens.size:
        w.draft_tokens[0] = 64                      # out of range: rejected
    gpu = sample_gpu(w, seed=0)
    assert gpu["err"] & 0x02
    ora = sample_oracle(w, seed=0)
    compare_sample(w, gpu, ora)
    bad = w.with_params([wl.Params(temperature=-1.0)] + w.params[1:])
    gpu = sample_gpu(bad, seed=0)
    assert gpu["err"] & 0x04                        # treated as greedy


def test_workspace_reuse_is_stateless():
    w = wl.make_workload("batched", with_kv=False)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    a = sample_gpu(w, seed=3, workspace=ws)
    b = sample_gpu(w, seed=3, workspace=ws)
    for k in ("accepted_len", "out_tokens", "diag_kept"):
        assert np.array_equal(a[k], b[k])


@pytest.mark.parametrize("cfg", [
    dict(temperature=1.0, top_k=0, top_p=1.0, pen=False),
    dict(temperature=1.3, top_k=6, top_p=0.95, pen=True),
    dict(temperature=1.0, top_k=0, top_p=0.85, pen=True),      # nucleus without top-k
])
def test_chi_square_losslessness_on_gpu(cfg):
    """The GPU's emitted tokens follow the (penalized, truncated) target: first token ~ p0,
    P(accept d1) = sum min(p0, q1), second token | accepted ~ p1 (d1 counted)."""
    from scipy import stats
    from oracle import sampling
    rng = np.random.default_rng(77)
    v, n = 8, 200000
    target = (1.0 * rng.standard_normal((3, v))).astype(np.float32)
    draft = (target[:2] + 1.0 * rng.standard_normal((2, v))).astype(np.float32)
    counts = rng.integers(0, 3, size=v).astype(np.int32) if cfg["pen"] else None
    pp, fp = (0.5, 0.3) if cfg["pen"] else (0.0, 0.0)
    prm = wl.Params(temperature=cfg["temperature"], top_k=cfg["top_k"], top_p=cfg["top_p"],
                    presence_penalty=pp, frequency_penalty=fp)
    ctr = np.zeros(v, np.int64) if counts is None else counts.astype(np.int64)
    q = [sampling.truncated_distribution(draft[t], prm.temperature, prm.top_k, prm.top_p).probs
         for t in range(2)]
    d = np.stack([rng.choice(v, size=n, p=q[t]) for t in range(2)], axis=1).astype(np.int32)
    w = wl.Workload(name="chi2", batch=n, num_q_heads=1, num_kv_heads=1, head_dim=64,
                    dtype=wl.BF16, vocab=v, ctx_lens=np.zeros(n, np.int32),
                    cu_rows=np.arange(0, 3 * n + 1, 3, dtype=np.int32), s_max=0, q=None,
                    k_cache=None, v_cache=None, target_logits=np.tile(target, (n, 1)),
                    draft_logits=np.tile(draft, (n, 1)), draft_tokens=d.reshape(-1),
                    token_counts=None if counts is None else np.tile(counts, (n, 1)),
                    params=[prm] * n, positions=np.full(n, 1000, np.int32), seed=0)
    _log(f"chi-square on GPU: {cfg}")
    gpu = sample_gpu(w, seed=11, max_top_k=max(cfg["top_k"], int(cfg["top_p"] < 1.0)))
    assert gpu["err"] == 0
    z0 = sampling.penalized_logits(target[0], ctr, pp, fp)
    p0 = sampling.truncated_distribution(z0, prm.temperature, prm.top_k, prm.top_p).probs
    first = gpu["out_tokens"][0::3]
    obs = np.bincount(first, minlength=v)
    sup = p0 > 0
    assert sup.sum() >= 3, "degenerate test distribution"
    assert obs[~sup].sum() == 0
    assert stats.chisquare(obs[sup], p0[sup] * n).pvalue > 1e-4
    rate = np.minimum(p0, q[0]).sum()
    hits = int(np.count_nonzero(gpu["accepted_len"] >= 1))
    assert stats.binomtest(hits, n, rate).pvalue > 1e-4
    acc = gpu["accepted_len"] >= 1
    x = np.bincount(d[acc, 0], minlength=v).argmax()
    sel = acc & (d[:, 0] == x)
    c1 = ctr.copy()
    c1[x] += 1
    z1 = sampling.penalized_logits(target[1], c1, pp, fp)
    p1 = sampling.truncated_distribution(z1, prm.temperature, prm.top_k, prm.top_p).probs
    obs2 = np.bincount(gpu["out_tokens"][1::3][sel], minlength=v)
    sup1 = p1 > 0
    assert obs2[~sup1].sum() == 0
    assert stats.chisquare(obs2[sup1], p1[sup1] * sel.sum()).pvalue > 1e-4


def test_wait_budget_zero_hands_the_draw_over(monkeypatch):
    """VSA_FUSED_WAIT_US = 0: every workgroup of the fused kernel that is not the last of
    its sequence gives up waiting at once and hands its chunk of the draw to the last
    arriver. Every kernel still ends, the error word says so, and the outputs equal the
    oracle's (the hand-over changes who races a chunk, not the race)."""
    monkeypatch.setenv("VSA_FUSED_WAIT_US", "0")
    for name in ("verify_b4k4_ctx8192", "tiny"):
        w = wl.make_workload(name, with_kv=False)
        if name == "tiny":
            w = w.with_params([wl.Params(temperature=1.0)])
        w.draft_tokens = q_distributed_drafts(w)
        _log(f"wait budget 0: {name}")
        gpu = sample_gpu(w, seed=9)
        assert gpu["err"] & ~0x20 == 0, hex(gpu["err"])
        compare_sample(w, gpu, sample_oracle(w, seed=9))
        # the state the kernel returns to zero serves the next call as usual
        monkeypatch.setenv("VSA_FUSED_WAIT_US", "2000")
        again = sample_gpu(w, seed=9)
        assert again["err"] == 0
        assert np.array_equal(again["out_tokens"], gpu["out_tokens"])
        monkeypatch.setenv("VSA_FUSED_WAIT_US", "0")


@pytest.mark.parametrize("name", ["verify_b4k4_ctx8192", "qwen3_4b", "tiny"])
def test_onehot_proposals_parity(name):
    """One-hot proposals (prompt lookup): the same comparison against the oracle with
    q_t = delta(d_t); fused kernel (no truncation) and truncation pipeline (qwen3_4b)."""
    w = wl.make_workload(name, with_kv=False)
    if name == "tiny":
        w = w.with_params([wl.Params(temperature=1.0)])
    if name == "verify_b4k4_ctx8192":
        w = w.with_params([wl.Params(temperature=0.8, presence_penalty=0.5,
                                     frequency_penalty=0.3, logprobs=1)] * w.batch)
    w.draft_tokens = q_distributed_drafts(w)
    _log(f"one-hot proposals: {name}")
    _run(w, seed=2, onehot=True)


def test_onehot_accept_rate_is_target_probability():
    """P(accept d) = p(d) for a one-hot proposal (binomial over 20000 sequences), and the
    token after a rejection never equals d (the residual is p without d)."""
    from scipy import stats
    from oracle import sampling
    rng = np.random.default_rng(5)
    v, n = 64, 20000
    target = (1.2 * rng.standard_normal((2, v))).astype(np.float32)
    d = int(np.argsort(target[0])[-3])
    p0 = sampling.truncated_distribution(target[0], 1.0, 0, 1.0).probs
    w = wl.Workload(name="onehot", batch=n, num_q_heads=1, num_kv_heads=1, head_dim=64,
                    dtype=wl.BF16, vocab=v, ctx_lens=np.zeros(n, np.int32),
                    cu_rows=np.arange(0, 2 * n + 1, 2, dtype=np.int32), s_max=0, q=None,
                    k_cache=None, v_cache=None, target_logits=np.tile(target, (n, 1)),
                    draft_logits=None, draft_tokens=np.full(n, d, np.int32),
                    token_counts=None, params=[wl.Params(temperature=1.0)] * n,
                    positions=np.arange(n, dtype=np.int32) * 3, seed=0)
    gpu = sample_gpu(w, seed=4, onehot=True)
    assert gpu["err"] == 0
    hits = int(np.count_nonzero(gpu["accepted_len"] == 1))
    assert stats.binomtest(hits, n, p0[d]).pvalue > 1e-4
    first = gpu["out_tokens"][0::2]
    rej = gpu["accepted_len"] == 0
    assert np.all(first[rej] != d)


@pytest.mark.parametrize("batch", [4, 64])
def test_dominant_weight_full_vocabulary_draws(batch):
    """V = 151936, one id at logit 0 and every other at ln(1e-12): the chance that a draw
    leaves the dominant id is ~1.5e-7, so 20480 draws (no drafts: every draw is a race over
    the whole vocabulary) must all return it. A race variate that could reach U = 1 (an
    infinite key) would miss in ~0.9% of draws. B = 4 runs the fused kernel, B = 64 the
    separate race kernel."""
    v = 151936
    rng = np.random.default_rng(6)
    dom = int(rng.integers(0, v))
    row = np.full(v, np.log(1e-12), np.float32)
    row[dom] = 0.0
    calls = 20480 // batch
    w = wl.Workload(name="dominant", batch=batch, num_q_heads=1, num_kv_heads=1,
                    head_dim=64, dtype=wl.BF16, vocab=v, ctx_lens=np.zeros(batch, np.int32),
                    cu_rows=np.arange(batch + 1, dtype=np.int32), s_max=0, q=None,
                    k_cache=None, v_cache=None, target_logits=np.tile(row, (batch, 1)),
                    draft_logits=None, draft_tokens=np.zeros(0, np.int32), token_counts=None,
                    params=[wl.Params(temperature=1.0)] * batch,
                    positions=np.zeros(batch, np.int32), seed=0)
    dev = wl.device_tensors(w, with_kv=False)
    miss = 0
    for c in range(calls):
        dev["positions"].copy_(torch.arange(batch, dtype=torch.int32) * 7 + c * 100003)
        gpu = sample_gpu(w, seed=c, dev=dev)
        assert gpu["err"] == 0
        miss += int(np.count_nonzero(gpu["out_tokens"] != dom))
    _log(f"dominant-weight draws: {calls * batch}, misses {miss}")
    assert miss == 0
