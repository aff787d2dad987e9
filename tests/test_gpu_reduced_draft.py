"""GPU parity of the reduced-draft-vocabulary path (draft_vocab_inverse and
verify_sample_accept_reduced_draft) against the CPU oracle run on the widened draft rows,
through the C ABI, with the bar of the full-vocabulary tests: accepted lengths, tokens,
thresholds and kept sizes bit-exact outside the oracle's counted margins, logprobs within
2e-5. The inverse table itself is compared bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_step_attention_amd as vsa  # noqa: E402
from verify_step_attention_amd import workloads as wl  # noqa: E402
from gpu_helpers import (compare_sample, q_distributed_drafts, sample_gpu,  # noqa: E402
                         sample_oracle)


def _log(msg):
    print(msg, flush=True)


def _reduce(w, dvocab, seed, keep_drafts=True):
    """A sorted subset of dvocab target ids (holding every draft token when keep_drafts),
    its offset table, and the workload with the draft rows restricted to it."""
    rng = np.random.default_rng(seed)
    must = np.unique(w.draft_tokens) if keep_drafts else np.zeros(0, np.int64)
    rest = np.setdiff1d(np.arange(w.vocab), must)
    subset = np.sort(np.concatenate([must, rng.choice(rest, dvocab - must.size,
                                                      replace=False)])).astype(np.int64)
    d2t = (subset - np.arange(dvocab)).astype(np.int32)
    reduced = np.ascontiguousarray(w.draft_logits[:, subset])
    return subset, d2t, reduced


def _inverse_gpu(d2t, vocab):
    t2d = torch.empty(vocab, dtype=torch.int32, device="cuda")
    vsa.draft_vocab_inverse(torch.from_numpy(d2t).cuda(), vocab, t2d)
    torch.cuda.synchronize()
    return t2d


def _run_reduced(w, subset, d2t, reduced, seed=0, max_top_k=None):
    from oracle.sampling import widen_draft_logits
    t2d = _inverse_gpu(d2t, w.vocab)
    ref = np.full(w.vocab, -1, np.int32)
    ref[subset] = np.arange(len(subset))
    assert np.array_equal(t2d.cpu().numpy(), ref)
    gpu = sample_gpu(w, seed=seed, reduced=(torch.from_numpy(reduced).cuda(), t2d),
                     max_top_k=max_top_k)
    wide = w.with_params(w.params)
    wide.draft_logits = widen_draft_logits(reduced, d2t, w.vocab)
    ora = sample_oracle(wide, seed=seed)
    return gpu, compare_sample(w, gpu, ora)


@pytest.mark.parametrize("name,dvocab", [("qwen3_4b", 32000), ("batched", 32000),
                                         ("verify_b4k4_ctx8192", 32000), ("long", 32000),
                                         ("swarm", 16384)])
def test_workload_parity(name, dvocab):
    _log(f"reduced draft vocabulary parity: {name}, V_d {dvocab}")
    w = wl.make_workload(name, with_kv=False)
    subset, d2t, reduced = _reduce(w, dvocab, seed=11)
    # proposals drawn from the widened draft distribution (so every draft is in the subset)
    from oracle.sampling import widen_draft_logits
    wide = w.with_params(w.params)
    wide.draft_logits = widen_draft_logits(reduced, d2t, w.vocab)
    w.draft_tokens = q_distributed_drafts(wide)
    assert np.isin(w.draft_tokens, subset).all()
    gpu, flagged = _run_reduced(w, subset, d2t, reduced)
    assert gpu["err"] == 0, hex(gpu["err"])
    assert flagged <= max(1, w.batch // 8)


@pytest.mark.parametrize("vocab", [1024, 1001])
def test_small_vocab_sampled_with_drafts_outside_subset(vocab):
    """Odd vocabulary (scalar loads), and drafts that the subset does not hold (their q is
    0: accepted with probability 1 when p > 0, R12 when p is 0 too)."""
    for off in range(4):
        _log(f"reduced draft vocabulary: tiny V {vocab} offset {off}")
        w = wl.make_workload("tiny", with_kv=False, seed_offset=off, vocab=vocab)
        w = w.with_params([wl.Params(temperature=1.0, top_k=40 if off % 2 else 0)])
        w.draft_tokens = q_distributed_drafts(w)
        subset, d2t, reduced = _reduce(w, 257, seed=off, keep_drafts=off < 2)
        gpu, _ = _run_reduced(w, subset, d2t, reduced, seed=off)
        assert gpu["err"] == 0, hex(gpu["err"])


def test_identity_table_matches_full_vocabulary_call():
    _log("reduced draft vocabulary: identity table == verify_sample_accept (bitwise)")
    w = wl.make_workload("batched", with_kv=False)
    w.draft_tokens = q_distributed_drafts(w)
    t2d = _inverse_gpu(np.zeros(w.vocab, np.int32), w.vocab)
    full = sample_gpu(w)
    red = sample_gpu(w, reduced=(torch.from_numpy(w.draft_logits).cuda(), t2d))
    for k in full:
        assert np.array_equal(np.asarray(full[k]), np.asarray(red[k]), equal_nan=True), k


def test_bad_inverse_entries_set_error_bit():
    _log("reduced draft vocabulary: t2d entries out of range -> error bit, read as -1")
    w = wl.make_workload("batched", with_kv=False)
    w.draft_tokens = q_distributed_drafts(w)
    subset, d2t, reduced = _reduce(w, 32000, seed=3)
    t2d = _inverse_gpu(d2t, w.vocab)
    bad = t2d.clone()
    bad[5] = 40000                        # beyond V_d: must read as "no draft id"
    bad[7] = -9
    gpu = sample_gpu(w, reduced=(torch.from_numpy(reduced).cuda(), bad))
    assert gpu["err"] & vsa.DEVERR_DRAFT_MAP


def test_reduced_draft_with_nucleus_without_top_k():
    """Nucleus rows without top-k whose draft rows come through the inverse table."""
    w = wl.make_workload("verify_b4k4_ctx8192", with_kv=False, seed_offset=3)
    w = w.with_params([wl.Params(temperature=0.6, top_p=0.85)] * w.batch)
    w.draft_tokens = q_distributed_drafts(w)
    subset, d2t, reduced = _reduce(w, 32000, 12)
    _log("reduced draft vocabulary 32000 with nuclei without top-k")
    _, flagged = _run_reduced(w, subset, d2t, reduced, seed=2, max_top_k=1)
    assert flagged <= 1
