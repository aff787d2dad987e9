"""Pins for the oracle's logit processing and acceptance (oracle/sampling.py).

Pinned against what the pages fix (mlx-dspark release notes / changelog) and against
mathematics rather than against the oracle's own formulas:
  * hand-worked penalty, top-k, top-p and greedy-acceptance cases (tests/golden/*.json);
  * brute-force characterizations of the top-k threshold and the nucleus cutoff that do
    not sort (largest threshold keeping >= k ids / >= top_p mass) on tiny vocabularies;
  * losslessness by chi-square (release v0.0.2 "Highlights": the output distribution equals
    the target's; release v0.1.0: also with top-p / top-k; Changelog [0.2.0]: also with
    penalties): the first emitted token ~ p_0, the next one given acceptance ~ p_1, the
    acceptance rate equals sum_j min(p_0j, q_1j), and the special cases q = p, disjoint
    supports, one-hot proposals (Changelog [0.2.0] prompt lookup) and K = 0;
  * a planted mistake in the residual is caught by the same chi-square;
  * logprob identities (Changelog [0.2.0]: raw target log-softmax).
"""
import concurrent.futures
import json
import math
import multiprocessing as mp
import os

import numpy as np
import pytest
from scipy import stats

from oracle import philox, sampling
from oracle.sampling import RowParams, truncated_distribution, verify_sample_accept

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- penalties
def test_penalties_hand_cases():
    g = _golden("penalties_hand.json")
    for case in g["cases"]:
        c = sampling.row_counts(np.array(case["counts"]), case["drafts"], case["row"],
                                len(case["x"]))
        z = sampling.penalized_logits(np.array(case["x"], np.float32), c, case["presence"],
                                      case["frequency"])
        assert z.dtype == np.float32
        assert z.tolist() == case["z"], case


def test_zero_penalties_are_identity_bitwise():
    rng = np.random.default_rng(0)
    x = (3 * rng.standard_normal(5000)).astype(np.float32)
    counts = rng.integers(0, 50, size=5000)
    z = sampling.penalized_logits(x, counts, 0.0, 0.0)
    assert np.array_equal(z.view(np.uint32), x.view(np.uint32))


def test_penalty_is_single_precision_close_to_exact():
    """Three fp32 operations: within a few fp32 ulps of the exact value of the fp32
    operands (penalties read as fp32 numbers)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000).astype(np.float32)
    counts = rng.integers(1, 2000, size=20000)
    z = sampling.penalized_logits(x, counts, 0.3, 0.7)
    exact = (x.astype(np.float64) - float(np.float32(0.7)) * counts
             - float(np.float32(0.3)))
    ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(z.astype(np.float64) - exact) <= 2.0 * ulp)


# ----------------------------------------------------------------------------- top-k / top-p
def test_topk_hand_cases():
    for case in _golden("truncation_hand.json")["topk"]:
        z = np.array(case["z"], dtype=np.float32)
        tr = truncated_distribution(z, 1.0, case["k"], 1.0)
        assert tr.theta == case["theta"]
        assert np.flatnonzero(tr.probs > 0).tolist() == case["kept"]
        assert tr.kept_topk == len(case["kept"])


def test_nucleus_hand_cases():
    for case in _golden("truncation_hand.json")["nucleus"]:
        z = np.log(np.array(case["logits_ln"], dtype=np.float64)).astype(np.float32)
        tr = truncated_distribution(z, case["T"], case["k"], case["top_p"])
        np.testing.assert_allclose(tr.probs, case["probs"], atol=1e-6)
        assert tr.kept_nucleus == int(np.count_nonzero(np.array(case["probs"]) > 0))


def test_topk_brute_force():
    """theta is the largest value v with #{z >= v} >= k (no sorting involved)."""
    rng = np.random.default_rng(2)
    for _ in range(300):
        v = int(rng.integers(2, 17))
        z = rng.integers(-4, 5, size=v).astype(np.float32)   # many ties
        k = int(rng.integers(1, v))
        tr = truncated_distribution(z, 1.0, k, 1.0)
        theta = max(c for c in set(z.tolist()) if np.count_nonzero(z >= c) >= k)
        assert tr.theta == theta
        assert tr.kept_topk == np.count_nonzero(z >= theta)
        assert np.array_equal(tr.probs > 0, z >= theta)


def test_nucleus_brute_force():
    """S' = {P >= c} for the largest cutoff c among the P values whose kept mass reaches
    top_p (no sorting or scanning involved)."""
    rng = np.random.default_rng(3)
    for _ in range(300):
        v = int(rng.integers(2, 17))
        z = (rng.integers(-6, 7, size=v) * 0.5).astype(np.float32)
        temp = float(rng.choice([0.5, 1.0, 1.7]))
        k = int(rng.choice([0, int(rng.integers(1, v + 1))]))
        top_p = float(rng.uniform(0.05, 0.99))
        tr = truncated_distribution(z, temp, k, top_p)
        base = truncated_distribution(z, temp, k, 1.0).probs
        support = base > 0
        cands = sorted(set(base[support].tolist()), reverse=True)
        cut = next(c for c in cands if base[base >= c].sum() >= top_p - 1e-12)
        if min(abs(base[base >= c].sum() - top_p) for c in cands) < 1e-9:
            continue   # boundary ties in fp64: ambiguous by construction
        keep = support & (base >= cut)
        assert np.array_equal(tr.probs > 0, keep)
        np.testing.assert_allclose(tr.probs[keep], base[keep] / base[keep].sum(), rtol=1e-12)


def test_truncation_special_cases():
    rng = np.random.default_rng(4)
    z = (3 * rng.standard_normal(64)).astype(np.float32)
    one = truncated_distribution(z, 0.9, 1, 1.0)
    assert one.probs[np.argmax(z)] == 1.0 and one.kept_nucleus == 1
    full = truncated_distribution(z, 0.9, 0, 1.0)
    assert np.array_equal(full.probs, truncated_distribution(z, 0.9, 64, 1.0).probs)
    assert full.kept_topk == 64 and full.kept_nucleus == 64
    np.testing.assert_allclose(full.probs.sum(), 1.0, rtol=1e-12)


# ----------------------------------------------------------------------------- greedy
def _greedy_rows(argmaxes, vocab):
    rows = np.zeros((len(argmaxes), vocab), dtype=np.float32)
    for i, g in enumerate(argmaxes):
        rows[i, g] = 5.0
    return rows


def test_greedy_acceptance_hand_cases():
    g = _golden("greedy_accept_hand.json")
    rows = _greedy_rows(g["target_argmax"], g["vocab"])
    for case in g["cases"]:
        res = sampling.verify_sequence(0, rows, None, np.array(case["drafts"]), None,
                                       RowParams(), 10, 0, 0)
        assert res.accepted == case["accepted"]
        assert res.tokens == case["tokens"]


def test_greedy_counts_its_own_draft_prefix():
    """Row 1's presence penalty must see d_1: the target's row-1 argmax flips."""
    x = np.array([[0, 0, 5, 0, 0], [0, 0, 3.0, 0, 2.9], [1, 0, 0, 0, 0]], np.float32)
    prm = RowParams(presence_penalty=0.5)
    res = sampling.verify_sequence(0, x, None, np.array([2, 4]), np.zeros(5, np.int64),
                                   prm, 0, 0, 0)
    assert res.accepted == 2 and res.tokens == [2, 4, 0]
    res = sampling.verify_sequence(0, x, None, np.array([2, 2]), np.zeros(5, np.int64),
                                   prm, 0, 0, 0)
    assert res.accepted == 1 and res.tokens == [2, 4]


def test_greedy_ties_lowest_id():
    x = np.array([[1, 3, 3, 0]], np.float32)
    res = sampling.verify_sequence(0, x, None, np.zeros(0, np.int64), None, RowParams(),
                                   0, 0, 0)
    assert res.tokens == [1]


# ----------------------------------------------------------------------------- sampled
def _batch(target_rows, draft_rows, params, n, seed=0, counts=None, draft_seed=1):
    """n identical sequences (b = 0..n-1); drafts drawn from q with `draft_seed`."""
    r = target_rows.shape[0]
    tl = np.tile(target_rows, (n, 1))
    dl = np.tile(draft_rows, (n, 1)) if r > 1 else np.zeros((0, target_rows.shape[1]),
                                                           np.float32)
    cu = np.arange(0, n * r + 1, r)
    prms = [params] * n
    pos = np.full(n, 100)
    drafts = sampling.sample_proposals(dl, cu, prms, pos, draft_seed) if r > 1 else \
        np.zeros(0, np.int32)
    cts = None if counts is None else np.tile(counts, (n, 1))
    out = verify_sample_accept(tl, dl, drafts, cu, cts, prms, pos, seed)
    return out, drafts.reshape(n, r - 1) if r > 1 else None


def _chi2_ok(observed_tokens, probs, min_expected=5.0):
    probs = np.asarray(probs, dtype=np.float64)
    obs = np.bincount(observed_tokens, minlength=probs.size).astype(np.float64)
    n = obs.sum()
    support = probs * n >= min_expected
    assert obs[probs == 0].sum() == 0, "token outside the support"
    exp_s = probs[support] * n
    obs_s = obs[support]
    # lump the rare tail into one bin
    rest_e, rest_o = n - exp_s.sum(), n - obs_s.sum()
    if rest_e > 0:
        exp_s, obs_s = np.append(exp_s, rest_e), np.append(obs_s, rest_o)
    return stats.chisquare(obs_s, exp_s).pvalue


def _rows(rng, r, v, sd=1.5):
    return (sd * rng.standard_normal((r, v))).astype(np.float32)


N_TRIALS = 12000


@pytest.fixture(scope="module")
def plain_case():
    rng = np.random.default_rng(10)
    v = 8
    target = _rows(rng, 3, v)
    draft = (target[:2] + 1.0 * rng.standard_normal((2, v))).astype(np.float32)
    prm = RowParams(temperature=1.0)
    out, drafts = _batch(target, draft, prm, N_TRIALS)
    return target, draft, prm, out, drafts


def test_first_token_follows_target(plain_case):
    target, draft, prm, out, _ = plain_case
    first = out["out_tokens"][0::3]
    p0 = truncated_distribution(target[0], 1.0, 0, 1.0).probs
    assert _chi2_ok(first, p0) > 1e-3


def test_acceptance_rate_closed_form(plain_case):
    target, draft, prm, out, _ = plain_case
    p0 = truncated_distribution(target[0], 1.0, 0, 1.0).probs
    q1 = truncated_distribution(draft[0], 1.0, 0, 1.0).probs
    rate = np.minimum(p0, q1).sum()
    hits = int(np.count_nonzero(out["accepted_len"] >= 1))
    assert stats.binomtest(hits, N_TRIALS, rate).pvalue > 1e-3


def test_second_token_given_acceptance(plain_case):
    target, draft, prm, out, _ = plain_case
    acc = out["accepted_len"] >= 1
    second = out["out_tokens"][1::3][acc]
    p1 = truncated_distribution(target[1], 1.0, 0, 1.0).probs
    assert _chi2_ok(second, p1) > 1e-3


def test_lossless_with_penalties_and_truncation():
    rng = np.random.default_rng(11)
    v = 12
    target = _rows(rng, 3, v, sd=1.2)
    draft = (target[:2] + 0.8 * rng.standard_normal((2, v))).astype(np.float32)
    counts = rng.integers(0, 3, size=v)
    prm = RowParams(temperature=0.7, top_k=6, top_p=0.9, presence_penalty=0.5,
                    frequency_penalty=0.3)
    out, drafts = _batch(target, draft, prm, N_TRIALS, counts=counts)
    z0 = sampling.penalized_logits(target[0], counts, 0.5, 0.3)
    p0 = truncated_distribution(z0, 0.7, 6, 0.9).probs
    assert _chi2_ok(out["out_tokens"][0::3], p0) > 1e-3
    # second token, given d_1 = x accepted, follows row 1 penalized with x counted
    acc = out["accepted_len"] >= 1
    x = np.bincount(drafts[acc, 0]).argmax()
    sel = acc & (drafts[:, 0] == x)
    c1 = counts.copy()
    c1[x] += 1
    p1 = truncated_distribution(sampling.penalized_logits(target[1], c1, 0.5, 0.3), 0.7, 6,
                                0.9).probs
    assert _chi2_ok(out["out_tokens"][1::3][sel], p1) > 1e-3


def test_q_equal_p_accepts_everything():
    rng = np.random.default_rng(12)
    target = _rows(rng, 3, 10)
    prm = RowParams(temperature=0.9, top_k=5)
    out, _ = _batch(target, target[:2].copy(), prm, 2000)
    assert np.all(out["accepted_len"] == 2)


def test_disjoint_supports_reject_and_resample_from_p():
    v = 8
    target = np.full((2, v), -5.0, np.float32)
    target[:, :2] = [2.0, 1.0]
    draft = np.full((1, v), -5.0, np.float32)
    draft[0, 5:7] = [2.0, 1.5]
    prm = RowParams(temperature=1.0, top_k=2)
    out, _ = _batch(target, draft, prm, 6000)
    assert np.all(out["accepted_len"] == 0)
    p0 = truncated_distribution(target[0], 1.0, 2, 1.0).probs
    assert _chi2_ok(out["out_tokens"][0::2], p0) > 1e-3


def test_one_hot_proposal_accept_probability():
    """A one-hot proposal q at d (prompt lookup, Changelog [0.2.0]): P(accept) = p(d)."""
    rng = np.random.default_rng(13)
    v, n = 8, 8000
    target = _rows(rng, 2, v)
    draft = np.zeros((1, v), np.float32)
    draft[0, 3] = 60.0                       # q(3) = 1 - O(e^-60): one-hot in fp64
    p_full = truncated_distribution(target[0], 1.0, 0, 1.0).probs
    tl, dl = np.tile(target, (n, 1)), np.tile(draft, (n, 1))
    cu = np.arange(0, 2 * n + 1, 2)
    out = verify_sample_accept(tl, dl, np.full(n, 3, np.int32), cu, None,
                               [RowParams(temperature=1.0)] * n, np.full(n, 5), 0)
    hits = int(np.count_nonzero(out["accepted_len"] == 1))
    assert stats.binomtest(hits, n, p_full[3]).pvalue > 1e-3


def test_no_drafts_is_plain_sampling():
    rng = np.random.default_rng(14)
    target = _rows(rng, 1, 9)
    prm = RowParams(temperature=1.3, top_p=0.95)
    out, _ = _batch(target, np.zeros((0, 9), np.float32), prm, 8000)
    p0 = truncated_distribution(target[0], 1.3, 0, 0.95).probs
    assert np.all(out["accepted_len"] == 0)
    assert _chi2_ok(out["out_tokens"], p0) > 1e-3


def test_exponential_race_is_categorical():
    w = np.array([0.5, 0.0, 2.0, 1.0, 0.25, 4.0])
    toks = np.array([sampling.exponential_race(w, 5, 0, p)[0] for p in range(20000)])
    assert _chi2_ok(toks, w / w.sum()) > 1e-3


def test_race_keys_are_finite_for_every_variate():
    """E lies in [2^-65, 65 ln 2] (open-interval uniforms), so a positive weight always has
    a finite positive key and a zero weight never wins, whatever the variate."""
    m = 0xFFFFFFFF
    e = philox.exponential64(np.array([0, m, m, 2 ** 31], np.uint64),
                             np.array([0, m, 0, 0], np.uint64))
    keys = sampling.race_keys(np.array([1.0, 1e-300, 0.0, 2.0]), e)
    assert np.all(np.isfinite(keys[[0, 1, 3]])) and keys[2] == -np.inf
    assert e.min() == 2.0 ** -65 and e.max() < 45.06


def _dominant_draws(args):
    lo, hi = args
    w = np.full(151936, 1e-12)
    w[777] = 1.0
    return sum(int(sampling.exponential_race(w, 42, 0, p)[0] != 777) for p in range(lo, hi))


def test_dominant_weight_at_full_vocabulary():
    """V = 151936, one id of weight 1, every other 1e-12: the exact chance that the draw
    leaves the dominant id is sum_j w_j / sum w ~ 1.5e-7 per draw, so in 20000 draws the
    count must be 0 (binomial, P(0) ~ 0.997). A uniform that can reach 1 (an infinite key
    for whichever id draws it) would leave it in ~0.9% of draws (V 2^-24), ~180 times."""
    n, parts = 20000, 16
    step = n // parts
    with concurrent.futures.ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1),
                                                mp_context=mp.get_context("fork")) as ex:
        bad = sum(ex.map(_dominant_draws, [(i * step, (i + 1) * step) for i in range(parts)]))
    assert bad == 0


# ----------------------------------------------------------------------------- exception points
def test_accept_margin_pins():
    """E1: u q(d) within the GPU's relative error of p(d) is ambiguous; clearly apart is
    not. Here e_p = e_q = 2e-6 (full rows) and SAFETY = 2: slack ~ 8e-6 p."""
    p, q = 0.4, 0.5
    u_edge = p / q
    for rel, amb in [(5e-7, True), (-5e-7, True), (3e-6, True), (-1e-3, False),
                     (1e-3, False), (2e-5, False)]:
        u = u_edge * (1 + rel)
        acc, a = sampling.accept_test(u, p, q, 2e-6, 2e-6)
        assert acc == (u * q < p)
        assert a == amb, (rel, a)
    # kept-list rows (fp64 on the GPU): only rounding-level distances are ambiguous
    assert sampling.accept_test(u_edge * (1 + 1e-13), p, q, 1e-12, 1e-12)[1]
    assert not sampling.accept_test(u_edge * (1 + 1e-9), p, q, 1e-12, 1e-12)[1]
    # p = q = 0 rejects, unambiguously (R12)
    assert sampling.accept_test(0.3, 0.0, 0.0, 2e-6, 2e-6) == (False, False)


def _nucleus_row(cum_at_cross, top_p, v=64):
    """fp32 logits whose sorted probabilities put the cumulative mass after the first two
    ids at `cum_at_cross`; T = 1. Returns z."""
    rest = (1.0 - cum_at_cross) / (v - 2)
    pr = np.array([cum_at_cross * 0.6, cum_at_cross * 0.4] + [rest] * (v - 2))
    return np.log(pr).astype(np.float32)


def test_nucleus_margin_pins():
    """E2: the crossing cumulative sum within the GPU's error of top_p offers the
    neighbouring crossing rank; a distance of 1e-3 does not. Whole-vocabulary nucleus rows
    (GPU error 1e-6, x2) and top-k rows (fp64 kept lists, 1e-12, x2)."""
    for d, opts in [(5e-7, True), (1.5e-6, True), (1e-3, False), (-1e-3, False)]:
        z = _nucleus_row(0.5, 0.5)
        c2 = float(np.cumsum(np.sort(np.exp(z.astype(np.float64)) /
                                     np.exp(z.astype(np.float64)).sum())[::-1])[1])
        top_p = np.float32(c2 - d)
        tr = truncated_distribution(z, 1.0, 0, float(top_p))
        assert tr.cls == "nuc"
        assert bool(tr.m_options) == opts, (d, tr.m_options)
    z = _nucleus_row(0.5, 0.5)
    zk = np.concatenate([z, np.full(8, -30, np.float32)])
    pr = np.exp(zk.astype(np.float64) - zk.max())
    top = np.sort(pr[pr > np.exp(-29.0)])[::-1]
    for d, opts in [(1e-13, True), (1e-9, False)]:
        c = float(np.cumsum(top / top.sum())[1])
        tr = truncated_distribution(zk, 1.0, 64, c - d)
        assert tr.cls == "kept" and bool(tr.m_options) == opts, (d, tr.m_options)


def test_race_margin_pins():
    """E3: two keys within the GPU's key error are both candidates; 1e-3 apart, only the
    winner. Explicit exponentials, so the keys are known."""
    e = np.array([1.0, 1.0, 2.0])
    w_tie = np.array([1.0, 1.0 - 1e-7, 0.1])
    tok, cand = sampling.race_candidates(w_tie, 2e-6 * w_tie, e, 1e-6)
    assert tok == 0 and sorted(cand) == [0, 1]
    w_far = np.array([1.0, 1.0 - 1e-3, 0.1])
    tok, cand = sampling.race_candidates(w_far, 2e-6 * w_far, e, 1e-6)
    assert tok == 0 and cand == [0]
    # a zero-weight id whose GPU weight may be positive competes only through its bound
    w0 = np.array([1e-6, 0.0])
    tok, cand = sampling.race_candidates(w0, np.array([0.0, 1e-6]), np.array([1.0, 0.5]), 0)
    assert tok == 0 and cand == [0, 1]
    tok, cand = sampling.race_candidates(w0, None, np.array([1.0, 0.5]), 0)
    assert cand == [0]


def test_enumerate_outcomes_follows_every_ambiguous_decision():
    """A sequence whose first acceptance test sits on the boundary: both branches are
    admissible results (accept: the second draft is tested too; reject: a residual draw)."""
    rng = np.random.default_rng(30)
    v = 16
    target = _rows(rng, 3, v)
    draft = (target[:2] + 0.5 * rng.standard_normal((2, v))).astype(np.float32)
    prm = RowParams(temperature=1.0)
    drafts = np.array([3, 5])
    base = sampling.verify_sequence(0, target, draft, drafts, None, prm, 10, 7, 0)
    forced_runs = []

    def run(forced):
        forced_runs.append(dict(forced))
        res = sampling.verify_sequence(0, target, draft, drafts, None, prm, 10, 7, 0, forced)
        res.points = [(("acc", 1), (True, False))] + res.points
        return res
    outs = sampling.enumerate_outcomes(run)
    accs = sorted({o.accepted for o in outs})
    assert accs[0] == 0 and accs[-1] >= 1
    assert any(o.tokens == base.tokens for o in outs)


def test_one_hot_proposals_accept_and_resample():
    """One-hot proposals (prompt lookup, Changelog [0.2.0]): P(accept) = p(d), and after a
    rejection the token follows p without d (the residual max(0, p - delta_d))."""
    rng = np.random.default_rng(31)
    v, n = 8, 12000
    target = _rows(rng, 2, v)
    tl = np.tile(target, (n, 1))
    cu = np.arange(0, 2 * n + 1, 2)
    out = verify_sample_accept(tl, None, np.full(n, 3, np.int32), cu, None,
                               [RowParams(temperature=1.0)] * n, np.arange(n) * 2, 0,
                               one_hot_drafts=True)
    p = truncated_distribution(target[0], 1.0, 0, 1.0).probs
    hits = int(np.count_nonzero(out["accepted_len"] == 1))
    assert stats.binomtest(hits, n, p[3]).pvalue > 1e-3
    rej = out["accepted_len"] == 0
    resid = p.copy()
    resid[3] = 0.0
    assert _chi2_ok(out["out_tokens"][0::2][rej], resid / resid.sum()) > 1e-3


def test_planted_residual_mistake_is_caught(monkeypatch):
    """If the resample ignored q (used p instead of max(0, p - q)), the first emitted token
    would be biased towards the draft; the same chi-square must reject it."""
    rng = np.random.default_rng(15)
    v = 6
    target = _rows(rng, 2, v)
    draft = (target[:1] + 1.5 * rng.standard_normal((1, v))).astype(np.float32)
    prm = RowParams(temperature=1.0)
    monkeypatch.setattr(sampling, "residual_distribution", lambda p, q: p)
    out, _ = _batch(target, draft, prm, N_TRIALS)
    p0 = truncated_distribution(target[0], 1.0, 0, 1.0).probs
    assert _chi2_ok(out["out_tokens"][0::2], p0) < 1e-6


# ----------------------------------------------------------------------------- logprobs
def test_logprob_identities():
    rng = np.random.default_rng(16)
    x = (3 * rng.standard_normal(1000)).astype(np.float32)
    lp = sampling.raw_logprobs(x)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-12
    np.testing.assert_allclose(sampling.raw_logprobs(x + np.float32(7.0)), lp, atol=1e-5)
    u = sampling.raw_logprobs(np.zeros(151936, np.float32))
    np.testing.assert_allclose(u, -math.log(151936), rtol=1e-14)


def test_logprob_outputs_of_a_batch():
    x = np.array([[1, 3, 3, 2], [0, 0, 9, 0]], np.float32)
    prm = RowParams(logprobs=1, top_logprobs=3)
    out = verify_sample_accept(x, np.zeros((1, 4), np.float32), np.array([2]),
                               np.array([0, 2]), None, [prm], np.array([0]), 0, 3)
    assert out["accepted_len"].tolist() == [0]
    assert out["out_tokens"].tolist() == [1, -1]
    assert out["top_lp_ids"][0].tolist() == [1, 2, 3]
    lp0 = sampling.raw_logprobs(x[0])
    assert out["chosen_logprob"][0] == lp0[1] and np.isnan(out["chosen_logprob"][1])
    np.testing.assert_allclose(out["top_lp_vals"][0], lp0[[1, 2, 3]])
