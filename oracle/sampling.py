"""Verify-step logit processing and acceptance, written out step by step (CPU).

TEST INFRASTRUCTURE: part of the CPU oracle. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.

Sources on the pages (mlx-dspark):
  * penalties: Changelog [0.2.0] "Added" (presence/frequency penalties applied to the target
    logits, each verify position by the base completion counts plus its own draft prefix,
    so output equals sequential decoding of the penalized target, temperature > 0 too);
  * logprobs: Changelog [0.2.0] "Added" (raw target log-softmax at each committed token,
    chosen + top entries);
  * top-k threshold and nucleus cutoff, bit-identical to the full-sort definition:
    Changelog [0.20.2] "Changed";
  * truncation applied to both the draft and the target distribution: release v0.1.0
    "Highlights" (lossless top-p / top-k);
  * sampled acceptance: release v0.0.2 "Highlights" (sample the draft, accept with
    probability min(1, p/q), resample the residual on rejection; output distribution equals
    the target's; default greedy);
  * one-hot proposals (prompt-lookup drafts carry no draft distribution; sampling stays an
    exact target sample): Changelog [0.2.0] "Added" (--mode lookup);
  * greedy acceptance: Changelog [0.2.0] "Decode-path performance" (accepted-prefix length
    as a cumulative product of positionwise matches); greedy output equals plain greedy
    decoding (release v0.0.2).

Readings where the pages are silent (each also listed in the design notes):
  R5  penalty form  z = (x - fp*c) - pp*[c>0], fp32, in exactly this operation order;
      applied before temperature.  R6  only target rows are penalized (q is not).
  R7  argmax ties go to the lowest token id.
  R8  top-k is a threshold: theta = k-th largest z (sorted by z desc, id asc); every id with
      z >= theta is kept, so ties at theta are all kept.  R9  top-k selects on z, before /T.
  R10 probabilities are the softmax of z / T over the kept set, evaluated in fp64 from the
      fp32 z as exp((z_j - z_max) / T) (no rounding of z / T to fp32); top-p acts on them:
      sort by z desc (id asc), which is the order of P, m* = first m whose cumulative sum of
      P reaches top_p, keep every id whose z is at least the crossing id's (the crossing id
      and ties with it are kept; ties are ties of z).
  R11 greedy emits the accepted drafts and then the target argmax of the first unmatched
      row (or of the last row when every draft matched).
  R12 a draft whose p and q are both 0 is rejected.  R13 if the residual max(0, p-q) sums
      to 0 the draw falls back to p.
  R14 categorical draws are exponential races: argmax_j r_j / E_j, E_j = -ln U_j with the
      64-bit open-interval uniforms of oracle/philox.py; ties go to the lowest id.
  R15 randoms are keyed (seed, sequence b, absolute position, tag); row i of sequence b
      decides the token at position positions[b] + i.
  R16 logprobs are of the raw target logits (before penalties, temperature, truncation).

Precision: penalized logits z are fp32 (IEEE, one rounding per operation); probabilities,
cumulative sums, acceptance tests and races are fp64; logprobs fp64.

Exception accounting. The GPU takes the same decisions in its own arithmetic; a decision
whose fp64 value lies within the GPU's error bound of the boundary can legitimately go
either way. Every such decision is an exception point with a list of admissible outcomes;
`enumerate_outcomes` follows every combination, so a flagged sequence is still checked: the
GPU's result must equal one of them. The error bounds (ERROR MODEL below) state how far the
GPU's values may sit from the fp64 ones, per precision class of a row:
  "kept"  a row truncated by top-k: the GPU evaluates the same fp64 formulas over the kept
          list (only the summation order differs);
  "full"  a full-vocabulary softmax row: per-id exp2 of fp32 exponents, fp32 chunk sums
          merged in fp64;
  "nuc"   a nucleus over the whole vocabulary (top_p < 1, no top-k): fp64 exponents split
          into integer and fraction, fp32 exp2 of the fraction, fp64 sums;
  "onehot" a one-hot proposal (q(d) = 1 exactly).
"""
from dataclasses import dataclass, field

import numpy as np

from . import philox


@dataclass
class RowParams:
    """Sampling parameters of one sequence (the request parameters the pages list:
    temperature, top_p, top_k, presence/frequency penalty, logprobs, top_logprobs)."""
    temperature: float = 0.0
    top_k: int = 0
    top_p: float = 1.0
    presence_penalty: float = 0.0
    frequency_penalty: float = 0.0
    logprobs: int = 0
    top_logprobs: int = 0


# ----------------------------------------------------------------------------- ERROR MODEL
# Relative error bounds of the GPU's probabilities against the fp64 values (per class), and
# of its race keys; absolute bounds of its cumulative nucleus sums. Stated generously (about
# ten times what the arithmetic gives) and used with a factor 2 below.
REL_KEPT = 1e-12          # fp64 over <= 256 kept ids
REL_FULL_BASE = 2e-6      # full rows: normalizer (fp32 chunk sums) + exp2 + roundings
REL_FULL_PER_LOG2 = 2.4e-7  # ... + per unit of |exponent| in log2 units (its fp32 rounding)
REL_NUC = 2e-6            # whole-vocabulary nuclei: fraction exp2 + fp64 sums
REL_RACE_KEY = 1e-6       # fp32 -log2 U, reciprocal and product of a key
CUM_KEPT = 1e-12          # nucleus cumulative sums over a kept list (fp64)
CUM_NUC = 1e-6            # nucleus cumulative sums over the whole vocabulary
SAFETY = 2.0


def rel_error(cls, z, z_max, temperature):
    """Per-id relative error bound of the GPU's probability in a row of class `cls`."""
    if cls == "kept":
        return np.full(z.shape, REL_KEPT)
    if cls == "nuc":
        return np.full(z.shape, REL_NUC)
    if cls == "onehot":
        return np.zeros(z.shape)
    t = np.abs((z.astype(np.float64) - float(z_max)) / float(temperature)) / np.log(2.0)
    t = np.where(np.isfinite(t), t, 0.0)
    return REL_FULL_BASE + REL_FULL_PER_LOG2 * t


# ----------------------------------------------------------------------------- penalties
def row_counts(base_counts, drafts, i, vocab):
    """c^(i): base completion counts plus the draft prefix d_1..d_i (ids outside the vocab
    are ignored; such a draft is always rejected before its row could be used)."""
    c = np.zeros(vocab, dtype=np.int64) if base_counts is None else \
        np.asarray(base_counts, dtype=np.int64).copy()
    for t in range(i):
        d = int(drafts[t])
        if 0 <= d < vocab:
            c[d] += 1
    return c


def penalized_logits(x, counts, presence, frequency):
    """z = (x - fp*c) - pp*[c>0] in fp32, one rounding per operation (R5)."""
    x = np.asarray(x, dtype=np.float32)
    c32 = np.asarray(counts).astype(np.float32)
    z = x - np.float32(frequency) * c32
    z = z - np.where(np.asarray(counts) > 0, np.float32(presence), np.float32(0.0))
    return z.astype(np.float32)


# ----------------------------------------------------------------------------- ordering
def order_desc(values):
    """Ids sorted by value descending, ties by id ascending (the full-sort definition)."""
    values = np.asarray(values)
    return np.lexsort((np.arange(values.size), -values.astype(np.float64)))


def greedy_token(z):
    """argmax z, lowest id on ties (R7)."""
    return int(order_desc(z)[0])


# ----------------------------------------------------------------------------- truncation
@dataclass
class Truncated:
    probs: np.ndarray        # fp64 [V], renormalized over the kept set S'
    theta: float             # top-k threshold on z (-inf when top-k is off)
    kept_topk: int           # |S|
    kept_nucleus: int        # |S'|
    cls: str                 # precision class of the GPU's values for this row
    rel_err: np.ndarray      # per-id relative error bound of the GPU's probability
    m_star: int = -1         # nucleus crossing rank used (-1: no nucleus)
    m_options: tuple = ()    # crossing ranks within the GPU's error of the boundary


def row_class(vocab, top_k, top_p):
    if 0 < top_k < vocab:
        return "kept"
    return "nuc" if top_p < 1.0 else "full"


def truncated_distribution(z, temperature, top_k, top_p, m_star=None):
    """Softmax of z / T truncated by top-k then top-p (R8-R10), fp64 result. `m_star` forces
    the nucleus crossing rank (an admissible alternative of an exception point)."""
    z = np.asarray(z, dtype=np.float32)
    vocab = z.size
    cls = row_class(vocab, top_k, top_p)
    if cls == "kept":
        theta = np.float32(z[order_desc(z)[top_k - 1]])
        kept = z >= theta
    else:
        theta = np.float32(-np.inf)
        kept = np.ones(vocab, dtype=bool)
    kept_topk = int(np.count_nonzero(kept))
    z64 = z.astype(np.float64)
    zmax = z64[kept].max() if kept.any() else -np.inf
    with np.errstate(invalid="ignore", over="ignore"):
        w = np.where(kept, np.exp((z64 - zmax) / float(np.float32(temperature))), 0.0)
    w = np.where(np.isnan(w), 0.0, w)
    tot = w.sum()
    probs = w / tot if tot > 0 else w
    used_m, options = -1, ()
    if top_p < 1.0 and tot > 0:
        ids = np.flatnonzero(kept)
        ranked = ids[order_desc(z[ids])]
        cum = np.cumsum(probs[ranked])
        reach = np.flatnonzero(cum >= top_p)
        m_def = int(reach[0]) if reach.size else ranked.size - 1
        eps = SAFETY * (CUM_KEPT if cls == "kept" else CUM_NUC)
        opts = [m_def]
        if reach.size and cum[m_def] - top_p <= eps and m_def + 1 < ranked.size:
            opts.append(m_def + 1)          # the GPU may see C_m* just below top_p
        if m_def > 0 and top_p - cum[m_def - 1] <= eps:
            opts.append(m_def - 1)          # ... or C_(m*-1) already at top_p
        options = tuple(opts) if len(opts) > 1 else ()
        used_m = m_def if m_star is None else int(m_star)
        kept = kept & (z >= z[ranked[used_m]])
        probs = np.where(kept, probs, 0.0)
        probs = probs / probs.sum()
    rel = rel_error(cls, z, zmax, temperature)
    return Truncated(probs, float(theta), kept_topk, int(np.count_nonzero(kept)), cls, rel,
                     used_m, options)


def one_hot(d, vocab):
    """A one-hot proposal at draft id d (prompt lookup): q(d) = 1, q = 0 elsewhere."""
    probs = np.zeros(vocab)
    if 0 <= d < vocab:
        probs[d] = 1.0
    return Truncated(probs, float("-inf"), vocab, 1, "onehot", np.zeros(vocab))


# ----------------------------------------------------------------------------- race
ANY = -2                  # a race outcome that admits any token (see race_candidates)
MAX_CANDIDATES = 512


def race_keys(weights, e):
    """Keys w_j / E_j of the exponential race (R14); E_j > 0 always (the uniforms lie in
    the open interval), ids with w_j = 0 never win (key -inf)."""
    weights = np.asarray(weights, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(weights > 0, weights / e, -np.inf)


def race_candidates(weights, delta, e, key_step):
    """The race winner (largest key w / E, lowest id on ties) and every id whose key may
    reach the winner's on the GPU: its weight may sit `delta` (absolute, per id) from the
    fp64 one and its key a further `key_step` (relative) away. An id of weight 0 whose
    delta is positive can thus be a candidate. More than MAX_CANDIDATES candidates (a
    race on weights all within rounding of zero) admit any token (ANY)."""
    weights = np.asarray(weights, dtype=np.float64)
    keys = race_keys(weights, e)
    tok = int(np.argmax(keys))
    if delta is None:
        return tok, [tok]
    w_lo = np.maximum(0.0, weights - SAFETY * delta)
    w_hi = weights + SAFETY * delta
    lo_best = w_lo[tok] / e[tok] * (1.0 - SAFETY * key_step)
    hi = w_hi / e * (1.0 + SAFETY * key_step)
    hi[tok] = -np.inf
    others = np.flatnonzero((hi >= lo_best) & (w_hi > 0))
    if others.size > MAX_CANDIDATES:
        return tok, [tok, ANY]
    return tok, [tok] + [int(j) for j in others]


def exponential_race(weights, seed, b, position, delta=None, key_step=0.0):
    """Categorical draw proportional to `weights` (R14): argmax_j w_j / E_j with E_j from
    the tag-1 stream of (seed, b, position); ties -> lowest id. Returns (token, the ids the
    GPU may pick given per-id weight errors `delta`; [token] when delta is None)."""
    weights = np.asarray(weights, dtype=np.float64)
    e = philox.race_exponentials(seed, b, position, np.arange(weights.size, dtype=np.uint64))
    return race_candidates(weights, delta, e, key_step)


def residual_distribution(p, q):
    """Weights of the resample after a rejection: max(0, p - q), or p if that is all zero
    (R13). Unnormalized; the race needs no normalization."""
    resid = np.maximum(0.0, p - q)
    return p if resid.sum() == 0.0 else resid


def key_step(cls):
    """Relative error of the GPU's race key beyond that of its weight: fp32 -log2 U,
    reciprocal and product for full rows and nuclei; fp64 for kept lists."""
    return 1e-12 if cls == "kept" else REL_RACE_KEY


def weight_delta(p, q=None):
    """Absolute error bound of the GPU's race weights: p alone, or p - q (whose error is the
    sum of both, however much they cancel)."""
    d = p.rel_err * p.probs
    return d if q is None else d + q.rel_err * q.probs


# ----------------------------------------------------------------------------- logprobs
def raw_logprobs(x):
    """log-softmax of the raw target logits in fp64 (R16)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return x - m - np.log(np.exp(x - m).sum())


# ----------------------------------------------------------------------------- acceptance
def accept_test(u, pd, qd, e_p, e_q):
    """Accept the draft iff u q(d) < p(d) (u < min(1, p/q); p = q = 0 rejects, R12).
    Returns (accepted, ambiguous): ambiguous when the GPU's p and q, each within its
    relative error, could put u q(d) on the other side of p(d)."""
    acc = u * qd < pd
    slack = SAFETY * (e_p * pd + e_q * u * qd)
    amb = (pd > 0 or qd > 0) and abs(u * qd - pd) <= slack
    return bool(acc), bool(amb)


# ----------------------------------------------------------------------------- one sequence
@dataclass
class SequenceResult:
    accepted: int
    tokens: list            # emitted tokens (accepted drafts + one target token)
    chosen_logprob: list    # raw logprob of each emitted token at its row
    top_ids: np.ndarray     # [R, n] raw top ids per row
    top_vals: np.ndarray    # [R, n] their raw logprobs
    theta: np.ndarray       # [R] top-k threshold per target row (nan for greedy)
    kept_topk: np.ndarray   # [R]
    kept_nucleus: np.ndarray  # [R] (the fp64 decision)
    kept_options: list = field(default_factory=list)  # [R] admissible |S'| per target row
    points: list = field(default_factory=list)   # exception points met: (key, options)

    @property
    def excepted(self):
        return bool(self.points) or any(len(o) > 1 for o in self.kept_options)


class _Decisions:
    """Forced outcomes of exception points (for enumerate_outcomes) and the record of the
    points met on the way."""

    def __init__(self, forced=None):
        self.forced = dict(forced or {})
        self.points = []

    def take(self, key, default, options):
        """The outcome of decision `key`: the forced one if any, else `default`; the point
        is recorded when more than one outcome is admissible."""
        if len(options) > 1:
            self.points.append((key, tuple(options)))
        return self.forced.get(key, default)


def truncated_versions(logits, params):
    """The row's truncated distribution (first) and, when its nucleus crossing lies within
    the GPU's error of top_p, the distribution at each admissible neighbouring crossing."""
    tr = truncated_distribution(logits, params.temperature, params.top_k, params.top_p)
    out = [tr]
    for m in tr.m_options:
        if m != tr.m_star:
            out.append(truncated_distribution(logits, params.temperature, params.top_k,
                                              params.top_p, m_star=m))
    return out


def _race_over(weights_fn, versions, e, step):
    """Winner under the first version combination and the union of every combination's
    candidates. weights_fn(v) -> (weights, delta) for one combination v."""
    tok, cand = None, []
    for v in versions:
        w, delta = weights_fn(v)
        t, c = race_candidates(w, delta, e, step)
        if tok is None:
            tok = t
        cand += [x for x in c if x not in cand]
    return tok, cand


def verify_sequence(b, target_rows, draft_rows, drafts, base_counts, params, position,
                    seed, n_top, forced=None, one_hot_drafts=False):
    """Verify one sequence: R = K+1 target rows, K draft rows (or None if greedy or one-hot),
    K drafted tokens. Returns the emitted tokens and diagnostics. `forced` maps exception
    points to chosen outcomes (see enumerate_outcomes). A nucleus row whose crossing is
    within the GPU's error of top_p contributes its admissible versions: each decision that
    uses the row is taken under every version, and only a disagreement is a point."""
    dec = _Decisions(forced)
    target_rows = np.asarray(target_rows, dtype=np.float32)
    rows, vocab = target_rows.shape
    k = rows - 1
    z = [penalized_logits(target_rows[i], row_counts(base_counts, drafts, i, vocab),
                          params.presence_penalty, params.frequency_penalty)
         for i in range(rows)]
    theta = np.full(rows, np.nan)
    kept_topk = np.zeros(rows, dtype=np.int64)
    kept_nucleus = np.zeros(rows, dtype=np.int64)
    kept_options = [(0,)] * rows

    def valid(d):
        return 0 <= int(d) < vocab

    if params.temperature == 0.0:
        g = [greedy_token(z[i]) for i in range(rows)]
        a = 0
        while a < k and valid(drafts[a]) and int(drafts[a]) == g[a]:
            a += 1
        tokens = [int(d) for d in drafts[:a]] + [g[a]]
    else:
        p = [truncated_versions(z[i], params) for i in range(rows)]
        if one_hot_drafts:
            q = [None] + [[one_hot(int(drafts[t - 1]), vocab)] for t in range(1, k + 1)]
        else:
            q = [None] + [truncated_versions(draft_rows[t - 1], params)
                          for t in range(1, k + 1)]
        for i in range(rows):
            theta[i], kept_topk[i] = p[i][0].theta, p[i][0].kept_topk
            kept_nucleus[i] = p[i][0].kept_nucleus
            kept_options[i] = tuple(sorted({v.kept_nucleus for v in p[i]}))
        tokens = None
        a = k
        for t in range(1, k + 1):
            pos = position + t - 1
            u = philox.acceptance_uniform(seed, b, pos)
            d = int(drafts[t - 1])
            outcomes = []
            for pv in p[t - 1]:
                for qv in q[t]:
                    pd = pv.probs[d] if valid(d) else 0.0
                    qd = qv.probs[d] if valid(d) else 0.0
                    e_p = pv.rel_err[d] if valid(d) else 0.0
                    e_q = qv.rel_err[d] if valid(d) else 0.0
                    acc, amb = accept_test(u, pd, qd, e_p, e_q)
                    outcomes += [acc, not acc] if amb else [acc]
            opts = [outcomes[0]] + [o for o in (True, False) if o in outcomes[1:] and
                                    o != outcomes[0]]
            acc = dec.take(("acc", t), outcomes[0], tuple(opts))
            if acc:
                continue
            e = philox.race_exponentials(seed, b, pos, np.arange(vocab, dtype=np.uint64))
            step = key_step(p[t - 1][0].cls)
            combos = [(pv, qv) for pv in p[t - 1] for qv in q[t]]

            def resid_race(pq):
                pv, qv = pq
                resid = residual_distribution(pv.probs, qv.probs)
                if resid is pv.probs:
                    return resid, weight_delta(pv)
                return resid, weight_delta(pv, qv)
            tok, cand = _race_over(resid_race, combos, e, step)
            for pv, qv in combos:
                resid = residual_distribution(pv.probs, qv.probs)
                if resid is pv.probs:
                    # R13: the residual is zero everywhere and the draw falls back to p; the
                    # GPU's residual may instead hold rounding-level weights, a race on noise
                    if np.any(weight_delta(pv, qv) > 0) and ANY not in cand:
                        cand.append(ANY)
                elif not np.any(resid > SAFETY * weight_delta(pv, qv)):
                    # every residual weight may round to zero on the GPU: its fallback race
                    # on p is admissible too
                    _, fcand = race_candidates(pv.probs, weight_delta(pv), e, step)
                    cand += [c for c in fcand if c not in cand]
            tok = dec.take(("race", t), tok, cand)
            tokens = [int(x) for x in drafts[:t - 1]] + [int(tok)]
            a = t - 1
            break
        if tokens is None:
            e = philox.race_exponentials(seed, b, position + k, np.arange(vocab, dtype=np.uint64))
            tok, cand = _race_over(lambda pv: (pv.probs, weight_delta(pv)), p[k], e,
                                   key_step(p[k][0].cls))
            tok = dec.take(("race", k + 1), tok, cand)
            tokens = [int(x) for x in drafts[:k]] + [int(tok)]

    lp_rows = [raw_logprobs(target_rows[i]) for i in range(len(tokens))]
    chosen = [float(lp_rows[i][tok]) if tok >= 0 else float("nan")
              for i, tok in enumerate(tokens)]
    top_ids = np.full((rows, n_top), -1, dtype=np.int64)
    top_vals = np.zeros((rows, n_top), dtype=np.float64)
    if n_top:
        for i in range(rows):
            lp = raw_logprobs(target_rows[i])
            ids = order_desc(target_rows[i])[:n_top]
            top_ids[i, :ids.size] = ids
            top_vals[i, :ids.size] = lp[ids]
    return SequenceResult(a, tokens, chosen, top_ids, top_vals, theta, kept_topk,
                          kept_nucleus, kept_options, dec.points)


def enumerate_outcomes(run, limit=4096):
    """Every result that some admissible combination of outcomes at the exception points
    gives. `run(forced)` returns a result with `.points`; the first exception point not yet
    forced is branched over each of its outcomes, recursively."""
    out = []

    def explore(forced):
        res = run(forced)
        free = [(key, opts) for key, opts in res.points if key not in forced]
        if not free:
            out.append(res)
            if len(out) > limit:
                raise RuntimeError("too many admissible outcomes")
            return
        key, opts = free[0]
        for o in opts:
            explore({**forced, key: o})

    explore({})
    return out


# ----------------------------------------------------------------------------- the batch
def verify_sample_accept(target_logits, draft_logits, draft_tokens, cu_rows, token_counts,
                         params, positions, seed, max_top_logprobs=0, one_hot_drafts=False,
                         alternatives=True):
    """Batched verify acceptance with the same argument semantics as the library call.

    target_logits [total_rows, V] f32; draft_logits [total_rows - B, V] f32 or None;
    draft_tokens [total_rows - B] int; cu_rows [B+1]; token_counts [B, V] int or None;
    params: list of RowParams (one per sequence); positions [B] (absolute index of the token
    that row 0 of the sequence decides); seed: 64-bit integer. one_hot_drafts: the drafts
    are one-hot proposals (draft_logits unused).
    Returns a dict of numpy arrays shaped like the library's outputs (the fp64 decisions),
    per-sequence exception flags, and for each flagged sequence the list of admissible
    results (`alternatives[b]`, each a SequenceResult; None when not flagged).
    """
    target_logits = np.asarray(target_logits, dtype=np.float32)
    total_rows, vocab = target_logits.shape
    batch = len(cu_rows) - 1
    n_top = int(max_top_logprobs)
    accepted = np.zeros(batch, dtype=np.int32)
    out_tokens = np.full(total_rows, -1, dtype=np.int32)
    chosen_lp = np.full(total_rows, np.nan, dtype=np.float64)
    top_ids = np.full((total_rows, n_top), -1, dtype=np.int32)
    top_vals = np.zeros((total_rows, n_top), dtype=np.float64)
    theta = np.full(total_rows, np.nan)
    kept_topk = np.zeros(total_rows, dtype=np.int64)
    kept_nucleus = np.zeros(total_rows, dtype=np.int64)
    excepted = np.zeros(batch, dtype=bool)
    alts = [None] * batch
    points = [None] * batch
    kept_opts = [(0,)] * total_rows
    for b in range(batch):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        d0 = r0 - b
        k = r1 - r0 - 1
        prm = params[b]
        drafts = np.asarray(draft_tokens[d0:d0 + k]) if k else np.zeros(0, np.int64)
        drows = None
        if prm.temperature > 0 and k and not one_hot_drafts:
            drows = np.asarray(draft_logits[d0:d0 + k], dtype=np.float32)
        counts = None if token_counts is None else token_counts[b]
        n_req = min(n_top, int(prm.top_logprobs))

        def run(forced, b=b, r0=r0, r1=r1, drows=drows, drafts=drafts, counts=counts,
                prm=prm, n_req=n_req):
            return verify_sequence(b, target_logits[r0:r1], drows, drafts, counts, prm,
                                   int(positions[b]), seed, n_req, forced, one_hot_drafts)

        res = run({})
        accepted[b] = res.accepted
        for i, tok in enumerate(res.tokens):
            out_tokens[r0 + i] = tok
            if prm.logprobs:
                chosen_lp[r0 + i] = res.chosen_logprob[i]
        if n_req:
            top_ids[r0:r1, :n_req] = res.top_ids
            top_vals[r0:r1, :n_req] = res.top_vals
        theta[r0:r1] = res.theta
        kept_topk[r0:r1] = res.kept_topk
        kept_nucleus[r0:r1] = res.kept_nucleus
        excepted[b] = res.excepted
        points[b] = res.points
        kept_opts[r0:r1] = res.kept_options
        if res.excepted and alternatives:
            alts[b] = enumerate_outcomes(run) if res.points else [res]
    return {"accepted_len": accepted, "out_tokens": out_tokens,
            "chosen_logprob": chosen_lp, "top_lp_ids": top_ids, "top_lp_vals": top_vals,
            "topk_threshold": theta, "kept_topk": kept_topk, "kept_nucleus": kept_nucleus,
            "kept_options": kept_opts, "excepted": excepted, "alternatives": alts,
            "points": points}


# ----------------------------------------------------------------------------- draft proposals
def sample_proposals(draft_logits, cu_rows, params, positions, seed):
    """Draw each draft token from its truncated draft distribution q (the drafter's side,
    used by tests that need drafts distributed as q). Draft t of sequence b is drawn at
    position positions[b] + t - 1 from the stream of `seed`; greedy sequences take argmax."""
    batch = len(cu_rows) - 1
    out = np.zeros(int(cu_rows[-1]) - batch, dtype=np.int32)
    for b in range(batch):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        prm = params[b]
        for t in range(1, r1 - r0):
            row = np.asarray(draft_logits[r0 - b + t - 1], dtype=np.float32)
            if prm.temperature == 0.0:
                out[r0 - b + t - 1] = greedy_token(row)
            else:
                q = truncated_distribution(row, prm.temperature, prm.top_k, prm.top_p)
                out[r0 - b + t - 1] = exponential_race(q.probs, seed, b,
                                                       int(positions[b]) + t - 1)[0]
    return out


def widen_draft_logits(draft_logits, d2t, vocab):
    """Reduced draft vocabulary (Changelog [0.8.0] "Added", reduced draft vocabularies): the
    draft head scores only a subset of V_d target tokens, and an offset table maps draft id
    j to target id j + d2t[j]. Before the accept test the draft distribution is widened
    onto the target vocabulary, so the residual still runs over every target id. Written
    out on logits: [rows, V_d] -> [rows, V], target id j + d2t[j] takes draft logit j and
    every other target id -inf (probability 0 after any softmax, truncation or race). The
    widened rows then enter verify_sample_accept unchanged. The table must map the draft
    ids to distinct target ids in [0, V)."""
    dl = np.asarray(draft_logits, dtype=np.float32)
    d2t = np.asarray(d2t, dtype=np.int64)
    rows, dvocab = dl.shape if dl.ndim == 2 else (0, len(d2t))
    if d2t.shape != (dvocab,):
        raise ValueError("d2t must hold one offset per draft id")
    target = np.arange(dvocab, dtype=np.int64) + d2t
    if target.size and (target.min() < 0 or target.max() >= vocab):
        raise ValueError("d2t maps a draft id outside the target vocabulary")
    if len(np.unique(target)) != dvocab:
        raise ValueError("d2t maps two draft ids to one target id")
    out = np.full((rows, vocab), -np.inf, dtype=np.float32)
    out[:, target] = dl.reshape(rows, dvocab)
    return out
