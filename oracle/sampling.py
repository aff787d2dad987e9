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
  * greedy acceptance: Changelog [0.2.0] "Decode-path performance" (accepted-prefix length
    as a cumulative product of positionwise matches); greedy output equals plain greedy
    decoding (release v0.0.2).

Readings where the pages are silent (each also listed in the design notes):
  R5  penalty form  z = (x - fp*c) - pp*[c>0], fp32, in exactly this operation order;
      applied before temperature.  R6  only target rows are penalized (q is not).
  R7  argmax ties go to the lowest token id.
  R8  top-k is a threshold: theta = k-th largest z (sorted by z desc, id asc); every id with
      z >= theta is kept, so ties at theta are all kept.  R9  top-k selects on z, before /T.
  R10 top-p acts on the temperature-scaled probabilities renormalized over the top-k set:
      sort by P desc (id asc), m* = first m whose cumulative sum reaches top_p, cutoff
      c = P_(m*), keep every id with P >= c (the crossing id and ties at it are kept).
  R11 greedy emits the accepted drafts and then the target argmax of the first unmatched
      row (or of the last row when every draft matched).
  R12 a draft whose p and q are both 0 is rejected.  R13 if the residual max(0, p-q) sums
      to 0 the draw falls back to p.
  R14 categorical draws are exponential races: argmax_j r_j / E_j, E_j = -ln U'_j.
  R15 randoms are keyed (seed, sequence b, absolute position, tag); row i of sequence b
      decides the token at position positions[b] + i.
  R16 logprobs are of the raw target logits (before penalties, temperature, truncation).

Precision: penalized logits z and y = z / T are fp32 (IEEE, one rounding per operation);
probabilities, cumulative sums, acceptance tests and races are fp64; logprobs fp64.
"""
from dataclasses import dataclass

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


# Exception margins (fp64) inside which the GPU's fp32 arithmetic may legitimately decide
# the other way; sequences touching one are counted rather than compared.
ACCEPT_MARGIN = 1e-5     # E1: |u - p/q|
NUCLEUS_MARGIN = 1e-5    # E2: |C_m - top_p| at the crossing
RACE_MARGIN = 1e-5       # E3: (best - second) / best of the race keys


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
    nucleus_margin: float    # min distance of the crossing cumulative sums to top_p (inf if off)


def truncated_distribution(z, temperature, top_k, top_p):
    """Temperature softmax of z truncated by top-k then top-p (R8-R10), fp64 result."""
    z = np.asarray(z, dtype=np.float32)
    vocab = z.size
    if 0 < top_k < vocab:
        theta = np.float32(z[order_desc(z)[top_k - 1]])
        kept = z >= theta
    else:
        theta = np.float32(-np.inf)
        kept = np.ones(vocab, dtype=bool)
    kept_topk = int(np.count_nonzero(kept))
    y = (z / np.float32(temperature)).astype(np.float32)          # IEEE fp32 division
    y64 = y.astype(np.float64)
    w = np.where(kept, np.exp(y64 - y64[kept].max()), 0.0)
    probs = w / w.sum()
    margin = np.inf
    if top_p < 1.0:
        ids = np.flatnonzero(kept)
        ranked = ids[order_desc(probs[ids])]
        cum = np.cumsum(probs[ranked])
        reach = np.flatnonzero(cum >= top_p)
        m_star = int(reach[0]) if reach.size else ranked.size - 1
        cutoff = probs[ranked[m_star]]
        margin = abs(cum[m_star] - top_p)
        if m_star > 0:
            margin = min(margin, abs(cum[m_star - 1] - top_p))
        kept = kept & (probs >= cutoff)
        probs = np.where(kept, probs, 0.0)
        probs = probs / probs.sum()
    return Truncated(probs, float(theta), kept_topk, int(np.count_nonzero(kept)), margin)


# ----------------------------------------------------------------------------- race
def race_keys(weights, u):
    """Keys w_j / E_j of the exponential race (R14), E_j = -ln U'_j >= 0 for U' in (0, 1].
    U' = 1 gives E = +0 and an infinite key (computed as 0 - ln U', so that the zero is
    not negative); ids with w_j = 0 never win (key -inf)."""
    weights = np.asarray(weights, dtype=np.float64)
    e = 0.0 - np.log(np.asarray(u, dtype=np.float64))
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(weights > 0, weights / e, -np.inf)


def exponential_race(weights, seed, b, position):
    """Categorical draw proportional to `weights` (R14): argmax_j w_j / E_j with
    E_j = -ln U'_j, U' from the tag-1 stream of (seed, b, position); ties -> lowest id.
    Returns (token, relative gap between the two best keys)."""
    weights = np.asarray(weights, dtype=np.float64)
    u = philox.race_uniforms(seed, b, position, np.arange(weights.size, dtype=np.uint64))
    keys = race_keys(weights, u)
    tok = int(np.argmax(keys))
    order = np.sort(keys)[::-1]
    best, second = order[0], (order[1] if order.size > 1 else -np.inf)
    # A key is +inf only when U' == 1 exactly (E = 0); both sides then break ties by id,
    # so such a draw is exact and carries no margin.
    gap = np.inf if (np.isinf(best) or best <= 0) else (best - second) / best
    return tok, gap


def residual_distribution(p, q):
    """Weights of the resample after a rejection: max(0, p - q), or p if that is all zero
    (R13). Unnormalized; the race needs no normalization."""
    resid = np.maximum(0.0, p - q)
    return p if resid.sum() == 0.0 else resid


# ----------------------------------------------------------------------------- logprobs
def raw_logprobs(x):
    """log-softmax of the raw target logits in fp64 (R16)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return x - m - np.log(np.exp(x - m).sum())


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
    kept_nucleus: np.ndarray  # [R]
    row_nucleus_margin: np.ndarray  # [R] E2 margin per target row (inf if n/a)
    excepted: bool          # an E1/E2/E3 margin was hit on a row that decided the output
    margins: dict           # the smallest margin of each class met on the used rows


def verify_sequence(b, target_rows, draft_rows, drafts, base_counts, params, position,
                    seed, n_top):
    """Verify one sequence: R = K+1 target rows, K draft rows (or None if greedy),
    K drafted tokens. Returns the emitted tokens and diagnostics."""
    target_rows = np.asarray(target_rows, dtype=np.float32)
    rows, vocab = target_rows.shape
    k = rows - 1
    z = [penalized_logits(target_rows[i], row_counts(base_counts, drafts, i, vocab),
                          params.presence_penalty, params.frequency_penalty)
         for i in range(rows)]
    theta = np.full(rows, np.nan)
    kept_topk = np.zeros(rows, dtype=np.int64)
    kept_nucleus = np.zeros(rows, dtype=np.int64)
    row_margin = np.full(rows, np.inf)
    margins = {"accept": np.inf, "nucleus": np.inf, "race": np.inf}

    def valid(d):
        return 0 <= int(d) < vocab

    if params.temperature == 0.0:
        g = [greedy_token(z[i]) for i in range(rows)]
        a = 0
        while a < k and valid(drafts[a]) and int(drafts[a]) == g[a]:
            a += 1
        tokens = [int(d) for d in drafts[:a]] + [g[a]]
    else:
        p = [truncated_distribution(z[i], params.temperature, params.top_k, params.top_p)
             for i in range(rows)]
        q = [None] + [truncated_distribution(draft_rows[t - 1], params.temperature,
                                             params.top_k, params.top_p)
                      for t in range(1, k + 1)]
        for i in range(rows):
            theta[i], kept_topk[i] = p[i].theta, p[i].kept_topk
            kept_nucleus[i], row_margin[i] = p[i].kept_nucleus, p[i].nucleus_margin
        tokens = None
        a = k
        for t in range(1, k + 1):
            pos = position + t - 1
            u = philox.acceptance_uniform(seed, b, pos)
            d = int(drafts[t - 1])
            pd = p[t - 1].probs[d] if valid(d) else 0.0
            qd = q[t].probs[d] if valid(d) else 0.0
            margins["nucleus"] = min(margins["nucleus"], p[t - 1].nucleus_margin,
                                     q[t].nucleus_margin)
            if qd > 0:
                margins["accept"] = min(margins["accept"], abs(u - pd / qd))
            if u * qd < pd:                                      # u < min(1, p/q)
                continue
            tok, gap = exponential_race(residual_distribution(p[t - 1].probs, q[t].probs),
                                        seed, b, pos)
            margins["race"] = min(margins["race"], gap)
            tokens = [int(x) for x in drafts[:t - 1]] + [tok]
            a = t - 1
            break
        if tokens is None:
            margins["nucleus"] = min(margins["nucleus"], p[k].nucleus_margin)
            tok, gap = exponential_race(p[k].probs, seed, b, position + k)
            margins["race"] = min(margins["race"], gap)
            tokens = [int(x) for x in drafts[:k]] + [tok]

    lp_rows = [raw_logprobs(target_rows[i]) for i in range(len(tokens))]
    chosen = [float(lp_rows[i][tok]) for i, tok in enumerate(tokens)]
    top_ids = np.full((rows, n_top), -1, dtype=np.int64)
    top_vals = np.zeros((rows, n_top), dtype=np.float64)
    if n_top:
        for i in range(rows):
            lp = raw_logprobs(target_rows[i])
            ids = order_desc(target_rows[i])[:n_top]
            top_ids[i, :ids.size] = ids
            top_vals[i, :ids.size] = lp[ids]
    excepted = (margins["accept"] < ACCEPT_MARGIN or margins["nucleus"] < NUCLEUS_MARGIN
                or margins["race"] < RACE_MARGIN)
    return SequenceResult(a, tokens, chosen, top_ids, top_vals, theta, kept_topk,
                          kept_nucleus, row_margin, excepted, margins)


# ----------------------------------------------------------------------------- the batch
def verify_sample_accept(target_logits, draft_logits, draft_tokens, cu_rows, token_counts,
                         params, positions, seed, max_top_logprobs=0):
    """Batched verify acceptance with the same argument semantics as the library call.

    target_logits [total_rows, V] f32; draft_logits [total_rows - B, V] f32 or None;
    draft_tokens [total_rows - B] int; cu_rows [B+1]; token_counts [B, V] int or None;
    params: list of RowParams (one per sequence); positions [B] (absolute index of the token
    that row 0 of the sequence decides); seed: 64-bit integer.
    Returns a dict of numpy arrays shaped like the library's outputs, plus per-sequence
    exception flags.
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
    row_margin = np.full(total_rows, np.inf)
    excepted = np.zeros(batch, dtype=bool)
    margins = []
    for b in range(batch):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        d0 = r0 - b
        k = r1 - r0 - 1
        prm = params[b]
        drafts = np.asarray(draft_tokens[d0:d0 + k]) if k else np.zeros(0, np.int64)
        drows = None
        if prm.temperature > 0 and k:
            drows = np.asarray(draft_logits[d0:d0 + k], dtype=np.float32)
        counts = None if token_counts is None else token_counts[b]
        n_req = min(n_top, int(prm.top_logprobs))
        res = verify_sequence(b, target_logits[r0:r1], drows, drafts, counts, prm,
                              int(positions[b]), seed, n_req)
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
        row_margin[r0:r1] = res.row_nucleus_margin
        excepted[b] = res.excepted
        margins.append(res.margins)
    return {"accepted_len": accepted, "out_tokens": out_tokens,
            "chosen_logprob": chosen_lp, "top_lp_ids": top_ids, "top_lp_vals": top_vals,
            "topk_threshold": theta, "kept_topk": kept_topk, "kept_nucleus": kept_nucleus,
            "row_nucleus_margin": row_margin, "excepted": excepted, "margins": margins}


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
