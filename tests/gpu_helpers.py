"""Helpers for the GPU parity tests: run the library on a workload through the C ABI."""
import numpy as np
import torch

import verify_step_attention_amd as vsa
from verify_step_attention_amd import workloads as wl


def attention_gpu(w, dev=None, max_kv_len=None, workspace=None, stream=None, flags=0):
    """Returns (out float32 numpy [T, Hq, D], device error word)."""
    dev = dev or wl.device_tensors(w)
    mkv = max_kv_len or w.max_kv_len
    size = vsa.verify_attention_workspace_size(w.batch, w.num_q_heads, w.num_kv_heads,
                                               w.head_dim, w.max_rows, mkv)
    assert size > 0
    ws = workspace if workspace is not None else torch.zeros(size, dtype=torch.uint8,
                                                             device="cuda")
    ws[:4].zero_()
    out = torch.full((w.total_rows, w.num_q_heads, w.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    vsa.verify_attention(dev["q"], dev["k_cache"], dev["v_cache"], dev["cu_rows"],
                         dev["ctx_lens"], out, ws, max_rows_per_seq=w.max_rows,
                         max_kv_len=mkv, flags=flags, stream=stream)
    torch.cuda.synchronize()
    err = int(ws[:4].view(torch.int32).item())
    return out.cpu().numpy(), err


def attention_oracle(w):
    from oracle.attention import verify_attention
    k, v = w.kv_f32()
    return verify_attention(w.q_f32(), k, v, w.cu_rows, w.ctx_lens, w.num_q_heads,
                            w.num_kv_heads)


ATOL, RTOL = 1e-3, 2e-3


def assert_attention_close(got, ref):
    bad = np.abs(got - ref) > ATOL + RTOL * np.abs(ref)
    assert not np.isnan(got).any(), "NaN in output"
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} elements out of tolerance; "
                           f"max abs err {np.nanmax(np.abs(got - ref)):.3e}")


# ----------------------------------------------------------------------------- sampling
def oracle_params(params):
    from oracle.sampling import RowParams
    return [RowParams(p.temperature, p.top_k, p.top_p, p.presence_penalty,
                      p.frequency_penalty, p.logprobs, p.top_logprobs) for p in params]


def q_distributed_drafts(w, seed=1):
    """Draft tokens drawn from the truncated draft distribution q (the oracle's sampler)."""
    from oracle.sampling import sample_proposals
    if w.total_rows == w.batch:
        return np.zeros(0, np.int32)
    return sample_proposals(w.draft_logits, w.cu_rows, oracle_params(w.params), w.positions,
                            seed).astype(np.int32)


def sample_gpu(w, seed=0, max_top_k=None, max_top_lp=None, workspace=None, dev=None,
               reduced=None, onehot=False):
    """reduced: (draft logits [T-B, V_d] device tensor, t2d [V] device tensor) to call
    verify_sample_accept_reduced_draft instead; onehot: call verify_sample_accept_onehot
    (the drafts are one-hot proposals, no draft logits)."""
    dev = dev or wl.device_tensors(w, with_kv=False)
    mtk = max_top_k if max_top_k is not None else max([p.top_k for p in w.params] + [0])
    mtl = max_top_lp if max_top_lp is not None else max([p.top_logprobs for p in w.params] + [0])
    size = vsa.verify_sample_accept_workspace_size(w.batch, w.total_rows, w.vocab, w.max_rows,
                                                   mtk, mtl)
    assert size > 0
    ws = workspace if workspace is not None else torch.zeros(size, dtype=torch.uint8,
                                                             device="cuda")
    ws[:4].zero_()
    params = torch.from_numpy(vsa.pack_row_params(w.params).view(np.uint8)).cuda()
    t = w.total_rows
    out = {
        "accepted_len": torch.full((w.batch,), -7, dtype=torch.int32, device="cuda"),
        "out_tokens": torch.full((t,), -7, dtype=torch.int32, device="cuda"),
        "chosen_logprob": torch.full((t,), 7.0, dtype=torch.float32, device="cuda"),
        "top_lp_vals": torch.full((t, max(mtl, 1)), 7.0, dtype=torch.float32, device="cuda"),
        "top_lp_ids": torch.full((t, max(mtl, 1)), -7, dtype=torch.int32, device="cuda"),
        "diag_threshold": torch.full((t,), 7.0, dtype=torch.float32, device="cuda"),
        "diag_kept": torch.full((t, 2), -7, dtype=torch.int32, device="cuda"),
    }
    sampled = any(p.temperature > 0 for p in w.params)
    opt = dict(max_rows_per_seq=w.max_rows, max_top_k=mtk, max_top_logprobs=mtl,
               chosen_logprob=out["chosen_logprob"], top_lp_vals=out["top_lp_vals"],
               top_lp_ids=out["top_lp_ids"], diag_threshold=out["diag_threshold"],
               diag_kept=out["diag_kept"])
    if onehot:
        vsa.verify_sample_accept_onehot(dev["target_logits"], dev["draft_tokens"],
                                        dev["cu_rows"], dev["token_counts"], params,
                                        dev["positions"], seed, out["accepted_len"],
                                        out["out_tokens"], ws, **opt)
    elif reduced is None:
        draft_logits = dev["draft_logits"] if sampled else None
        vsa.verify_sample_accept(dev["target_logits"], draft_logits, dev["draft_tokens"],
                                 dev["cu_rows"], dev["token_counts"], params, dev["positions"],
                                 seed, out["accepted_len"], out["out_tokens"], ws, **opt)
    else:
        draft_logits, t2d = reduced
        vsa.verify_sample_accept_reduced_draft(
            dev["target_logits"], draft_logits if sampled else None, t2d, dev["draft_tokens"],
            dev["cu_rows"], dev["token_counts"], params, dev["positions"], seed,
            out["accepted_len"], out["out_tokens"], ws, **opt)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["top_lp_vals"] = res["top_lp_vals"][:, :mtl]
    res["top_lp_ids"] = res["top_lp_ids"][:, :mtl]
    res["err"] = int(ws[:4].view(torch.int32).item())
    return res


def sample_oracle(w, seed=0, max_top_lp=None, onehot=False):
    from oracle.sampling import verify_sample_accept
    mtl = max_top_lp if max_top_lp is not None else max([p.top_logprobs for p in w.params] + [0])
    return verify_sample_accept(w.target_logits, None if onehot else w.draft_logits,
                                w.draft_tokens, w.cu_rows, w.token_counts,
                                oracle_params(w.params), w.positions, seed, mtl,
                                one_hot_drafts=onehot)


LP_TOL = 2e-5


def _seq_result_matches(w, gpu, b, res, prm):
    """The GPU's accepted length, emitted tokens (-1 after them) and chosen logprobs of
    sequence b equal the oracle result `res` (an admissible outcome; a race outcome ANY
    admits any token id)."""
    from oracle.sampling import ANY, raw_logprobs
    r0, r1 = int(w.cu_rows[b]), int(w.cu_rows[b + 1])
    if int(gpu["accepted_len"][b]) != res.accepted:
        return False
    toks = gpu["out_tokens"][r0:r1]
    n = len(res.tokens)
    for i, t in enumerate(res.tokens):
        if t == ANY:
            if not 0 <= int(toks[i]) < w.vocab:
                return False
        elif int(toks[i]) != t:
            return False
    if np.any(toks[n:] != -1):
        return False
    if prm.logprobs:
        g = gpu["chosen_logprob"][r0:r1]
        if not np.all(np.isnan(g[n:])):
            return False
        for i in range(n):
            ref = raw_logprobs(w.target_logits[r0 + i])[int(toks[i])]
            if not abs(float(g[i]) - ref) <= LP_TOL:
                return False
    return True


def compare_sample(w, gpu, ora):
    """Every sequence is compared. Exact (no exception class): top-k thresholds, top-k kept
    counts, raw top-n ids; logprob values within 2e-5; nucleus kept counts equal the fp64
    one or an admissible neighbour. A sequence without exception points must equal the
    oracle's fp64 decisions exactly (accepted length, emitted tokens, chosen logprobs); a
    flagged one must equal one of the oracle's admissible outcomes (every combination of
    outcomes at its exception points).
    Returns the number of flagged sequences."""
    flagged = 0
    for b in range(w.batch):
        r0, r1 = int(w.cu_rows[b]), int(w.cu_rows[b + 1])
        prm = w.params[b]
        if ora["excepted"][b]:
            flagged += 1
            alts = ora["alternatives"][b]
            assert any(_seq_result_matches(w, gpu, b, alt, prm) for alt in alts), (
                "flagged sequence matches no admissible outcome", b, ora["points"][b],
                gpu["accepted_len"][b], gpu["out_tokens"][r0:r1],
                [(a.accepted, a.tokens) for a in alts[:8]])
        else:
            assert gpu["accepted_len"][b] == ora["accepted_len"][b], (b, gpu["accepted_len"][b],
                                                                    ora["accepted_len"][b])
            assert np.array_equal(gpu["out_tokens"][r0:r1], ora["out_tokens"][r0:r1]), (
                b, gpu["out_tokens"][r0:r1], ora["out_tokens"][r0:r1])
            if prm.logprobs:
                g, o = gpu["chosen_logprob"][r0:r1], ora["chosen_logprob"][r0:r1]
                assert np.array_equal(np.isnan(g), np.isnan(o))
                ok = ~np.isnan(o)
                assert np.all(np.abs(g[ok] - o[ok]) <= LP_TOL), (b, g, o)
        if prm.temperature > 0:
            th_g, th_o = gpu["diag_threshold"][r0:r1], ora["topk_threshold"][r0:r1]
            assert np.array_equal(th_g.astype(np.float64), th_o), (b, th_g, th_o)
            assert np.array_equal(gpu["diag_kept"][r0:r1, 0], ora["kept_topk"][r0:r1])
            # nucleus kept counts: the fp64 one, or a neighbouring crossing's within the
            # GPU's error of top_p
            for i in range(r0, r1):
                assert int(gpu["diag_kept"][i, 1]) in ora["kept_options"][i], (
                    b, i, gpu["diag_kept"][i, 1], ora["kept_options"][i])
        else:
            assert np.all(np.isnan(gpu["diag_threshold"][r0:r1]))
            assert np.all(gpu["diag_kept"][r0:r1] == 0)
        n = min(prm.top_logprobs, gpu["top_lp_ids"].shape[1])
        if gpu["top_lp_ids"].shape[1]:
            assert np.array_equal(gpu["top_lp_ids"][r0:r1, :n], ora["top_lp_ids"][r0:r1, :n])
            assert np.all(np.abs(gpu["top_lp_vals"][r0:r1, :n] - ora["top_lp_vals"][r0:r1, :n])
                          <= LP_TOL)
            assert np.all(gpu["top_lp_ids"][r0:r1, n:] == -1)
    return flagged
