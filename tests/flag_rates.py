"""Exception-flag rate of the oracle's decisions on the named workloads (CPU only).

TEST INFRASTRUCTURE: runs the CPU oracle, never the library.

A sampled sequence is flagged when one of its decisions lies within the GPU's error bound
of a boundary: an acceptance test u * q(d) < p(d) within the accept margin, a nucleus
crossing within the margin of top_p, or a race whose two best keys lie within the key
margin. There the GPU may take either side, and the parity tests accept any admissible
outcome; the design target is fewer than 0.1% flagged sequences per workload.

Each trial draws a fresh copy of the workload (its random data with another seed offset),
drafts distributed as the truncated draft distribution q (the drafter's own sampler),
and a fresh Philox seed, and counts the flagged sampled sequences. Greedy sequences are
never flagged and are not counted. The tiny workload is taken at T = 1.0 (its sampled
setting).

    python tests/flag_rates.py [--trials-scale S | --trials N] [--first I] [--procs P]
                               [workload ...]

prints one markdown table row per workload: sampled sequences, flagged, rate, and the
95% Clopper-Pearson upper bound of the rate.
"""
import argparse
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from verify_step_attention_amd import workloads as wl  # noqa: E402
from oracle import sampling as osamp  # noqa: E402

# workload: trials at scale 1 (chosen so that each has about 3000 sampled sequences)
TRIALS = {"tiny": 3000, "qwen3_4b": 3000, "batched": 1500, "verify_b4k4_ctx8192": 1500,
          "long": 1500, "swarm": 200}


def _params(w):
    if w.name == "tiny":
        return [osamp.RowParams(1.0, 0, 1.0, 0.0, 0.0, 0, 0)] * w.batch
    return [osamp.RowParams(p.temperature, p.top_k, p.top_p, p.presence_penalty,
                            p.frequency_penalty, p.logprobs, p.top_logprobs) for p in w.params]


def trial(args):
    name, t = args
    w = wl.make_workload(name, with_kv=False, seed_offset=7919 * (t + 1))
    prm = _params(w)
    drafts = osamp.sample_proposals(w.draft_logits, w.cu_rows, prm, w.positions, 1000 + t)
    res = osamp.verify_sample_accept(w.target_logits, w.draft_logits, drafts, w.cu_rows,
                                     w.token_counts, prm, w.positions, 5000 + t,
                                     max(p.top_logprobs for p in prm), alternatives=False)
    sampled = [b for b in range(w.batch) if prm[b].temperature > 0]
    return len(sampled), int(sum(bool(res["excepted"][b]) for b in sampled))


def upper95(k, n):
    from scipy.stats import beta
    return 1.0 if k >= n else float(beta.ppf(0.975, k + 1, n - k))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trials-scale", type=float, default=1.0)
    ap.add_argument("--procs", type=int, default=os.cpu_count() or 1)
    ap.add_argument("--first", type=int, default=0, help="index of the first trial")
    ap.add_argument("--trials", type=int, default=0,
                    help="trials per workload (default: the table above times the scale)")
    ap.add_argument("workloads", nargs="*", default=list(TRIALS))
    args = ap.parse_args()
    print("| workload | sampled sequences | flagged | rate | 95% upper bound |")
    print("|---|---|---|---|---|")
    with ProcessPoolExecutor(max_workers=args.procs) as pool:
        for name in args.workloads:
            n_trials = args.trials or max(1, int(TRIALS[name] * args.trials_scale))
            n = k = 0
            trials = [(name, t) for t in range(args.first, args.first + n_trials)]
            for ns, nf in pool.map(trial, trials, chunksize=4):
                n += ns
                k += nf
            print(f"| {name} | {n} | {k} | {k / max(n, 1):.2e} | {upper95(k, n):.2e} |",
                  flush=True)


if __name__ == "__main__":
    main()
