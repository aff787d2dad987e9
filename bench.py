"""Benchmark of the verify step on one MI355X: verified draft-block rows per second and
achieved HBM bandwidth on the B=4, K=4, ctx 8192 workload (32 q / 8 kv heads, D=128, bf16
K/V; vocabulary 151936 fp32 logits, penalties 0.5 / 0.3, sequences 0 and 2 greedy, 1 and 3
sampled at T=0.8).

One step = verify_attention (one layer's attention of the 20 verify rows) followed by
verify_sample_accept on the same stream, on one of R distinct input sets in HBM (R * 154 MB
> 1 GB, so the 256 MB last-level cache cannot hold the working set between steps).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--static-splits] [--kv-bits 16|8|4]

Attention runs with dynamic key splits (VSA_ATTN_DYNAMIC_SPLITS: splits claim key tiles
at run time) unless --static-splits asks for fixed, bitwise reproducible ranges.
--kv-bits 8 or 4 runs the same step over a quantized copy of the cache (affine codes per
group of 64 dimensions with fp16 scale and bias) through verify_attention_kvq; the default
16 is the bf16 cache.

--draft-vocab N gives the step's drafts a reduced vocabulary of N ids (a seeded subset of the
target vocabulary and its offset table, as EAGLE-3-style heads ship): draft logits are
[rows, N] and verify_sample_accept_reduced_draft reads them through the inverse table.

    python bench.py --verify-matmul [--rows M] [--weight-bits 4|8]

times small_m_qmm instead: the four weight matmuls of one 27B-class decoder layer (hidden
5120, 64 q / 8 kv heads of 128, MLP 25600: qkv 10240x5120, o 5120x8192, gate+up 51200x5120,
down 5120x25600) on M verify rows, with synthetic quantized weights (random codes, scale
and bias) resident in HBM; one JSON line, value = layers per second.

    python bench.py --sampling WORKLOAD [--top-p P --temperature T]

times verify_sample_accept alone on a workload's logits (qwen3_4b, long, swarm, ...), with
its own parameters or, given --top-p, a nucleus without top-k on every sequence.

    python bench.py --drafter-block [--window W] [--bidirectional] [--sliding]

times block_attention alone on a drafter's block instead: B=4 blocks of 8 rows over a
32768-token context (32 q / 8 kv heads, D=128, bf16), attending the last W = 4096 context
rows by default; one JSON line in the same form, rows = block rows.

Prints one JSON line. Roofline: the dominant stage (attention: one kernel, which also
merges its key splits) is timed per call with HIP events on the stream it runs on; its
algorithmic bytes are the K/V of every sequence (ctx + R keys x Hkv x D x 2 bytes x 2), Q
and the fp32 output. HBM traffic counters come from rocprofv3 runs recorded under profiles/
and are reported only while the attention source still matches the one they were taken on.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "verify_b4k4_ctx8192"
ATTN_FLAGS = 0                   # set in main(): dynamic splits unless --static-splits
PEAK_HBM_GBPS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "attention_b4k4_ctx8192_counters.json")
ATTN_SRC = os.path.join(ROOT, "verify_step_attention_amd", "csrc", "attention.hip")


def algorithmic_bytes(w, kv_bits=16, draft_vocab=0):
    """Bytes each kernel must move at least once (inputs read once, outputs written once).
    A quantized key row is D * bits / 8 code bytes and 4 bytes of (scale, bias) per group
    of 64 dimensions."""
    rows = np.diff(w.cu_rows)
    per_key = (w.head_dim * 2 if kv_bits == 16 else
               w.head_dim * kv_bits // 8 + 4 * (w.head_dim // 64))
    kv = int(((w.ctx_lens + rows) * w.num_kv_heads * per_key * 2).sum())
    q = w.total_rows * w.num_q_heads * w.head_dim * 2
    o = w.total_rows * w.num_q_heads * w.head_dim * 4
    sampled = [b for b in range(w.batch) if w.params[b].temperature > 0]
    tl = w.total_rows * w.vocab * 4
    dl = sum(int(rows[b] - 1) for b in sampled) * (draft_vocab or w.vocab) * 4
    if draft_vocab and sampled:
        dl += w.vocab * 4                                   # the inverse table, once
    cnt = w.batch * w.vocab * 4 if w.token_counts is not None else 0
    small = w.total_rows * 4 * 2 + w.batch * 4 * 4          # drafts, tokens, lengths, params
    return {"attention": kv + q + o, "sample": tl + dl + cnt + small,
            "kv": kv, "q_out": q + o, "target_logits": tl, "draft_logits": dl, "counts": cnt}


def attention_build_digest():
    """SHA-256 of the attention source and the flags it is compiled with: the recorded
    counters hold for the kernel binary these two determine."""
    from verify_step_attention_amd import build as vbuild
    h = hashlib.sha256()
    with open(ATTN_SRC, "rb") as f:
        h.update(f.read())
    flags = vbuild.FLAGS + vbuild.SOURCE_FLAGS.get(os.path.basename(ATTN_SRC), [])
    h.update(json.dumps([f for f in flags if not f.startswith(ROOT)]).encode())
    return h.hexdigest()


def counters_traffic():
    """(fetch+write bytes per attention launch) from the recorded rocprofv3 runs, if they were
    taken on the current attention source; else None."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
        if rec.get("attention_build_sha256") != attention_build_digest():
            return None
        return rec["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def host_cpu():
    """(logical CPUs this process may run on, os.cpu_count(), CPU model string)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return avail, os.cpu_count() or 1, model


def cpu_baseline(w, name, kq=None, budget_s=8.0):
    """The oracle as it stands, timed on the host on whole verify steps of the same workload
    until about budget_s seconds have passed (at least one step), twice: with numpy's BLAS
    limited to one thread, and with it at its default (every core it sees). kq: the
    quantized cache, when the step reads one."""
    from oracle import attention as oatt, sampling as osamp
    from threadpoolctl import threadpool_info, threadpool_limits
    q = w.q_f32()
    if kq is None:
        k, v = w.kv_f32()

        def attend():
            oatt.verify_attention(q, k, v, w.cu_rows, w.ctx_lens, w.num_q_heads,
                                  w.num_kv_heads)
    else:
        def attend():
            oatt.verify_attention_kvq(q, kq.k_codes, kq.k_sb, kq.v_codes, kq.v_sb, kq.bits,
                                      w.cu_rows, w.ctx_lens, w.num_q_heads, w.num_kv_heads)
    prm = [osamp.RowParams(p.temperature, p.top_k, p.top_p, p.presence_penalty,
                           p.frequency_penalty, p.logprobs, p.top_logprobs) for p in w.params]

    def timed():
        steps, t0 = 0, time.perf_counter()
        while True:
            attend()
            osamp.verify_sample_accept(w.target_logits, w.draft_logits, w.draft_tokens,
                                       w.cu_rows, w.token_counts, prm, w.positions, w.seed)
            steps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return steps, time.perf_counter() - t0

    with threadpool_limits(limits=1):
        s1, t1 = timed()
    sn, tn = timed()
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    avail, total, model = host_cpu()
    return {"value": round(sn * w.total_rows / tn, 3), "unit": "rows/s", "cores": threads,
            "kind": "oracle",
            "single_thread_value": round(s1 * w.total_rows / t1, 3),
            "nproc": avail, "cpu_count": total, "cpu_model": model,
            "sample": f"whole verify steps of {name} (attention of all {w.total_rows} rows"
                      f"{'' if kq is None else f' over the {kq.bits}-bit cache'} + "
                      f"sample/accept of all {w.batch} sequences): {sn} step(s) in "
                      f"{tn:.1f} s with numpy's BLAS at {threads} threads (value), {s1} "
                      f"step(s) in {t1:.1f} s at 1 thread (single_thread_value); the oracle "
                      f"is numpy, so only its BLAS calls use more than one core"}


def sampling_main(args):
    """verify_sample_accept alone on a named workload's logits (its own parameters, or a
    nucleus without top-k when --top-p is given): HIP-event timing of graph replays of the
    call over 3 input sets. Drafts are the stand-in greedy drafter's (argmax of each draft
    row)."""
    import torch
    import verify_step_attention_amd as vsa
    from verify_step_attention_amd import workloads as wl
    name = args.sampling
    w = wl.make_workload(name, with_kv=False)
    if args.top_p < 1.0:
        w = w.with_params([wl.Params(temperature=args.temperature, top_p=args.top_p)] *
                          w.batch)
    mtk = max([p.top_k for p in w.params] + [1 if args.top_p < 1.0 else 0])
    mtl = max(p.top_logprobs for p in w.params)
    dev0 = wl.device_tensors(w, with_kv=False)
    sets = [dev0] + [{k: (None if t is None else t.clone()) for k, t in dev0.items()}
                     for _ in range(2)]
    params = torch.from_numpy(vsa.pack_row_params(w.params).view(np.uint8)).cuda()
    ws = torch.zeros(vsa.verify_sample_accept_workspace_size(
        w.batch, w.total_rows, w.vocab, w.max_rows, mtk, mtl), dtype=torch.uint8, device="cuda")
    acc = torch.empty(w.batch, dtype=torch.int32, device="cuda")
    toks = torch.empty(w.total_rows, dtype=torch.int32, device="cuda")
    lp = torch.empty(w.total_rows, dtype=torch.float32, device="cuda")
    tv = torch.empty((w.total_rows, max(mtl, 1)), dtype=torch.float32, device="cuda")
    ti = torch.empty((w.total_rows, max(mtl, 1)), dtype=torch.int32, device="cuda")

    def call(d, s):
        vsa.verify_sample_accept(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                                 d["cu_rows"], d["token_counts"], params, d["positions"], 0,
                                 acc, toks, ws, max_rows_per_seq=w.max_rows, max_top_k=mtk,
                                 max_top_logprobs=mtl, chosen_logprob=lp,
                                 top_lp_vals=tv if mtl else None,
                                 top_lp_ids=ti if mtl else None, stream=s)
    stream = torch.cuda.current_stream()
    for d in sets:
        call(d, stream)
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for d in sets:
                call(d, torch.cuda.current_stream())
    stream.wait_stream(cs)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // len(sets))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(sets))
    err = int(ws[:4].view(torch.int32).item())
    if err:
        print(f"[bench] device error word {err:#x}", file=sys.stderr)
    nbytes = (w.total_rows + (w.total_rows - w.batch)) * w.vocab * 4 + \
        (0 if w.token_counts is None else w.batch * w.vocab * 4)
    print(json.dumps({
        "metric": f"verify_sample_accept calls/sec, {name}" +
                  (f", nucleus T={args.temperature} top_p={args.top_p}"
                   if args.top_p < 1.0 else ""),
        "value": round(1e6 / us, 1), "unit": "calls/s", "n_gpus": 1,
        "steps": reps * len(sets), "warmup": len(sets), "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "launch": "hip_graph_replay",
        "config": {"workload": name, "batch": w.batch, "rows": w.total_rows,
                   "vocab": w.vocab, "call_us": round(us, 2),
                   "logit_bytes": nbytes}}), flush=True)


def drafter_block_main(args):
    """block_attention on drafter_b4r8_ctx32768: HIP-event timing over graph replays of the
    call on R input sets, roofline against the keys the rows attend, the oracle as the CPU
    baseline."""
    import torch
    import verify_step_attention_amd as vsa
    from verify_step_attention_amd import workloads as wl
    name = "drafter_b4r8_ctx32768"
    flags = (0 if args.static_splits else vsa.ATTN_DYNAMIC_SPLITS) | \
        (vsa.ATTN_BIDIRECTIONAL if args.bidirectional else 0) | \
        (vsa.ATTN_SLIDING_WINDOW if args.sliding else 0)
    print(f"[bench] building inputs for {name}", file=sys.stderr, flush=True)
    w = wl.make_workload(name)
    rows = np.diff(w.cu_rows)
    win = args.window
    # keys some row of the block attends (context window + block), each read once
    first = np.maximum(0, w.ctx_lens - (win - (1 if args.sliding else 0))) if win else \
        np.zeros_like(w.ctx_lens)
    kv = int(((w.ctx_lens + rows - first) * w.num_kv_heads * w.head_dim * 2 * 2).sum())
    nbytes = kv + w.total_rows * w.num_q_heads * w.head_dim * (2 + 4)
    dev0 = wl.device_tensors(w, with_kv=True)
    sets = [dev0] + [{k: (None if t is None else t.clone()) for k, t in dev0.items()}
                     for _ in range(args.sets - 1)]
    ws = torch.zeros(vsa.verify_attention_workspace_size(
        w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_rows, w.max_kv_len),
        dtype=torch.uint8, device="cuda")
    out = torch.empty((w.total_rows, w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")

    def call(d, s):
        vsa.block_attention(d["q"], d["k_cache"], d["v_cache"], d["cu_rows"], d["ctx_lens"],
                            out, ws, max_rows_per_seq=w.max_rows, max_kv_len=w.max_kv_len,
                            window=win, flags=flags, stream=s)
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        call(sets[i % len(sets)], stream)
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for d in sets:
                call(d, torch.cuda.current_stream())
    stream.wait_stream(cs)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // len(sets))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(sets))
    err = int(ws[:4].view(torch.int32).item())
    if err:
        print(f"[bench] device error word {err:#x}", file=sys.stderr)
    achieved = nbytes / (us * 1e-6) / 1e9
    mode = ("bidirectional" if args.bidirectional else "causal") + \
        (", sliding" if args.sliding else "")
    line = {
        "metric": f"drafter block attention rows/sec + achieved HBM GB/s, B=4 block 8 "
                  f"ctx 32768 window {win}",
        "value": round(w.total_rows / (us * 1e-6), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": reps * len(sets), "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "launch": "hip_graph_replay",
        "config": {"workload": name, "batch": w.batch, "block_rows": 8, "ctx": 32768,
                   "window": win, "mask": mode, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "input_sets": len(sets), "attention_us": round(us, 2),
                   "attention_splits": "static" if args.static_splits else "dynamic"},
        "roofline": {"bound": "hbm", "kernel": "block_attention call (attn_bf16_kernel<128,"
                     "1,true>)", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        from oracle import attention as oatt
        k, v = w.kv_f32()
        q = w.q_f32()
        n, t0 = 0, time.perf_counter()
        while True:
            oatt.block_attention(q, k, v, w.cu_rows, w.ctx_lens, w.num_q_heads,
                                 w.num_kv_heads, window=win, sliding=args.sliding,
                                 bidirectional=args.bidirectional)
            n += 1
            if time.perf_counter() - t0 >= 10.0:
                break
        dt = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            cores = 1
        line["cpu_baseline"] = {"value": round(n * w.total_rows / dt, 3), "unit": "rows/s",
                                "cores": cores, "kind": "oracle",
                                "sample": f"{n} whole block_attention call(s) of {name} on "
                                          f"the host, {dt:.1f} s"}
    print(json.dumps(line), flush=True)


LAYER_27B = (("qkv", 10240, 5120), ("o", 5120, 8192), ("gate_up", 51200, 5120),
             ("down", 5120, 25600))


def verify_matmul_main(args):
    """small_m_qmm over one 27B-class layer's projections; HIP-event timing of graph replays
    rotating over weight sets (more than the 256 MB last-level cache); the oracle timed on a
    sample of output features as the CPU baseline."""
    import torch
    import verify_step_attention_amd as vsa
    bits, m = args.weight_bits, args.rows
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    layer_bytes = sum(n * k * bits // 8 + n * (k // 64) * 4 for _, n, k in LAYER_27B)
    nsets = max(2, -(-(1 << 30) // layer_bytes))           # > 1 GB of distinct weights
    print(f"[bench] {nsets} weight sets of {layer_bytes / 1e6:.1f} MB", file=sys.stderr,
          flush=True)
    sets = []
    for _ in range(nsets):
        mats = []
        for name, n, k in LAYER_27B:
            codes = torch.randint(0, 256, (n, k * bits // 8), dtype=torch.uint8, device="cuda",
                                  generator=gen)
            sb = torch.empty((n, k // 64, 2), dtype=torch.float16, device="cuda")
            sb[..., 0].uniform_(1e-4, 2e-3, generator=gen)
            sb[..., 1].uniform_(-0.2, 0.0, generator=gen)
            mats.append((codes, sb))
        sets.append(mats)
    xs = {k: torch.randn((m, k), dtype=torch.float32, device="cuda", generator=gen).to(
        torch.bfloat16) for k in {k for _, _, k in LAYER_27B}}
    ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for _, n, _ in LAYER_27B]
    wss = [torch.zeros(vsa.small_m_qmm_workspace_size(m, n, k), dtype=torch.uint8,
                       device="cuda") for _, n, k in LAYER_27B]

    def layer(mats, s):
        for i, (name, n, k) in enumerate(LAYER_27B):
            vsa.small_m_qmm(xs[k], mats[i][0], mats[i][1], bits, ys[i], wss[i], stream=s)
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        layer(sets[i % nsets], stream)
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for mats in sets:
                layer(mats, torch.cuda.current_stream())
    stream.wait_stream(cs)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // nsets)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * nsets)
    nbytes = layer_bytes + sum(m * k * 2 + m * n * 4 for _, n, k in LAYER_27B)
    achieved = nbytes / (us * 1e-6) / 1e9
    line = {
        "metric": f"verify matmul layers/sec + achieved HBM GB/s, 27B-class layer, {m} rows, "
                  f"{bits}-bit weights",
        "value": round(1e6 / us, 1), "unit": "layers/s", "n_gpus": 1,
        "steps": reps * nsets, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"bf16 x, u{bits} weight codes", "data": "synthetic",
        "launch": "hip_graph_replay",
        "config": {"workload": "layer27b_small_m_qmm", "rows": m, "weight_bits": bits,
                   "matmuls": [f"{name} {n}x{k}" for name, n, k in LAYER_27B],
                   "weight_sets": nsets, "layer_us": round(us, 2),
                   "algorithmic_bytes_per_layer": nbytes},
        "roofline": {"bound": "hbm", "kernel": f"small_m_qmm x4 (qmm_kernel<{bits}> + "
                     "qmm_reduce_kernel)", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        from oracle.qmm import small_m_qmm
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            cores = 1
        # a bounded sample: 256 output features of each projection, whole input width
        feats, t0, done = 256, time.perf_counter(), 0
        mats = sets[0]
        while True:
            for i, (name, n, k) in enumerate(LAYER_27B):
                small_m_qmm(xs[k].float().cpu().numpy(), mats[i][0][:feats].cpu().numpy(),
                            mats[i][1][:feats].cpu().numpy(), bits)
            done += 1
            if time.perf_counter() - t0 >= 10.0:
                break
        dt = time.perf_counter() - t0
        frac = feats * len(LAYER_27B) / sum(n for _, n, _ in LAYER_27B)
        per_layer = dt / done / (sum(feats * k for _, n, k in LAYER_27B) /
                                 sum(n * k for _, n, k in LAYER_27B))
        line["cpu_baseline"] = {"value": round(1.0 / per_layer, 4), "unit": "layers/s",
                                "cores": cores, "kind": "oracle",
                                "sample": f"{done} pass(es) over 256 output features of each "
                                          f"projection ({frac:.4f} of the layer's features, "
                                          f"weighted by input width), {dt:.1f} s on the host, "
                                          "scaled to whole layers"}
    print(json.dumps(line), flush=True)


def _counter_rows(d, counter):
    """Per-kernel values of one rocprofv3 --pmc counter (KiB per dispatch) under folder d."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def record_traffic(fetch_dir, write_dir, copy_mib, command):
    """Turn two rocprofv3 --pmc runs of `bench.py --eager --copy-probe-mib M` (FETCH_SIZE, then
    WRITE_SIZE) into bytes per verify_attention call (its one kernel). Each counter is scaled by what it reads for the plain copy of M MiB that the
    run starts with (read M MiB, write M MiB)."""
    fetch = _counter_rows(fetch_dir, "FETCH_SIZE")
    write = _counter_rows(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib << 20
    copy_k = max((k for k in fetch if "copy" in k.lower()), key=lambda k: max(fetch[k]))
    f_scale = max(fetch[copy_k]) * 1024 / copy_bytes
    w_scale = max(write[copy_k]) * 1024 / copy_bytes
    kernels = {}
    for k in fetch:
        if "vsa::" not in k:
            continue
        fb = float(np.median(fetch[k])) * 1024 / f_scale
        wb = float(np.median(write.get(k, [0.0]))) * 1024 / w_scale
        kernels[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                      "dispatches": len(fetch[k])}
    attn = [k for k in kernels if "attn_bf16_kernel" in k]
    if not any("attn_bf16_kernel" in k for k in attn):
        raise SystemExit(f"no attention kernel in the counters: {list(kernels)}")
    a = {"fetch_bytes": sum(kernels[k]["fetch_bytes"] for k in attn),
         "write_bytes": sum(kernels[k]["write_bytes"] for k in attn)}
    rec = {"command": command, "copy_probe_mib": copy_mib,
           "copy_fetch_scale": round(f_scale, 4), "copy_write_scale": round(w_scale, 4),
           "attention_build_sha256": attention_build_digest(),
           "bytes_per_launch": a["fetch_bytes"] + a["write_bytes"], "kernels": kernels}
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def summarize_stats(path, command):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv."""
    import csv
    print(f"command: `{command}`\n")
    print("| kernel | calls | avg us | min us | max us | share % |")
    print("|---|---|---|---|---|---|")
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
            print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{float(r['Percentage']):.1f} |")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--record-traffic":
        # bench.py --record-traffic FETCH_DIR WRITE_DIR COPY_MIB "<command>"
        record_traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-stats":
        # bench.py --summarize-stats KERNEL_STATS_CSV "<command>"
        summarize_stats(sys.argv[2], sys.argv[3])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=7)
    ap.add_argument("--workload", default=WORKLOAD,
                    help="the workload of the timed steps (default: the metric's, "
                         f"{WORKLOAD}); the others are the configurations of the parity "
                         "tests, measured one by one for the per-configuration table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--static-splits", action="store_true",
                    help="attention with fixed key ranges per split (bitwise reproducible) "
                         "instead of tiles claimed at run time")
    ap.add_argument("--kv-bits", type=int, default=16, choices=(16, 8, 4),
                    help="K/V cache: bf16 (16) or affine codes of 8 or 4 bits")
    ap.add_argument("--draft-vocab", type=int, default=0,
                    help="reduced draft vocabulary size (0: drafts over the whole vocabulary)")
    ap.add_argument("--verify-matmul", action="store_true",
                    help="time small_m_qmm on a 27B-class layer instead of the step")
    ap.add_argument("--rows", type=int, default=8)
    ap.add_argument("--weight-bits", type=int, default=4, choices=(4, 8))
    ap.add_argument("--sampling", default="",
                    help="time verify_sample_accept alone on this workload's logits")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="with --sampling: every sequence a nucleus without top-k")
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--drafter-block", action="store_true",
                    help="time block_attention on a drafter's block instead of the step")
    ap.add_argument("--window", type=int, default=4096)
    ap.add_argument("--bidirectional", action="store_true")
    ap.add_argument("--sliding", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call from Python instead of replaying HIP graphs")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "reference for rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the verify step's sharding across GPUs is a design note, not a run.",
              file=sys.stderr)
        sys.exit(2)
    if args.sampling:
        sampling_main(args)
        return
    if args.drafter_block:
        drafter_block_main(args)
        return
    if args.verify_matmul:
        verify_matmul_main(args)
        return

    import torch
    import verify_step_attention_amd as vsa
    from verify_step_attention_amd import workloads as wl
    global ATTN_FLAGS
    ATTN_FLAGS = 0 if args.static_splits else vsa.ATTN_DYNAMIC_SPLITS

    name = args.workload
    print(f"[bench] building inputs for {name}", file=sys.stderr, flush=True)
    w = wl.make_workload(name)
    nbytes = algorithmic_bytes(w, args.kv_bits, args.draft_vocab)
    step_bytes = nbytes["attention"] + nbytes["sample"]
    dev0 = wl.device_tensors(w)
    kq = None
    if args.kv_bits != 16:
        kq = wl.quantized_cache(w, args.kv_bits)
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
        dev0.update(k_codes=dev(kq.k_codes), k_sb=dev(kq.k_sb), v_codes=dev(kq.v_codes),
                    v_sb=dev(kq.v_sb))
        del dev0["k_cache"], dev0["v_cache"]
    t2d = None
    if args.draft_vocab:
        rng = np.random.default_rng(77)
        subset = np.sort(rng.choice(w.vocab, size=args.draft_vocab, replace=False))
        d2t = torch.from_numpy((subset - np.arange(args.draft_vocab)).astype(np.int32)).cuda()
        t2d = torch.empty(w.vocab, dtype=torch.int32, device="cuda")
        vsa.draft_vocab_inverse(d2t, w.vocab, t2d)
        idx = torch.from_numpy(subset).cuda()
        # draft rows over the subset; the step's drafts are ids of the subset
        dev0["draft_logits"] = dev0["draft_logits"][:, idx].contiguous()
        dev0["draft_tokens"] = idx[torch.argmax(dev0["draft_logits"], dim=1)].to(torch.int32)
    sets = [dev0] + [{k: (None if t is None else t.clone()) for k, t in dev0.items()}
                     for _ in range(args.sets - 1)]
    params = torch.from_numpy(vsa.pack_row_params(w.params).view(np.uint8)).cuda()
    mtk = max(p.top_k for p in w.params)
    mtl = max(p.top_logprobs for p in w.params)
    ws_a = torch.zeros(vsa.verify_attention_workspace_size(
        w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_rows, w.max_kv_len),
        dtype=torch.uint8, device="cuda")
    ws_s = torch.zeros(vsa.verify_sample_accept_workspace_size(
        w.batch, w.total_rows, w.vocab, w.max_rows, mtk, mtl), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.total_rows, w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")
    acc = torch.empty(w.batch, dtype=torch.int32, device="cuda")
    toks = torch.empty(w.total_rows, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def attention(d, s=None):
        if kq is None:
            vsa.verify_attention(d["q"], d["k_cache"], d["v_cache"], d["cu_rows"],
                                 d["ctx_lens"], out, ws_a, max_rows_per_seq=w.max_rows,
                                 max_kv_len=w.max_kv_len, flags=ATTN_FLAGS,
                                 stream=stream if s is None else s)
        else:
            vsa.verify_attention_kvq(d["q"], d["k_codes"], d["k_sb"], d["v_codes"], d["v_sb"],
                                     kq.bits, d["cu_rows"], d["ctx_lens"], out, ws_a,
                                     max_rows_per_seq=w.max_rows, max_kv_len=w.max_kv_len,
                                     flags=ATTN_FLAGS, stream=stream if s is None else s)

    def sample(d, s=None):
        if t2d is None:
            vsa.verify_sample_accept(d["target_logits"], d["draft_logits"], d["draft_tokens"],
                                     d["cu_rows"], d["token_counts"], params, d["positions"],
                                     0, acc, toks, ws_s, max_rows_per_seq=w.max_rows,
                                     max_top_k=mtk, max_top_logprobs=mtl,
                                     stream=stream if s is None else s)
        else:
            vsa.verify_sample_accept_reduced_draft(
                d["target_logits"], d["draft_logits"], t2d, d["draft_tokens"], d["cu_rows"],
                d["token_counts"], params, d["positions"], 0, acc, toks, ws_s,
                max_rows_per_seq=w.max_rows, max_top_k=mtk, max_top_logprobs=mtl,
                stream=stream if s is None else s)

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        d = sets[i % len(sets)]
        attention(d)
        sample(d)
    torch.cuda.synchronize()

    # HIP graphs hold whole steps (the library only launches kernels on the given stream; no
    # memsets, no allocations): one graph per input set, and one "ring" graph that runs a
    # step on every set in turn, so step-to-step transitions happen inside a graph.
    graphs, ring = [], None
    if not args.eager:
        def capture(step_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=capture_stream):
                cs = torch.cuda.current_stream()
                for d in step_sets:
                    attention(d, cs)
                    sample(d, cs)
            return g
        capture_stream = torch.cuda.Stream()
        capture_stream.wait_stream(stream)
        with torch.cuda.stream(capture_stream):
            graphs = [capture([d]) for d in sets]
            ring = capture(sets)
        stream.wait_stream(capture_stream)
        ring.replay()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

    def run_steps(k):
        """Exactly k steps, rotating through the input sets."""
        i = 0
        if graphs:
            while k - i >= len(sets):
                ring.replay()
                i += len(sets)
            while i < k:
                graphs[i % len(graphs)].replay()
                i += 1
        else:
            for i in range(k):
                d = sets[i % len(sets)]
                attention(d)
                sample(d)

    # whole-step timing
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    run_steps(args.steps)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    print(f"[bench] {args.steps} steps timed ({'eager' if not graphs else 'graph replay'}): "
          f"{ms_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)

    # per-kernel timing on the launch stream. Graph mode: one graph per stage that runs that
    # stage on every input set in turn, replayed back to back between two HIP events (the
    # same launch sequence as the steps, minus the other stage). Eager mode: events around
    # each call.
    if graphs:
        def stage_graph(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(capture_stream):
                with torch.cuda.graph(g, stream=capture_stream):
                    for d in sets:
                        fn(d, torch.cuda.current_stream())
            stream.wait_stream(capture_stream)
            return g
        g_att = stage_graph(lambda d, s: attention(d, s))
        g_smp = stage_graph(lambda d, s: sample(d, s))
        reps = max(1, args.steps // len(sets))

        def time_graph(g):
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            per = []
            for _ in range(reps):
                e0.record(stream)
                g.replay()
                e1.record(stream)
                e1.synchronize()
                per.append(e0.elapsed_time(e1) / len(sets))
            return np.array(per)
        attn_ms, samp_ms = time_graph(g_att), time_graph(g_smp)
    else:
        n_k = min(args.steps, 100)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_k)]
        for i in range(n_k):
            d = sets[i % len(sets)]
            ev[i][0].record(stream)
            attention(d)
            ev[i][1].record(stream)
            sample(d)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        attn_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
        samp_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    torch.cuda.synchronize()
    err_a = int(ws_a[:4].view(torch.int32).item())
    err_s = int(ws_s[:4].view(torch.int32).item())
    if err_a or err_s:
        print(f"[bench] device error words: attention {err_a:#x} sample {err_s:#x}",
              file=sys.stderr)

    attn_us = float(np.mean(attn_ms)) * 1e3
    achieved = nbytes["attention"] / (attn_us * 1e-6) / 1e9
    traffic = counters_traffic() if kq is None and name == WORKLOAD else None
    rows_per_s = w.total_rows / (ms_step * 1e-3)
    rows = np.diff(w.cu_rows)
    line = {
        "metric": ("verified draft-block rows/sec + achieved HBM GB/s, B=4 K=4 ctx 8192"
                   if name == WORKLOAD else
                   f"verified draft-block rows/sec + achieved HBM GB/s, {name}"),
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if w.dtype == wl.BF16 else "f32") if kq is None else
                 f"bf16 q, u{kq.bits} kv codes",
        "data": "synthetic",
        "achieved_hbm_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "launch": "eager" if not graphs else "hip_graph_replay",
        "config": {
            "workload": name, "batch": w.batch,
            "drafts_per_seq": sorted({int(r) - 1 for r in rows}),
            "ctx": [int(w.ctx_lens.min()), int(w.ctx_lens.max())],
            "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "vocab": w.vocab, "rows_per_step": w.total_rows, "input_sets": len(sets),
            "algorithmic_bytes_per_step": step_bytes,
            "step_fraction_of_8TBps": round(step_bytes / (ms_step * 1e-3) / 1e9 /
                                            PEAK_HBM_GBPS, 4),
            "attention_us": round(attn_us, 2),
            "attention_us_p10_p90": [round(float(np.percentile(attn_ms, 10)) * 1e3, 2),
                                     round(float(np.percentile(attn_ms, 90)) * 1e3, 2)],
            "sample_accept_us": round(float(np.mean(samp_ms)) * 1e3, 2),
            "logits_dtype": "f32",
            "attention_splits": "dynamic" if ATTN_FLAGS else "static",
            "kv_bits": args.kv_bits,
            "draft_vocab": args.draft_vocab or w.vocab,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": (f"verify_attention call (attn_{'bf16' if w.dtype == wl.BF16 else 'f32'}"
                       f"_kernel, D={w.head_dim})"
                       if kq is None else
                       f"verify_attention_kvq call (attn_kvq_kernel<128,1,{kq.bits}>)"),
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": nbytes["attention"],
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on the host", file=sys.stderr, flush=True)
        wc = w
        if t2d is not None:
            from oracle.sampling import widen_draft_logits
            wc = w.with_params(w.params)
            wc.draft_logits = widen_draft_logits(dev0["draft_logits"].cpu().numpy(),
                                                 d2t.cpu().numpy(), w.vocab)
            wc.draft_tokens = dev0["draft_tokens"].cpu().numpy()
        line["cpu_baseline"] = cpu_baseline(wc, name, kq)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
