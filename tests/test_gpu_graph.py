"""Both entry points captured in one HIP graph: every replay, with eager calls on other
inputs and host synchronizations in between, gives exactly the eager results (the library
launches only kernels, keeps its counters self-resetting and records no memsets)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_step_attention_amd as vsa  # noqa: E402
from verify_step_attention_amd import workloads as wl  # noqa: E402


@pytest.mark.parametrize("flags", [0, vsa.ATTN_DYNAMIC_SPLITS])
def test_graph_replays_match_eager(flags):
    print(f"graph replays, attention flags {flags}", flush=True)
    w = wl.make_workload("batched")
    other = wl.make_workload("batched", seed_offset=7)
    if other.total_rows != w.total_rows or other.s_max != w.s_max:
        other = w
    d = wl.device_tensors(w)
    d2 = wl.device_tensors(other)
    params = torch.from_numpy(vsa.pack_row_params(w.params).view(np.uint8)).cuda()
    ws_a = torch.zeros(vsa.verify_attention_workspace_size(
        w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_rows, w.s_max),
        dtype=torch.uint8, device="cuda")
    ws_s = torch.zeros(vsa.verify_sample_accept_workspace_size(
        w.batch, w.total_rows, w.vocab, w.max_rows, 0, 0), dtype=torch.uint8, device="cuda")
    out = torch.zeros((w.total_rows, w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")
    acc = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    toks = torch.zeros(w.total_rows, dtype=torch.int32, device="cuda")

    def step(dd, stream):
        vsa.verify_attention(dd["q"], dd["k_cache"], dd["v_cache"], dd["cu_rows"],
                             dd["ctx_lens"], out, ws_a, max_rows_per_seq=w.max_rows,
                             max_kv_len=w.s_max, flags=flags, stream=stream)
        vsa.verify_sample_accept(dd["target_logits"], dd["draft_logits"], dd["draft_tokens"],
                                 dd["cu_rows"], dd["token_counts"], params, dd["positions"], 3,
                                 acc, toks, ws_s, max_rows_per_seq=w.max_rows, max_top_k=0,
                                 max_top_logprobs=0, stream=stream)

    step(d, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = (out.clone(), acc.clone(), toks.clone())

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(d, torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        out.zero_()
        acc.zero_()
        toks.zero_()
        g.replay()
        torch.cuda.synchronize()
        if flags & vsa.ATTN_DYNAMIC_SPLITS:
            # tile sets of the splits depend on timing: equal up to fp32 rounding order
            assert torch.allclose(out, ref[0], rtol=1e-5, atol=1e-6), f"replay {rep}"
        else:
            assert torch.equal(out, ref[0]), f"replay {rep}: attention differs"
        assert torch.equal(acc, ref[1]) and torch.equal(toks, ref[2]), f"replay {rep}: tokens"
        step(d2, torch.cuda.current_stream())          # eager work on other inputs between
        torch.cuda.synchronize()
    assert int(ws_a[:4].view(torch.int32).item()) == 0
    assert int(ws_s[:4].view(torch.int32).item()) == 0
