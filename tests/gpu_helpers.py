"""Helpers for the GPU parity tests: run the library on a workload through the C ABI."""
import numpy as np
import torch

import verify_step_attention_amd as vsa
from verify_step_attention_amd import workloads as wl


def attention_gpu(w, dev=None, max_kv_len=None, workspace=None, stream=None):
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
                         max_kv_len=mkv, stream=stream)
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
