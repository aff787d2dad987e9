"""verify_attention_noalloc (no workspace argument: the library's static per-GPU scratch
holds the partial results) against verify_attention through the C ABI. Two calls in a row
on one GPU, the second on a smaller problem: each output equals verify_attention's on the
same inputs (bitwise with fixed splits) and lies within the oracle's tolerance."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_step_attention_amd as vsa  # noqa: E402
from verify_step_attention_amd import workloads as wl  # noqa: E402
from gpu_helpers import attention_gpu, attention_oracle, assert_attention_close  # noqa: E402


def _log(msg):
    print(msg, flush=True)


def _noalloc(w, dev, device_error=None, flags=0):
    out = torch.full((w.total_rows, w.num_q_heads, w.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    vsa.verify_attention_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["cu_rows"],
                                 dev["ctx_lens"], out, device_error,
                                 max_rows_per_seq=w.max_rows, max_kv_len=w.max_kv_len,
                                 flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("flags", [0, vsa.ATTN_DYNAMIC_SPLITS])
def test_noalloc_matches_verify_attention_on_two_calls(flags):
    # the second problem is smaller (fewer sequences, heads, keys and rows)
    for name in ("verify_b4k4_ctx8192", "tiny"):
        _log(f"noalloc attention: workload {name} flags {flags}")
        w = wl.make_workload(name)
        dev = wl.device_tensors(w)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        got = _noalloc(w, dev, err, flags)
        want, werr = attention_gpu(w, dev=dev, flags=flags)
        assert int(err.item()) == 0 and werr == 0
        if flags == 0:
            assert np.array_equal(got, want), name
        assert_attention_close(got, attention_oracle(w))
        assert_attention_close(want, attention_oracle(w))


def test_noalloc_error_word_and_size_limit():
    _log("noalloc attention: device error word, scratch size limit")
    w = wl.make_workload("tiny")
    w.ctx_lens = np.array([w.s_max], np.int32)          # ctx + R beyond S_max: clamped
    dev = wl.device_tensors(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((w.total_rows, w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")
    vsa.verify_attention_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["cu_rows"],
                                 dev["ctx_lens"], out, err, max_rows_per_seq=w.max_rows,
                                 max_kv_len=w.s_max)
    torch.cuda.synchronize()
    assert int(err.item()) & 0x01
    # a problem whose workspace exceeds the scratch is refused before anything is enqueued
    big = vsa.verify_attention_workspace_size(64, 32, 8, 128, 32, 65536)
    assert big > vsa.NOALLOC_SCRATCH_BYTES
    lib = vsa.library()
    p = [dev[k].data_ptr() for k in ("q", "k_cache", "v_cache", "cu_rows", "ctx_lens")]
    st = lib.verify_attention_noalloc(p[0], p[1], p[2], vsa.VSA_BF16, p[3], p[4], 64, 64, 32, 8,
                                      128, 65536, 32, 65536, 0.0, 0, out.data_ptr(), None, None)
    assert st == vsa.VSA_ERR_WORKSPACE
    # the next call after the refusal still matches the workspace path
    w = wl.make_workload("qwen3_4b")
    dev = wl.device_tensors(w)
    got = _noalloc(w, dev)
    want, _ = attention_gpu(w, dev=dev)
    assert np.array_equal(got, want)
