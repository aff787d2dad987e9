"""GPU parity of verify_attention_kvq (8- and 4-bit affine K/V cache) against the CPU
oracle on the dequantized values, elementwise |gpu - oracle| <= 1e-3 + 2e-3 |oracle|,
through the C ABI."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_step_attention_amd as vsa  # noqa: E402
from verify_step_attention_amd import workloads as wl  # noqa: E402
from gpu_helpers import assert_attention_close  # noqa: E402
from test_gpu_attention import _custom  # noqa: E402


def _log(msg):
    print(msg, flush=True)


def kvq_gpu(w, kq, flags=0, max_kv_len=None, workspace=None):
    mkv = max_kv_len or w.max_kv_len
    size = vsa.verify_attention_workspace_size(w.batch, w.num_q_heads, w.num_kv_heads,
                                               w.head_dim, w.max_rows, mkv)
    ws = workspace if workspace is not None else torch.zeros(size, dtype=torch.uint8,
                                                             device="cuda")
    ws[:4].zero_()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    q = dev(w.q.view(np.int16)).view(torch.bfloat16)
    out = torch.full((w.total_rows, w.num_q_heads, w.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    vsa.verify_attention_kvq(q, dev(kq.k_codes), dev(kq.k_sb), dev(kq.v_codes),
                             dev(kq.v_sb), kq.bits, dev(w.cu_rows.astype(np.int32)),
                             dev(w.ctx_lens.astype(np.int32)), out, ws,
                             max_rows_per_seq=w.max_rows, max_kv_len=mkv, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(ws[:4].view(torch.int32).item())


def kvq_oracle(w, kq):
    from oracle.attention import verify_attention_kvq
    return verify_attention_kvq(w.q_f32(), kq.k_codes, kq.k_sb, kq.v_codes, kq.v_sb, kq.bits,
                                w.cu_rows, w.ctx_lens, w.num_q_heads, w.num_kv_heads)


@pytest.mark.parametrize("flags", [0, vsa.ATTN_DYNAMIC_SPLITS])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("name", ["verify_b4k4_ctx8192", "qwen3_4b", "batched", "long"])
def test_workload_parity(name, bits, flags):
    _log(f"kvq attention parity: {name} bits {bits} flags {flags}")
    w = wl.make_workload(name)
    kq = wl.quantized_cache(w, bits)
    got, err = kvq_gpu(w, kq, flags=flags)
    assert err == 0
    assert_attention_close(got, kvq_oracle(w, kq))


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("case", [
    # (Hq, Hkv, D, ctx list, drafts list, max_kv_len override)
    (32, 8, 128, [0, 1, 127, 128], [0, 3, 4, 31], None),    # ctx 0, K=0, K=31
    (8, 8, 64, [300, 5], [2, 6], 4096),                      # D=64, MHA, empty splits
    (64, 8, 128, [700], [15], None),                         # 128 columns (4 blocks)
    (48, 8, 128, [1000, 2000], [8, 2], None),                # 2 column blocks
    (16, 2, 64, [333, 40], [3, 9], None),                    # D=64, ragged
    (32, 8, 128, [5], [4], 8192),                            # mostly empty splits
])
def test_edge_shapes(case, bits):
    hq, hkv, d, ctxs, drafts, mkv = case
    _log(f"kvq attention edge case {case} bits {bits}")
    w = _custom(hq, hkv, d, wl.BF16, ctxs, drafts)
    if mkv is not None:
        mkv = min(mkv, w.s_max)
    kq = wl.quantized_cache(w, bits)
    got, err = kvq_gpu(w, kq, max_kv_len=mkv)
    assert err == 0
    assert_attention_close(got, kvq_oracle(w, kq))


def test_static_splits_reproducible_and_reuse_workspace():
    _log("kvq attention: bitwise repeat with fixed splits, workspace reuse with dynamic ones")
    w = wl.make_workload("batched")
    kq = wl.quantized_cache(w, 8)
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    x, _ = kvq_gpu(w, kq, workspace=ws)
    y, _ = kvq_gpu(w, kq, workspace=ws)
    assert np.array_equal(x, y)
    ref = kvq_oracle(w, kq)
    for _ in range(3):
        z, err = kvq_gpu(w, kq, flags=vsa.ATTN_DYNAMIC_SPLITS, workspace=ws)
        assert err == 0
        assert_attention_close(z, ref)
