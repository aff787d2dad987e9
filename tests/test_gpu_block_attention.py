"""GPU parity of block_attention (a drafter's block over its context: a recent or sliding
window, causal or bidirectional in the block) against the CPU oracle, elementwise
|gpu - oracle| <= 1e-3 + 2e-3 |oracle|, through the C ABI. Keys below the first one any row
sees are NaN in these caches, as are keys past each block: the result must not touch them."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_step_attention_amd as vsa  # noqa: E402
from verify_step_attention_amd import workloads as wl  # noqa: E402
from gpu_helpers import assert_attention_close, attention_gpu  # noqa: E402
from test_gpu_attention import _custom  # noqa: E402

BIDIR, SLIDING, DYN = vsa.ATTN_BIDIRECTIONAL, vsa.ATTN_SLIDING_WINDOW, vsa.ATTN_DYNAMIC_SPLITS


def _log(msg):
    print(msg, flush=True)


def _poison_below_window(w, window, flags):
    from oracle.attention import block_visible_range
    nan = np.uint16(0x7FC0) if w.dtype == wl.BF16 else np.float32(np.nan)
    rows = np.diff(w.cu_rows)
    for b in range(w.batch):
        lo, _ = block_visible_range(int(w.ctx_lens[b]), int(rows[b]), 0, window,
                                    bool(flags & SLIDING), bool(flags & BIDIR))
        w.k_cache[b, :, :lo] = nan
        w.v_cache[b, :, :lo] = nan


def block_gpu(w, window, flags, max_kv_len=None):
    dev = wl.device_tensors(w)
    mkv = max_kv_len or w.max_kv_len
    size = vsa.verify_attention_workspace_size(w.batch, w.num_q_heads, w.num_kv_heads,
                                               w.head_dim, w.max_rows, mkv)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    out = torch.full((w.total_rows, w.num_q_heads, w.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    vsa.block_attention(dev["q"], dev["k_cache"], dev["v_cache"], dev["cu_rows"],
                        dev["ctx_lens"], out, ws, max_rows_per_seq=w.max_rows,
                        max_kv_len=mkv, window=window, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(ws[:4].view(torch.int32).item())


def block_oracle(w, window, flags):
    from oracle.attention import block_attention
    k, v = w.kv_f32()
    return block_attention(w.q_f32(), k, v, w.cu_rows, w.ctx_lens, w.num_q_heads,
                           w.num_kv_heads, window=window, sliding=bool(flags & SLIDING),
                           bidirectional=bool(flags & BIDIR))


CASES = [
    # (Hq, Hkv, D, dtype, ctx list, drafts list (rows - 1), window, mask flags)
    (32, 8, 128, wl.BF16, [8192, 3000, 5000], [7, 7, 7], 4096, 0),       # block 8, recent
    (32, 8, 128, wl.BF16, [8192, 3000, 5000], [7, 7, 7], 4096, BIDIR),   # DeepSpec-style
    (32, 8, 128, wl.BF16, [6000, 100, 0], [14, 14, 14], 2048, SLIDING),  # block 15, trained
    (32, 8, 128, wl.BF16, [2500, 1100], [7, 7], 1024, SLIDING | BIDIR),
    (64, 8, 128, wl.BF16, [5000], [15], 4096, BIDIR),                    # 128 columns
    (32, 8, 128, wl.BF16, [3000, 200], [7, 3], 4096, 0),                 # window > context
    (32, 8, 128, wl.BF16, [777, 64], [7, 7], 1, SLIDING),                # own key only
    (32, 8, 128, wl.BF16, [4000, 129], [7, 7], 127, 0),                  # lo inside a tile
    (16, 2, 64, wl.BF16, [700, 3000], [7, 3], 256, SLIDING | BIDIR),     # D = 64
    (8, 2, 64, wl.F32, [300, 50], [3, 7], 100, 0),                       # fp32 path
    (8, 2, 64, wl.F32, [300, 50], [3, 7], 40, SLIDING | BIDIR),
]


@pytest.mark.parametrize("dyn", [0, DYN])
@pytest.mark.parametrize("case", CASES)
def test_block_parity(case, dyn):
    hq, hkv, d, dtype, ctxs, drafts, window, mask = case
    _log(f"block attention parity {case} dyn {dyn}")
    w = _custom(hq, hkv, d, dtype, ctxs, drafts)
    _poison_below_window(w, window, mask)
    got, err = block_gpu(w, window, mask | dyn)
    assert err == 0
    assert_attention_close(got, block_oracle(w, window, mask))


def test_window_zero_is_verify_attention():
    _log("block attention, no window, causal == verify_attention (bitwise)")
    w = wl.make_workload("batched")
    got, err = block_gpu(w, 0, 0)
    ref, err2 = attention_gpu(w)
    assert err == 0 and err2 == 0
    assert np.array_equal(got, ref)


def test_recent_window_on_bench_shape():
    _log("block attention: verify_b4k4_ctx8192 with a 4096-row window, both masks")
    w = wl.make_workload("verify_b4k4_ctx8192")
    for mask in (0, BIDIR):
        got, err = block_gpu(w, 4096, mask | DYN)
        assert err == 0
        assert_attention_close(got, block_oracle(w, 4096, mask))


_DRAFTER = {}


@pytest.mark.parametrize("mask", [0, BIDIR, SLIDING])
def test_drafter_workload_full_size(mask):
    """The benchmark's drafter shape (4 blocks of 8 rows over 32768 context tokens) with the
    pages' 4096-row window, in the benchmark's launch configuration (dynamic splits)."""
    _log(f"block attention: drafter_b4r8_ctx32768, window 4096, mask {mask}")
    if "w" not in _DRAFTER:
        _DRAFTER["w"] = wl.make_workload("drafter_b4r8_ctx32768")
    w = _DRAFTER["w"]
    got, err = block_gpu(w, 4096, mask | DYN)
    assert err == 0
    assert_attention_close(got, block_oracle(w, 4096, mask))


def test_host_rejects_bad_window_flags():
    w = _custom(8, 2, 64, wl.BF16, [10], [2])
    for window, flags in [(-1, 0), (0, SLIDING), (4, 8)]:
        with pytest.raises(vsa.VsaError):
            block_gpu(w, window, flags)
