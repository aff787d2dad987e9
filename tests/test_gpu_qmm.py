"""GPU parity of small_m_qmm (few-row quantized matmul) against the CPU oracle through the C
ABI. Bound, from the arithmetic: codes and the power-of-two-scaled x are exact fp16
operands, every product is exact in fp32, and the sums round in fp32 (MFMA partial sums,
one fma per group for scale and bias, the split reduction), so
    |gpu - oracle| <= 2^-22 (K / 64 + 128) sum_k |x[m][k]| (|scale * code| + |bias|)
elementwise, the right side computed by the test in fp64."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_step_attention_amd as vsa  # noqa: E402
from verify_step_attention_amd import workloads as wl  # noqa: E402


def _log(msg):
    print(msg, flush=True)


def _problem(m, n, k, bits, seed):
    rng = np.random.default_rng(seed)
    xb = wl.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[:, :64] += 0.05                                      # groups with an offset
    codes, sb = wl.quantize_kv(w, bits)
    return xb, codes, sb


def _gpu(xb, codes, sb, bits, m, n, k):
    size = vsa.small_m_qmm_workspace_size(m, n, k)
    assert size > 0
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    x = torch.from_numpy(xb).cuda().view(torch.bfloat16)
    vsa.small_m_qmm(x, torch.from_numpy(codes).cuda(), torch.from_numpy(sb).cuda(), bits, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check(got, xb, codes, sb, bits, rows=None):
    from oracle.attention import dequantize_kv
    from oracle.qmm import small_m_qmm
    if rows is not None:
        codes, sb = codes[rows], sb[rows]
        got = got[:, rows]
    x = wl.bf16_to_f32(xb)
    ref = small_m_qmm(x, codes, sb, bits)
    k = x.shape[1]
    one = np.ones_like(sb)
    one[..., 1] = 0
    mag = np.abs(dequantize_kv(codes, np.abs(sb) * one, bits)) + np.repeat(
        np.abs(sb[..., 1]).astype(np.float64), 64, axis=-1)
    bound = 2.0 ** -22 * (k / 64 + 128) * (np.abs(x).astype(np.float64) @ mag.T) + 1e-30
    assert not np.isnan(got).any()
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > bound
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} out of bound, max err {err.max():.3e}"


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m,n,k", [
    (8, 1024, 5120),        # many splits of a 27B-class input width
    (16, 384, 1024),
    (1, 256, 64),           # one row, one group
    (5, 1000, 704),         # N not a multiple of 4 or of 128; a partial chunk
    (3, 37, 2048),          # fewer rows than one tile
    (16, 64, 25600),        # the widest input, most splits
])
def test_parity(m, n, k, bits):
    _log(f"small_m_qmm parity M {m} N {n} K {k} bits {bits}")
    xb, codes, sb = _problem(m, n, k, bits, seed=m * 7 + bits)
    _check(_gpu(xb, codes, sb, bits, m, n, k), xb, codes, sb, bits)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m,n,k", [(8, 10240, 5120), (16, 5120, 8192), (8, 25600, 5120)])
def test_full_size_sampled_columns(m, n, k, bits):
    """27B-class projections at full size; the oracle computes 256 sampled outputs."""
    _log(f"small_m_qmm full size M {m} N {n} K {k} bits {bits}")
    xb, codes, sb = _problem(m, n, k, bits, seed=n + bits)
    got = _gpu(xb, codes, sb, bits, m, n, k)
    rows = np.sort(np.random.default_rng(n).choice(n, size=256, replace=False))
    _check(got, xb, codes, sb, bits, rows=rows)


def test_deterministic_and_row_independent():
    _log("small_m_qmm: repeat bitwise, rows independent of the others")
    xb, codes, sb = _problem(16, 512, 4096, 4, seed=3)
    a = _gpu(xb, codes, sb, 4, 16, 512, 4096)
    b = _gpu(xb, codes, sb, 4, 16, 512, 4096)
    assert np.array_equal(a, b)
    c = _gpu(np.ascontiguousarray(xb[:5]), codes, sb, 4, 5, 512, 4096)
    assert np.array_equal(a[:5], c)


def test_host_rejects_bad_arguments():
    xb, codes, sb = _problem(2, 16, 128, 8, seed=1)
    x = torch.from_numpy(xb).cuda().view(torch.bfloat16)
    y = torch.empty((2, 16), dtype=torch.float32, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        vsa.small_m_qmm(x, torch.from_numpy(codes).cuda(), torch.from_numpy(sb).cuda(), 4, y, ws)
