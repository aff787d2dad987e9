"""The C-ABI library on the host, without a GPU: it loads, exports every function that
include/vsa.h declares, and its host-side checks return the documented status before
anything is enqueued (every call below fails such a check, so no kernel is launched)."""
import ctypes
import os
import re

import pytest

import verify_step_attention_amd as vsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")

OK, INVALID_ARG, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
BF16, F32 = 1, 0
FAKE = 0x100000                  # never dereferenced: each call fails a host check first


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return set(re.findall(r"^(?:int|size_t|vsa_status|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                          text, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vsa.LIB_PATH):
        pytest.fail(f"{vsa.LIB_PATH} is not built (run __graft_entry__.build())")
    return vsa._lib()


def test_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert declared == set(vsa.EXPORTED_SYMBOLS)
    raw = ctypes.CDLL(vsa.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name


def test_header_enums_match_binding():
    text = open(HEADER).read()
    for name, value in [("VSA_OK", OK), ("VSA_ERR_INVALID_ARG", INVALID_ARG),
                        ("VSA_ERR_UNSUPPORTED", UNSUPPORTED), ("VSA_ERR_WORKSPACE", WORKSPACE),
                        ("VSA_BF16", BF16), ("VSA_F32", F32)]:
        assert re.search(rf"\b{name}\s*=\s*{value}\b", text), name
    for name, value in [("VSA_ATTN_DYNAMIC_SPLITS", vsa.ATTN_DYNAMIC_SPLITS),
                        ("VSA_ATTN_BIDIRECTIONAL", vsa.ATTN_BIDIRECTIONAL),
                        ("VSA_ATTN_SLIDING_WINDOW", vsa.ATTN_SLIDING_WINDOW)]:
        assert re.search(rf"#define {name}\s+{value}u", text), name


def test_version_and_status_strings(lib):
    assert lib.vsa_version() > 0
    for code, name in [(OK, b"VSA_OK"), (INVALID_ARG, b"VSA_ERR_INVALID_ARG"),
                       (UNSUPPORTED, b"VSA_ERR_UNSUPPORTED"), (WORKSPACE, b"VSA_ERR_WORKSPACE")]:
        assert lib.vsa_status_string(code) == name


def test_attention_workspace_size_limits(lib):
    ok = lib.verify_attention_workspace_size(4, 32, 8, 128, 5, 8197)
    assert ok > 0 and ok % 256 == 0
    assert lib.verify_attention_workspace_size(4, 32, 8, 128, 5, 16000) >= ok
    for bad in [(4, 30, 8, 128, 5, 8197),       # Hq % Hkv != 0
                (4, 32, 8, 96, 5, 8197),        # D not in {64, 128}
                (4, 32, 8, 128, 33, 8197),      # more than 32 rows per sequence
                (4, 64, 2, 128, 5, 8197),       # (Hq / Hkv) * R > 128
                (0, 32, 8, 128, 5, 8197)]:      # no sequence
        assert lib.verify_attention_workspace_size(*bad) == 0, bad
    # (sequence, KV head) units past the workspace's counter region add their own area
    assert lib.verify_attention_workspace_size(2049, 32, 8, 128, 5, 64) >= \
        lib.verify_attention_workspace_size(2048, 32, 8, 128, 5, 64) + 8 * 4


def _attention(lib, *, q=FAKE, dtype=BF16, B=4, total=20, hq=32, hkv=8, d=128, s_max=8256,
               rows=5, mkv=8197, scale=0.0, flags=0, ws=FAKE * 256, ws_bytes=1 << 30):
    return lib.verify_attention(q, FAKE, FAKE, dtype, FAKE, FAKE, B, total, hq, hkv, d, s_max,
                                rows, mkv, scale, flags, FAKE, ws, ws_bytes, None)


def test_attention_host_checks(lib):
    assert _attention(lib, q=None) == INVALID_ARG
    assert _attention(lib, dtype=7) == INVALID_ARG
    assert _attention(lib, flags=2) == INVALID_ARG
    assert _attention(lib, flags=0x80000000) == INVALID_ARG
    assert _attention(lib, total=41) == INVALID_ARG           # more rows than B * max rows
    assert _attention(lib, mkv=9000) == INVALID_ARG           # max_kv_len > S_max
    assert _attention(lib, scale=float("nan")) == INVALID_ARG
    assert _attention(lib, scale=-1.0) == INVALID_ARG
    assert _attention(lib, d=96) == UNSUPPORTED
    assert _attention(lib, hq=64, hkv=2) == UNSUPPORTED
    assert _attention(lib, ws=None) == WORKSPACE
    assert _attention(lib, ws=FAKE * 256 + 64) == WORKSPACE   # not 256-byte aligned
    assert _attention(lib, ws_bytes=1024) == WORKSPACE


def _block(lib, *, window=0, flags=0, d=128, ws_bytes=1 << 30):
    return lib.block_attention(FAKE, FAKE, FAKE, BF16, FAKE, FAKE, 4, 20, 32, 8, d, 8256, 5,
                               8197, 0.0, window, flags, FAKE, FAKE * 256, ws_bytes, None)


def test_block_attention_host_checks(lib):
    assert _block(lib, window=-1) == INVALID_ARG
    assert _block(lib, flags=vsa.ATTN_SLIDING_WINDOW) == INVALID_ARG     # needs a window
    assert _block(lib, flags=8) == INVALID_ARG
    assert _block(lib, window=4096, d=96) == UNSUPPORTED
    assert _block(lib, window=4096, flags=vsa.ATTN_BIDIRECTIONAL, ws_bytes=1024) == WORKSPACE
    # verify_attention takes no mask flags
    assert _attention(lib, flags=vsa.ATTN_BIDIRECTIONAL) == INVALID_ARG


def _attention_kvq(lib, *, q=FAKE, bits=8, d=128, flags=0, ws_bytes=1 << 30, sb=FAKE):
    return lib.verify_attention_kvq(q, FAKE, sb, FAKE, FAKE, bits, FAKE, FAKE, 4, 20, 32, 8,
                                    d, 8256, 5, 8197, 0.0, flags, FAKE, FAKE * 256, ws_bytes,
                                    None)


def test_attention_kvq_host_checks(lib):
    assert _attention_kvq(lib, q=None) == INVALID_ARG
    assert _attention_kvq(lib, sb=None) == INVALID_ARG
    assert _attention_kvq(lib, bits=6) == INVALID_ARG
    assert _attention_kvq(lib, bits=16) == INVALID_ARG
    assert _attention_kvq(lib, flags=4) == INVALID_ARG
    assert _attention_kvq(lib, d=96) == UNSUPPORTED
    assert _attention_kvq(lib, bits=4, ws_bytes=1024) == WORKSPACE


def test_sample_workspace_size_limits(lib):
    ok = lib.verify_sample_accept_workspace_size(4, 20, 151936, 5, 0, 0)
    assert ok > 0
    assert lib.verify_sample_accept_workspace_size(4, 20, 151936, 5, 20, 5) >= ok
    for bad in [(4, 20, 1 << 30, 5, 0, 0),     # vocabulary beyond the supported maximum
                (4, 20, 151936, 5, 257, 0),    # top_k beyond 256
                (4, 20, 151936, 5, 0, 33),     # top_logprobs beyond 32
                (4, 3, 151936, 5, 0, 0),       # fewer rows than sequences
                (4, 21, 151936, 5, 0, 0)]:     # more rows than B * max rows
        assert lib.verify_sample_accept_workspace_size(*bad) == 0, bad


def _sample(lib, *, target=FAKE, drafts=FAKE, B=4, total=20, V=151936, rows=5, mtk=0, mtl=0,
            ws=FAKE * 256, ws_bytes=1 << 30):
    return lib.verify_sample_accept(target, FAKE, drafts, FAKE, None, FAKE, FAKE, 0, B, total,
                                    V, rows, mtk, mtl, FAKE, FAKE, None, None, None, None,
                                    None, ws, ws_bytes, None)


def test_sample_host_checks(lib):
    assert _sample(lib, target=None) == INVALID_ARG
    assert _sample(lib, drafts=None) == INVALID_ARG            # drafts needed when T > B
    assert _sample(lib, total=3) == INVALID_ARG
    assert _sample(lib, mtk=-1) == INVALID_ARG
    assert _sample(lib, V=1 << 30) == UNSUPPORTED
    assert _sample(lib, mtk=300) == UNSUPPORTED
    assert _sample(lib, rows=40, total=20) == UNSUPPORTED
    assert _sample(lib, ws=None) == WORKSPACE
    assert _sample(lib, ws_bytes=256) == WORKSPACE


def test_reduced_draft_host_checks(lib):
    def call(dvocab=32000, t2d=FAKE * 256, V=151936):
        return lib.verify_sample_accept_reduced_draft(
            FAKE, FAKE, dvocab, t2d, FAKE, FAKE, None, FAKE, FAKE, 0, 4, 20, V, 5, 0, 0, FAKE,
            FAKE, None, None, None, None, None, FAKE * 256, 1 << 30, None)
    assert call(t2d=None) == INVALID_ARG                      # a reduced vocab needs t2d
    assert call(dvocab=0) == INVALID_ARG
    assert call(dvocab=151937) == INVALID_ARG                 # larger than V
    assert call(t2d=FAKE * 256 + 4) == INVALID_ARG            # t2d not 16-byte aligned
    assert lib.draft_vocab_inverse(None, 10, 100, FAKE * 256, None) == INVALID_ARG
    assert lib.draft_vocab_inverse(FAKE, 101, 100, FAKE * 256, None) == INVALID_ARG
    assert lib.draft_vocab_inverse(FAKE, 10, 100, FAKE * 256 + 8, None) == INVALID_ARG


def test_small_m_qmm_host_checks(lib):
    assert lib.small_m_qmm_workspace_size(17, 1024, 4096) == 0     # more than 16 rows
    assert lib.small_m_qmm_workspace_size(8, 1024, 100) == 0       # K not a multiple of 64
    assert lib.small_m_qmm_workspace_size(8, 1024, 4096) > 0
    call = lambda **kw: lib.small_m_qmm(kw.get("x", FAKE * 256), FAKE * 256, FAKE * 256,
                                        kw.get("bits", 4), kw.get("M", 8), 1024,
                                        kw.get("K", 4096), FAKE * 256, kw.get("ws", FAKE * 256),
                                        kw.get("ws_bytes", 1 << 30), None)
    assert call(x=None) == INVALID_ARG
    assert call(bits=6) == INVALID_ARG
    assert call(x=FAKE * 256 + 2) == INVALID_ARG                    # x not 16-byte aligned
    assert call(M=17) == UNSUPPORTED
    assert call(K=4000) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE                               # splits need partials
