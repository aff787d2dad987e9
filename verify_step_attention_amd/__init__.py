"""MI355X (gfx950) library for the batched verify step of lossless speculative decoding.

Python binding of the C ABI in include/vsa.h: argument marshalling only. Every step of the
verify path runs in the HIP kernels of libvsa.so; torch is used for device memory and
streams. Importing this package never loads the library; the first call does, and fails
loudly if libvsa.so has not been built (`python -m verify_step_attention_amd.build`).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa.so")

VSA_OK, VSA_ERR_INVALID_ARG, VSA_ERR_UNSUPPORTED, VSA_ERR_WORKSPACE, VSA_ERR_LAUNCH = range(5)
VSA_F32, VSA_BF16 = 0, 1
DEVERR_SEQ_SHAPE = 0x01
DEVERR_DRAFT_ID = 0x02
DEVERR_PARAMS = 0x04
DEVERR_NO_DRAFT_LOGITS = 0x08
DEVERR_TIE_OVERFLOW = 0x10
DEVERR_WAIT_TIMEOUT = 0x20
DEVERR_DRAFT_MAP = 0x40

# attention flags (verify_attention: only ATTN_DYNAMIC_SPLITS)
ATTN_DYNAMIC_SPLITS = 0x1
ATTN_BIDIRECTIONAL = 0x2
ATTN_SLIDING_WINDOW = 0x4

# vsa_row_params, field for field
ROW_PARAMS_DTYPE = np.dtype([("temperature", "<f4"), ("top_k", "<i4"), ("top_p", "<f4"),
                             ("presence_penalty", "<f4"), ("frequency_penalty", "<f4"),
                             ("logprobs", "<i4"), ("top_logprobs", "<i4")])

EXPORTED_SYMBOLS = ("vsa_version", "vsa_status_string", "verify_attention_workspace_size",
                    "verify_attention", "block_attention", "verify_attention_kvq",
                    "verify_sample_accept_workspace_size", "verify_sample_accept",
                    "draft_vocab_inverse", "verify_sample_accept_reduced_draft",
                    "verify_sample_accept_onehot",
                    "small_m_qmm_workspace_size", "small_m_qmm", "verify_attention_noalloc")


class VsaError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m verify_step_attention_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        c_int, c_size, c_void, c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, \
            ctypes.c_float
        lib.vsa_version.restype = c_int
        lib.vsa_status_string.restype = ctypes.c_char_p
        lib.vsa_status_string.argtypes = [c_int]
        lib.verify_attention_workspace_size.restype = c_size
        lib.verify_attention_workspace_size.argtypes = [c_int] * 6
        lib.verify_attention.restype = c_int
        lib.verify_attention.argtypes = [c_void, c_void, c_void, c_int, c_void, c_void,
                                         c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                         c_int, c_float, ctypes.c_uint32, c_void, c_void,
                                         c_size, c_void]
        lib.verify_attention_noalloc.restype = c_int
        lib.verify_attention_noalloc.argtypes = [c_void, c_void, c_void, c_int, c_void, c_void,
                                                 c_int, c_int, c_int, c_int, c_int, c_int,
                                                 c_int, c_int, c_float, ctypes.c_uint32, c_void,
                                                 c_void, c_void]
        lib.block_attention.restype = c_int
        lib.block_attention.argtypes = [c_void, c_void, c_void, c_int, c_void, c_void,
                                        c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                        c_int, c_float, c_int, ctypes.c_uint32, c_void,
                                        c_void, c_size, c_void]
        lib.verify_attention_kvq.restype = c_int
        lib.verify_attention_kvq.argtypes = [c_void, c_void, c_void, c_void, c_void, c_int,
                                             c_void, c_void, c_int, c_int, c_int, c_int,
                                             c_int, c_int, c_int, c_int, c_float,
                                             ctypes.c_uint32, c_void, c_void, c_size, c_void]
        lib.verify_sample_accept_workspace_size.restype = c_size
        lib.verify_sample_accept_workspace_size.argtypes = [c_int] * 6
        lib.verify_sample_accept.restype = c_int
        lib.verify_sample_accept.argtypes = [c_void, c_void, c_void, c_void, c_void, c_void,
                                             c_void, ctypes.c_uint64, c_int, c_int, c_int,
                                             c_int, c_int, c_int, c_void, c_void, c_void,
                                             c_void, c_void, c_void, c_void, c_void, c_size,
                                             c_void]
        lib.draft_vocab_inverse.restype = c_int
        lib.draft_vocab_inverse.argtypes = [c_void, c_int, c_int, c_void, c_void]
        lib.verify_sample_accept_reduced_draft.restype = c_int
        lib.verify_sample_accept_reduced_draft.argtypes = [
            c_void, c_void, c_int, c_void, c_void, c_void, c_void, c_void, c_void,
            ctypes.c_uint64, c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void, c_void,
            c_void, c_void, c_void, c_void, c_void, c_size, c_void]
        lib.verify_sample_accept_onehot.restype = c_int
        lib.verify_sample_accept_onehot.argtypes = [c_void, c_void, c_void, c_void, c_void,
                                                    c_void, ctypes.c_uint64, c_int, c_int,
                                                    c_int, c_int, c_int, c_int, c_void, c_void,
                                                    c_void, c_void, c_void, c_void, c_void,
                                                    c_void, c_size, c_void]
        lib.small_m_qmm_workspace_size.restype = c_size
        lib.small_m_qmm_workspace_size.argtypes = [c_int, c_int, c_int]
        lib.small_m_qmm.restype = c_int
        lib.small_m_qmm.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_void,
                                    c_void, c_size, c_void]
        _lib_handle = lib
    return _lib_handle


def library():
    """The loaded ctypes handle of libvsa.so."""
    return _lib()


def vsa_version():
    return _lib().vsa_version()


def status_string(status):
    return _lib().vsa_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status, where):
    if status != VSA_OK:
        raise VsaError(status, where)


# ----------------------------------------------------------------------------- attention
def verify_attention_workspace_size(B, Hq, Hkv, D, max_rows_per_seq, max_kv_len):
    return int(_lib().verify_attention_workspace_size(B, Hq, Hkv, D, max_rows_per_seq,
                                                      max_kv_len))


def _attention_dtype(q, k_cache, v_cache, out, cu_rows, ctx_lens, workspace):
    import torch
    total, hq, d = q.shape
    batch, hkv, s_max, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q / k_cache / v_cache shapes disagree")
    if q.dtype == torch.bfloat16:
        dtype = VSA_BF16
    elif q.dtype == torch.float32:
        dtype = VSA_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or out.dtype != torch.float32:
        raise ValueError("dtype mismatch")
    for t in (q, k_cache, v_cache, cu_rows, ctx_lens, out, workspace):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dtype


def block_attention(q, k_cache, v_cache, cu_rows, ctx_lens, out, workspace, *,
                    max_rows_per_seq, max_kv_len, window=0, scale=0.0, flags=0, stream=None):
    """A drafter's block over its context: verify_attention's arguments plus window (0 =
    the whole context) and flags (ATTN_DYNAMIC_SPLITS | ATTN_BIDIRECTIONAL |
    ATTN_SLIDING_WINDOW)."""
    dtype = _attention_dtype(q, k_cache, v_cache, out, cu_rows, ctx_lens, workspace)
    total, hq, d = q.shape
    batch, hkv, s_max, _ = k_cache.shape
    st = _lib().block_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), dtype, _ptr(cu_rows),
                                _ptr(ctx_lens), batch, total, hq, hkv, d, s_max,
                                int(max_rows_per_seq), int(max_kv_len), float(scale),
                                int(window), int(flags), _ptr(out), _ptr(workspace),
                                workspace.numel(), _stream(stream))
    _check(st, "block_attention")


def verify_attention(q, k_cache, v_cache, cu_rows, ctx_lens, out, workspace, *,
                     max_rows_per_seq, max_kv_len, scale=0.0, flags=0, stream=None):
    """q [T, Hq, D], k_cache / v_cache [B, Hkv, S_max, D] (bf16 or float32 tensors on the
    GPU), cu_rows [B+1] / ctx_lens [B] int32, out [T, Hq, D] float32, workspace uint8;
    flags 0 or ATTN_DYNAMIC_SPLITS."""
    dtype = _attention_dtype(q, k_cache, v_cache, out, cu_rows, ctx_lens, workspace)
    total, hq, d = q.shape
    batch, hkv, s_max, _ = k_cache.shape
    st = _lib().verify_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), dtype, _ptr(cu_rows),
                                 _ptr(ctx_lens), batch, total, hq, hkv, d, s_max,
                                 int(max_rows_per_seq), int(max_kv_len), float(scale),
                                 int(flags), _ptr(out), _ptr(workspace), workspace.numel(),
                                 _stream(stream))
    _check(st, "verify_attention")


NOALLOC_SCRATCH_BYTES = 16 << 20


def verify_attention_noalloc(q, k_cache, v_cache, cu_rows, ctx_lens, out, device_error=None,
                             *, max_rows_per_seq, max_kv_len, scale=0.0, flags=0, stream=None):
    """verify_attention without a workspace: the library's static per-GPU scratch holds the
    partial results. device_error: None or a one-element int32/uint32 device tensor that
    receives the device error bits."""
    dtype = _attention_dtype(q, k_cache, v_cache, out, cu_rows, ctx_lens, out)
    if device_error is not None and (device_error.numel() < 1 or
                                     device_error.element_size() != 4):
        raise ValueError("device_error must hold one 32-bit word")
    total, hq, d = q.shape
    batch, hkv, s_max, _ = k_cache.shape
    st = _lib().verify_attention_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), dtype,
                                         _ptr(cu_rows), _ptr(ctx_lens), batch, total, hq, hkv,
                                         d, s_max, int(max_rows_per_seq), int(max_kv_len),
                                         float(scale), int(flags), _ptr(out),
                                         _ptr(device_error), _stream(stream))
    _check(st, "verify_attention_noalloc")


def verify_attention_kvq(q, k_codes, k_sb, v_codes, v_sb, bits, cu_rows, ctx_lens, out,
                         workspace, *, max_rows_per_seq, max_kv_len, scale=0.0, flags=0,
                         stream=None):
    """verify_attention over a quantized K/V cache: q [T, Hq, D] bf16, k_codes / v_codes
    [B, Hkv, S_max, D * bits / 8] uint8, k_sb / v_sb [B, Hkv, S_max, D / 64, 2] float16
    (scale, bias), bits 8 or 4; the rest as verify_attention (same workspace size)."""
    import torch
    total, hq, d = q.shape
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    batch, hkv, s_max, rowb = k_codes.shape
    if q.dtype != torch.bfloat16 or out.dtype != torch.float32:
        raise ValueError("q must be bfloat16 and out float32")
    if rowb * 8 != d * bits or tuple(v_codes.shape) != tuple(k_codes.shape):
        raise ValueError("code arrays disagree with q / bits")
    if k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8")
    if tuple(k_sb.shape) != (batch, hkv, s_max, d // 64, 2) or \
            tuple(v_sb.shape) != tuple(k_sb.shape) or k_sb.dtype != torch.float16 or \
            v_sb.dtype != torch.float16:
        raise ValueError("scale / bias arrays must be float16 [B, Hkv, S_max, D/64, 2]")
    for t in (q, k_codes, k_sb, v_codes, v_sb, cu_rows, ctx_lens, out, workspace):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    st = _lib().verify_attention_kvq(_ptr(q), _ptr(k_codes), _ptr(k_sb), _ptr(v_codes),
                                     _ptr(v_sb), int(bits), _ptr(cu_rows), _ptr(ctx_lens),
                                     batch, total, hq, hkv, d, s_max, int(max_rows_per_seq),
                                     int(max_kv_len), float(scale), int(flags), _ptr(out),
                                     _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "verify_attention_kvq")


# ----------------------------------------------------------------------------- sampling
def verify_sample_accept_workspace_size(B, total_rows, V, max_rows_per_seq, max_top_k,
                                        max_top_logprobs):
    return int(_lib().verify_sample_accept_workspace_size(B, total_rows, V, max_rows_per_seq,
                                                          max_top_k, max_top_logprobs))


def pack_row_params(params):
    """List of objects with the vsa_row_params fields -> numpy structured array."""
    arr = np.zeros(len(params), dtype=ROW_PARAMS_DTYPE)
    for i, p in enumerate(params):
        for name in ROW_PARAMS_DTYPE.names:
            arr[i][name] = getattr(p, name)
    return arr


def verify_sample_accept(target_logits, draft_logits, draft_tokens, cu_rows, token_counts,
                         params, positions, seed, accepted_len, out_tokens, workspace, *,
                         max_rows_per_seq, max_top_k, max_top_logprobs, chosen_logprob=None,
                         top_lp_vals=None, top_lp_ids=None, diag_threshold=None,
                         diag_kept=None, stream=None):
    """target_logits [T, V] float32, draft_logits [T-B, V] float32 or None, draft_tokens
    [T-B] int32, cu_rows [B+1] int32, token_counts [B, V] int32 or None, params: a device
    uint8 tensor holding B packed vsa_row_params (see pack_row_params), positions [B] int32;
    outputs as in include/vsa.h."""
    total, vocab = target_logits.shape
    batch = cu_rows.numel() - 1
    st = _lib().verify_sample_accept(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(cu_rows),
        _ptr(token_counts), _ptr(params), _ptr(positions),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), batch, total, vocab,
        int(max_rows_per_seq), int(max_top_k), int(max_top_logprobs), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(chosen_logprob), _ptr(top_lp_vals), _ptr(top_lp_ids),
        _ptr(diag_threshold), _ptr(diag_kept), _ptr(workspace), workspace.numel(),
        _stream(stream))
    _check(st, "verify_sample_accept")


def verify_sample_accept_onehot(target_logits, draft_tokens, cu_rows, token_counts, params,
                                positions, seed, accepted_len, out_tokens, workspace, *,
                                max_rows_per_seq, max_top_k, max_top_logprobs,
                                chosen_logprob=None, top_lp_vals=None, top_lp_ids=None,
                                diag_threshold=None, diag_kept=None, stream=None):
    """verify_sample_accept for one-hot proposals (prompt-lookup drafts): no draft logits,
    q_t = 1 at d_t and 0 elsewhere; arguments otherwise as verify_sample_accept."""
    total, vocab = target_logits.shape
    batch = cu_rows.numel() - 1
    st = _lib().verify_sample_accept_onehot(
        _ptr(target_logits), _ptr(draft_tokens), _ptr(cu_rows), _ptr(token_counts),
        _ptr(params), _ptr(positions), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), batch,
        total, vocab, int(max_rows_per_seq), int(max_top_k), int(max_top_logprobs),
        _ptr(accepted_len), _ptr(out_tokens), _ptr(chosen_logprob), _ptr(top_lp_vals),
        _ptr(top_lp_ids), _ptr(diag_threshold), _ptr(diag_kept), _ptr(workspace),
        workspace.numel(), _stream(stream))
    _check(st, "verify_sample_accept_onehot")


def draft_vocab_inverse(d2t, vocab, t2d, stream=None):
    """Reduced draft vocabulary: d2t [V_d] int32 offsets (target id = j + d2t[j]) -> t2d [V]
    int32 (draft id of each target id, -1 where none), both device tensors."""
    if d2t.dtype != t2d.dtype or t2d.numel() != vocab or not d2t.is_contiguous() or \
            not t2d.is_contiguous():
        raise ValueError("d2t / t2d must be contiguous int32 tensors, t2d of size V")
    _check(_lib().draft_vocab_inverse(_ptr(d2t), d2t.numel(), int(vocab), _ptr(t2d),
                                      _stream(stream)), "draft_vocab_inverse")


def verify_sample_accept_reduced_draft(target_logits, draft_logits, t2d, draft_tokens, cu_rows,
                                       token_counts, params, positions, seed, accepted_len,
                                       out_tokens, workspace, *, max_rows_per_seq, max_top_k,
                                       max_top_logprobs, chosen_logprob=None, top_lp_vals=None,
                                       top_lp_ids=None, diag_threshold=None, diag_kept=None,
                                       stream=None):
    """verify_sample_accept with draft_logits [T-B, V_d] over a reduced draft vocabulary and
    t2d [V] int32 from draft_vocab_inverse; everything else in target ids as before."""
    total, vocab = target_logits.shape
    batch = cu_rows.numel() - 1
    dvocab = draft_logits.shape[1] if draft_logits is not None else vocab
    st = _lib().verify_sample_accept_reduced_draft(
        _ptr(target_logits), _ptr(draft_logits), int(dvocab), _ptr(t2d), _ptr(draft_tokens),
        _ptr(cu_rows), _ptr(token_counts), _ptr(params), _ptr(positions),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), batch, total, vocab,
        int(max_rows_per_seq), int(max_top_k), int(max_top_logprobs), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(chosen_logprob), _ptr(top_lp_vals), _ptr(top_lp_ids),
        _ptr(diag_threshold), _ptr(diag_kept), _ptr(workspace), workspace.numel(),
        _stream(stream))
    _check(st, "verify_sample_accept_reduced_draft")


# ----------------------------------------------------------------------------- verify matmul
def small_m_qmm_workspace_size(M, N, K):
    return int(_lib().small_m_qmm_workspace_size(int(M), int(N), int(K)))


def small_m_qmm(x, codes, sb, bits, y, workspace, stream=None):
    """y [M, N] float32 = x [M, K] bf16 times the quantized weights' transpose: codes
    [N, K * bits / 8] uint8, sb [N, K / 64, 2] float16 (scale, bias), bits 8 or 4; M <= 16.
    workspace: uint8 device tensor of small_m_qmm_workspace_size(M, N, K) bytes."""
    import torch
    m, k = x.shape
    n = codes.shape[0]
    if x.dtype != torch.bfloat16 or y.dtype != torch.float32 or codes.dtype != torch.uint8 \
            or sb.dtype != torch.float16:
        raise ValueError("x bf16, codes uint8, sb float16, y float32")
    if tuple(codes.shape) != (n, k * bits // 8) or tuple(sb.shape) != (n, k // 64, 2) or \
            tuple(y.shape) != (m, n):
        raise ValueError("shapes disagree")
    for t in (x, codes, sb, y, workspace):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    st = _lib().small_m_qmm(_ptr(x), _ptr(codes), _ptr(sb), int(bits), m, n, k, _ptr(y),
                            _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "small_m_qmm")
