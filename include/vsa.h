/*
 * vsa.h -- C ABI of the MI355X (gfx950) library for the batched verify step of lossless
 * speculative decoding.
 *
 * The step (as the mlx-dspark pages describe it): a target model verifies, for each of B
 * sequences, a block of R_b = K_b + 1 rows -- the last committed token (the "anchor") and
 * K_b drafted tokens -- in one forward pass, then accepts a prefix of the drafts.
 *   - verify_attention: the multi-row causal attention of those rows against the
 *     sequence's KV cache (mlx-dspark Changelog [0.20.0] "Added": multi-row decode
 *     attention over the whole KV cache, every GQA head x query row of a KV head consuming
 *     each KV tile; [0.3.1] "Fixed": native GQA, n_kv-head K/V with no tiling).
 *   - verify_sample_accept: penalties, temperature, top-k / top-p truncation and
 *     acceptance over the full vocabulary (Changelog [0.2.0] "Added": presence/frequency
 *     penalties per verify position, logprobs / top_logprobs; [0.20.2] "Changed": top-k
 *     threshold and nucleus cutoff without full-vocabulary sorts; release v0.1.0
 *     "Highlights": truncation of both draft and target; release v0.0.2 "Highlights":
 *     accept with probability min(1, p/q), resample the residual on rejection, greedy by
 *     default; Changelog [0.2.0] "Decode-path performance": greedy acceptance as the
 *     cumulative product of positionwise matches, one device sync per round).
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers into caller-owned memory (e.g. torch
 *     tensors' data_ptr()), row-major and densely packed, unless stated otherwise.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue work: they
 *     never synchronize and never allocate. Results are valid once the stream reaches the
 *     point after the call.
 *   - Host-checkable argument errors return a status before anything is enqueued. A launch
 *     failure returns VSA_ERR_LAUNCH.
 *   - Values only the device can see (lengths, token ids, per-sequence parameters) get
 *     defined behaviour (clamped, or the row is treated as stated below) and set a bit in
 *     the workspace's device error word: the uint32 at byte 0 of `workspace`. Bits are ORed
 *     in and never cleared by the library; the caller reads (and may zero) it after the
 *     stream completes.
 *   - Workspace: caller-owned device memory of at least *_workspace_size() bytes, 256-byte
 *     aligned, ZERO-FILLED BEFORE ITS FIRST USE. Every workspace starts with the same header:
 *     the error word (byte 0) and, from byte 256, a 64 KB region of counters that every call
 *     returns to zero and no call uses for anything else (a call that needs more than 16384
 *     counters keeps the rest in its own area and clears them first). So one workspace
 *     serves any number of calls of any of these functions and shapes in stream order. Two calls that
 *     share a workspace must not run concurrently (different streams), and a workspace
 *     sized for one problem serves any problem whose size query is not larger.
 *   - No call keeps state between calls; the library is reentrant across workspaces.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vsa_status {
    VSA_OK = 0,
    VSA_ERR_INVALID_ARG = 1,  /* a host-side argument is null, negative or inconsistent */
    VSA_ERR_UNSUPPORTED = 2,  /* valid but outside the supported shapes (see limits) */
    VSA_ERR_WORKSPACE = 3,    /* workspace missing, misaligned or too small */
    VSA_ERR_LAUNCH = 4,       /* the HIP runtime refused a launch */
    VSA_STATUS_MAX_ENUM = 0x7fffffff  /* not a status: gives the type the range of int */
} vsa_status;

typedef enum vsa_dtype {
    VSA_F32 = 0,              /* IEEE binary32 */
    VSA_BF16 = 1,             /* bfloat16 bit patterns (uint16) */
    VSA_DTYPE_MAX_ENUM = 0x7fffffff  /* not a type: any int a caller passes is a value of
                                        the enumeration, and other values are rejected */
} vsa_dtype;

/* Device error word bits (uint32 at workspace byte 0). */
#define VSA_DEVERR_SEQ_SHAPE      0x01u /* R_b outside [1, max_rows_per_seq], ctx_b < 0, or
                                           ctx_b + R_b > S_max or > max_kv_len: the
                                           sequence is clamped into range */
#define VSA_DEVERR_DRAFT_ID       0x02u /* a draft token id outside [0, V): that draft is
                                           rejected and adds nothing to penalty counts */
#define VSA_DEVERR_PARAMS         0x04u /* a sequence's parameters are out of range
                                           (T < 0 or not finite, top_p outside (0, 1],
                                           top_k < 0 or > max_top_k, top_logprobs outside
                                           [0, max_top_logprobs], a nucleus without top-k
                                           when max_top_k = 0): the sequence is verified
                                           greedily with no logprobs */
#define VSA_DEVERR_NO_DRAFT_LOGITS 0x08u /* T > 0 but draft_logits is NULL: greedy */
#define VSA_DEVERR_TIE_OVERFLOW   0x10u /* more ids tie at a top-k threshold than the
                                           candidate capacity holds: the kept set is
                                           truncated to the capacity */
#define VSA_DEVERR_WAIT_TIMEOUT   0x20u /* a workgroup gave up waiting for its sequence's
                                           statistics (the call's workgroups did not all
                                           run at once, e.g. other work held the GPU) and
                                           handed its share of the draw to another: the
                                           outputs are still exact, the call was slower */
#define VSA_DEVERR_DRAFT_MAP      0x40u /* a t2d entry outside [-1, draft_vocab): read as
                                           "no draft id" (probability 0) */

/* Per-sequence sampling parameters: the request parameters the pages list (temperature,
 * top_p, top_k, presence/frequency penalty, logprobs, top_logprobs; release v0.1.0 and
 * Changelog [0.2.0]). 28 bytes, 4-byte aligned, field order fixed. */
typedef struct vsa_row_params {
    float temperature;        /* 0 => greedy; > 0 => sampled at this temperature */
    int32_t top_k;            /* 0 => off; else keep every id whose penalized logit is >= the
                                 k-th largest (ties at the threshold are kept) */
    float top_p;              /* 1 => off; in (0, 1): nucleus over the top-k set, or
                                 over the whole vocabulary when top-k is off */
    float presence_penalty;   /* subtracted once from every id with count > 0 */
    float frequency_penalty;  /* subtracted count times from every id */
    int32_t logprobs;         /* nonzero => write the chosen token's raw logprob */
    int32_t top_logprobs;     /* number of raw top logprobs to write per row */
} vsa_row_params;

/* Library version (major * 10000 + minor * 100 + patch). */
int vsa_version(void);

/* Human-readable name of a status code (static string). */
const char* vsa_status_string(vsa_status status);

/* ------------------------------------------------------------------------------------
 * verify_attention
 *
 * For sequence b (rows cu_rows[b] .. cu_rows[b+1]-1, R_b rows, ctx_b = ctx_lens[b] cached
 * tokens before the block, whose K/V the caller has already written at cache positions
 * ctx_b .. ctx_b + R_b - 1), verify row i and query head h, with G = Hq / Hkv:
 *     g = h / G;  n = ctx_b + i + 1   (row i sees the cache and block rows 0..i)
 *     out[row][h][:] = sum_{t<n} softmax_t(scale * <q[row][h], k[b][g][t]>) v[b][g][t][:]
 * computed with fp32 accumulation (bf16 products are exact in fp32).
 *
 *   q          [total_rows, Hq, D]     dtype
 *   k_cache    [B, Hkv, S_max, D]      dtype (positions >= ctx_b + R_b never enter the
 *                                      result; reads stay below max_kv_len)
 *   v_cache    [B, Hkv, S_max, D]      dtype
 *   dtype      VSA_BF16 (MFMA path) or VSA_F32
 *   cu_rows    [B + 1] int32           0 = cu_rows[0] < cu_rows[1] < ... = total_rows
 *   ctx_lens   [B] int32
 *   B, total_rows, Hq, Hkv, D, S_max   host sizes; Hq % Hkv == 0; D in {64, 128}
 *   max_rows_per_seq  host bound >= every R_b (at most 32)
 *   max_kv_len host bound >= every ctx_b + R_b (sizes the key split; <= S_max)
 *   scale      softmax scale; 0 => 1/sqrt(D)
 *   flags      0, or VSA_ATTN_DYNAMIC_SPLITS (other bits: VSA_ERR_INVALID_ARG)
 *   out        [total_rows, Hq, D] float32, written for every row
 * Limits: (Hq / Hkv) * max_rows_per_seq <= 128; B * Hkv <= 4194304.
 *
 * The keys of each (sequence, KV head) are split over several workgroups whose partial
 * softmax states are merged. With flags = 0 every split owns a fixed key range, so the
 * output is bitwise reproducible run to run and identical for identical sequences in one
 * batch. With VSA_ATTN_DYNAMIC_SPLITS the splits claim key tiles at run time (the ones
 * that start early or stream fast take more), which shortens the call when workgroups
 * start at different times; the output then differs between runs at the level of fp32
 * rounding order, within the same error bound to the exact result. The flag applies to
 * the bf16 path; the fp32 path always uses fixed ranges.
 * ------------------------------------------------------------------------------------ */
#define VSA_ATTN_DYNAMIC_SPLITS 1u

size_t verify_attention_workspace_size(int B, int Hq, int Hkv, int D, int max_rows_per_seq,
                                       int max_kv_len);

vsa_status verify_attention(const void* q, const void* k_cache, const void* v_cache,
                            vsa_dtype dtype, const int32_t* cu_rows, const int32_t* ctx_lens,
                            int B, int total_rows, int Hq, int Hkv, int D, int S_max,
                            int max_rows_per_seq, int max_kv_len, float scale,
                            uint32_t flags, float* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * verify_attention_noalloc
 *
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): verify_attention without a workspace
 * argument. Its partial results and counters live in a static device array of the library,
 * VSA_NOALLOC_SCRATCH_BYTES (16 MiB) on each GPU, present from the library's load until the
 * process ends. The call allocates nothing; its first call on a device looks up that
 * device's copy and enqueues a kernel on `stream` that clears the copy's counters.
 *
 *   device_error  device pointer to a uint32 into which the device error bits are ORed
 *                 (as in the workspace's error word), or NULL to drop them
 *   every other argument as for verify_attention; the stream must belong to the current
 *   device.
 * Returns VSA_ERR_WORKSPACE when verify_attention_workspace_size() of the problem exceeds
 * VSA_NOALLOC_SCRATCH_BYTES. Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (different streams, or different host threads without ordering)
 * race and give undefined results; calls in stream order are safe.
 * ------------------------------------------------------------------------------------ */
#define VSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

vsa_status verify_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    vsa_dtype dtype, const int32_t* cu_rows,
                                    const int32_t* ctx_lens, int B, int total_rows, int Hq,
                                    int Hkv, int D, int S_max, int max_rows_per_seq,
                                    int max_kv_len, float scale, uint32_t flags, float* out,
                                    uint32_t* device_error, void* stream);

/* ------------------------------------------------------------------------------------
 * block_attention
 *
 * The same multi-row attention for a drafter's block over its context (Changelog
 * [0.20.0] "Added": the kernel serves verify widths and a drafter's block; "Changed": the
 * drafter's context K/V sits in one buffer with the block written at its tail, the
 * drafter attends only the last N context rows (0 = all), heads with a trained sliding
 * window keep it; [0.8.1] "Changed": causal-block heads never see later block positions,
 * DeepSpec-native heads are bidirectional in the block). Layout as verify_attention: the
 * block's R_b rows have their K/V at positions ctx_b .. ctx_b + R_b - 1. Row i, at
 * position p = ctx_b + i, attends keys lo .. hi:
 *     lo = 0                         window == 0
 *        = max(0, ctx_b - window)    window > 0 (the last `window` context rows)
 *        = max(0, p - window + 1)    window > 0 and VSA_ATTN_SLIDING_WINDOW
 *     hi = p                         (causal in the block)
 *        = ctx_b + R_b - 1           VSA_ATTN_BIDIRECTIONAL
 * window = 0 with flags 0 is exactly verify_attention.
 *
 *   window     >= 0; VSA_ATTN_SLIDING_WINDOW needs window > 0 (else VSA_ERR_INVALID_ARG)
 *   flags      any of VSA_ATTN_DYNAMIC_SPLITS, VSA_ATTN_BIDIRECTIONAL,
 *              VSA_ATTN_SLIDING_WINDOW (other bits: VSA_ERR_INVALID_ARG)
 *   every other argument as for verify_attention (same workspace size query; a window
 *   only lowers the split count). Keys below lo are not read from HBM beyond the tile
 *   (128 keys; 32 on the fp32 path) that holds the first one any row sees.
 * ------------------------------------------------------------------------------------ */
#define VSA_ATTN_BIDIRECTIONAL 2u
#define VSA_ATTN_SLIDING_WINDOW 4u

vsa_status block_attention(const void* q, const void* k_cache, const void* v_cache,
                           vsa_dtype dtype, const int32_t* cu_rows, const int32_t* ctx_lens,
                           int B, int total_rows, int Hq, int Hkv, int D, int S_max,
                           int max_rows_per_seq, int max_kv_len, float scale, int window,
                           uint32_t flags, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * verify_attention_kvq
 *
 * verify_attention over a quantized K/V cache (Changelog [0.3.0] "Added": KV-cache
 * quantization, --kv-bits 4|8, the target's cache quantized from token 0; [0.13.1]: 8 bits
 * halve and 4 bits quarter the per-token cache). The pages do not give the format; this
 * library reads it as affine quantization in groups of 64 consecutive head dimensions:
 *     value = scale * code + bias,  one (scale, bias) pair of fp16 per group,
 *     code unsigned: 8 bits (0..255) or 4 bits (0..15, two per byte, element 2i in the
 *     low nibble).
 * The result is the definition above applied to those exact values (fp32 accumulation).
 *
 *   q          [total_rows, Hq, D]               bf16
 *   k_codes    [B, Hkv, S_max, D * bits / 8]     uint8   (v_codes the same)
 *   k_sb       [B, Hkv, S_max, D / 64, 2]        fp16 (scale, bias)   (v_sb the same)
 *   bits       8 or 4
 *   every other argument as for verify_attention (same workspace size query)
 * Codes and (scale, bias) of positions >= ctx_b + R_b are never used in the result.
 * ------------------------------------------------------------------------------------ */
vsa_status verify_attention_kvq(const void* q, const uint8_t* k_codes, const void* k_sb,
                                const uint8_t* v_codes, const void* v_sb, int bits,
                                const int32_t* cu_rows, const int32_t* ctx_lens, int B,
                                int total_rows, int Hq, int Hkv, int D, int S_max,
                                int max_rows_per_seq, int max_kv_len, float scale,
                                uint32_t flags, float* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * verify_sample_accept
 *
 * Row i of sequence b (i = 0..K_b, K_b = R_b - 1) holds the target logits that decide the
 * token at absolute position positions[b] + i; draft t (1..K_b) of sequence b is entry
 * cu_rows[b] - b + t - 1 of draft_tokens / draft_logits and proposes that same token for
 * row t - 1. For each sequence, with its parameters:
 *   z_i = (x_i - frequency * c_i) - presence * [c_i > 0]   (fp32, this operation order)
 *         c_i = token_counts[b] + the counts of drafts d_1..d_i
 *   greedy (T == 0): a = length of the longest prefix with d_{t} = argmax z_{t-1} (lowest
 *         id on ties); emit d_1..d_a and argmax z_a.
 *   sampled (T > 0): p_i = softmax(z_i / T) (exp((z - z_max) / T) in fp64 from the fp32
 *         z) truncated to {z >= k-th largest z} (top-k) then to the smallest prefix by z
 *         (descending) whose probability reaches top_p (ties of z kept), and renormalized;
 *         q_t likewise from draft row t (no penalties). For t = 1..K_b draw u
 *         (Philox4x32-10 keyed by seed, counter (0, position, b, 0), words 0 and 1); accept
 *         d_t iff u * q_t(d_t) < p_{t-1}(d_t); at the first rejection emit a draw from
 *         max(0, p_{t-1} - q_t) and stop; if all are accepted emit a draw from p_{K_b}.
 *         Draws are exponential races argmax_j w_j / E_j, E_j = -ln U_j, U_j from words
 *         2 (j & 1) and 2 (j & 1) + 1 of counter (j >> 1, position, b, 1). Every uniform
 *         is a 64-bit one on the open interval: U = (hi 2^32 + lo + 1/2) 2^-64, so no E is
 *         0 or infinite and the draw is an exact sample up to the rounding of the weights.
 *   logprobs: raw log-softmax of x (no penalties, temperature or truncation).
 *
 *   target_logits  [total_rows, V] float32
 *   draft_logits   [total_rows - B, V] float32, or NULL when no sequence is sampled
 *   draft_tokens   [total_rows - B] int32 (may be NULL when total_rows == B)
 *   cu_rows        [B + 1] int32 (as above)
 *   token_counts   [B, V] int32 base completion counts, or NULL (all zero)
 *   params         [B] vsa_row_params (device memory)
 *   positions      [B] int32 absolute position decided by row 0
 *   seed           64-bit Philox key
 *   max_rows_per_seq host bound >= every R_b (at most 32)
 *   max_top_k      host bound >= every top_k in use, and >= 1 when any sampled sequence
 *                  has top_p < 1 without top-k (0 when no sequence truncates); <= 256
 *   max_top_logprobs host bound >= every top_logprobs (<= 32); the width of top_lp_*
 * Outputs (each may be NULL when not wanted, except accepted_len and out_tokens):
 *   accepted_len   [B] int32   accepted drafts a_b
 *   out_tokens     [total_rows] int32   row i < a_b + 1 holds the emitted token, else -1
 *   chosen_logprob [total_rows] float32 raw logprob of the emitted token at that row
 *                  (sequences with logprobs != 0), NaN elsewhere
 *   top_lp_vals    [total_rows, max_top_logprobs] float32 raw top logprobs, best first
 *   top_lp_ids     [total_rows, max_top_logprobs] int32 their ids (ties: lower id first);
 *                  entries past a sequence's top_logprobs are -1 / 0
 *   diag_threshold [total_rows] float32 top-k threshold of each target row of a sampled
 *                  sequence (-inf when top-k is off), NaN for greedy sequences
 *   diag_kept      [total_rows, 2] int32 kept-set sizes after top-k and after top-p of
 *                  each target row of a sampled sequence (0 for greedy sequences)
 * Limits: 1 <= V <= 524288; B <= 4194304, B * ceil(V / 2048) <= 16777215 and
 * 3 * B * max_rows_per_seq <= 16777215 (workgroups of one launch); K_b <= 31; top_k <= 256;
 * at most 256 ids may tie into one top-k kept set (VSA_DEVERR_TIE_OVERFLOW beyond). A nucleus without top-k (top_p < 1 and
 * top_k 0 or >= V) keeps {j : z_j >= z*} over the whole vocabulary, z* found by a
 * weighted selection rather than a sort; it runs in the truncation pipeline, so a call
 * with such a sequence and max_top_k = 0 sets VSA_DEVERR_PARAMS for it (decoded greedily).
 * A call with max_top_k = 0 and max_top_logprobs = 0 runs as one kernel whose workgroups
 * wait for each other (it is launched that way only when they all fit on the device at
 * once); a workgroup that waits longer than VSA_FUSED_WAIT_US microseconds (environment,
 * default 2000) hands its share of the draw to another one and sets
 * VSA_DEVERR_WAIT_TIMEOUT. The outputs stay exact; only the call is slower.
 * ------------------------------------------------------------------------------------ */
size_t verify_sample_accept_workspace_size(int B, int total_rows, int V, int max_rows_per_seq,
                                           int max_top_k, int max_top_logprobs);

vsa_status verify_sample_accept(const float* target_logits, const float* draft_logits,
                                const int32_t* draft_tokens, const int32_t* cu_rows,
                                const int32_t* token_counts, const vsa_row_params* params,
                                const int32_t* positions, uint64_t seed, int B, int total_rows,
                                int V, int max_rows_per_seq, int max_top_k,
                                int max_top_logprobs, int32_t* accepted_len,
                                int32_t* out_tokens, float* chosen_logprob, float* top_lp_vals,
                                int32_t* top_lp_ids, float* diag_threshold, int32_t* diag_kept,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Reduced draft vocabularies (Changelog [0.8.0] "Added": EAGLE-3-style heads score a
 * frequent-token subset of draft_vocab ids and ship an offset table d2t, draft id j
 * standing for target id j + d2t[j]; temperature sampling widens the draft distribution
 * onto the target vocabulary before the accept test, so the residual runs over every
 * target id).
 *
 * draft_vocab_inverse builds, once per drafter, the inverse table the verify call reads:
 *   d2t    [draft_vocab] int32 offsets (device); entries mapping outside [0, V) are
 *          skipped; the map must be one-to-one (if two draft ids share a target id the
 *          higher one is kept)
 *   t2d    [V] int32 output (device, 16-byte aligned): the draft id of each target id,
 *          -1 where none maps. Two kernels on `stream`; nothing is allocated.
 *
 * verify_sample_accept_reduced_draft is verify_sample_accept with
 *   draft_logits  [total_rows - B, draft_vocab] float32 (draft ids), or NULL
 *   draft_vocab   1 <= draft_vocab <= V
 *   t2d           [V] int32 from draft_vocab_inverse (16-byte aligned when V % 4 == 0)
 * and computes exactly what verify_sample_accept computes on the widened draft rows
 * (target id x takes the draft logit of t2d[x], or -inf when t2d[x] = -1). Draft tokens,
 * outputs and every other argument are in target ids as before.
 * ------------------------------------------------------------------------------------ */
vsa_status draft_vocab_inverse(const int32_t* d2t, int draft_vocab, int V, int32_t* t2d,
                               void* stream);

vsa_status verify_sample_accept_reduced_draft(
    const float* target_logits, const float* draft_logits, int draft_vocab, const int32_t* t2d,
    const int32_t* draft_tokens, const int32_t* cu_rows, const int32_t* token_counts,
    const vsa_row_params* params, const int32_t* positions, uint64_t seed, int B,
    int total_rows, int V, int max_rows_per_seq, int max_top_k, int max_top_logprobs,
    int32_t* accepted_len, int32_t* out_tokens, float* chosen_logprob, float* top_lp_vals,
    int32_t* top_lp_ids, float* diag_threshold, int32_t* diag_kept, void* workspace,
    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * verify_sample_accept_onehot
 * verify_sample_accept for one-hot proposals (Changelog [0.2.0] "Added": --mode lookup,
 * prompt-lookup drafts with no draft distribution; temperature > 0 through one-hot-proposal
 * speculative sampling, still an exact target sample): q_t = 1 at d_t and 0 elsewhere
 * (truncation leaves it so). Draft t is accepted iff u < p_{t-1}(d_t); after a rejection
 * the draw is from max(0, p_{t-1} - q_t), i.e. p_{t-1} without d_t. No draft logits are
 * read. Arguments, outputs, workspace size query and limits as verify_sample_accept.
 * ------------------------------------------------------------------------------------ */
vsa_status verify_sample_accept_onehot(
    const float* target_logits, const int32_t* draft_tokens, const int32_t* cu_rows,
    const int32_t* token_counts, const vsa_row_params* params, const int32_t* positions,
    uint64_t seed, int B, int total_rows, int V, int max_rows_per_seq, int max_top_k,
    int max_top_logprobs, int32_t* accepted_len, int32_t* out_tokens, float* chosen_logprob,
    float* top_lp_vals, int32_t* top_lp_ids, float* diag_threshold, int32_t* diag_kept,
    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * small_m_qmm
 *
 * The few-row quantized matmul of the verify forward (Changelog [0.20.0] "Changed": a
 * small-M verify matmul for verify widths up to 16, the weights as the matrix operand
 * shared by every row; [0.12.0] "Changed": 4-bit and 8-bit weights in groups of 64):
 *     y[m][n] = sum_k x[m][k] * (scale[n][k / 64] * code[n][k] + bias[n][k / 64])
 * with fp32 accumulation of exact products (codes and x enter the matrix units exactly).
 *
 *   x          [M, K] bf16 (16-byte aligned)
 *   codes      [N, K * bits / 8] uint8 (16-byte aligned); 4 bits: element 2i in the low
 *              nibble of byte i
 *   sb         [N, K / 64, 2] fp16 (scale, bias)
 *   bits       8 or 4
 *   M, N, K    1 <= M <= 16; K a multiple of 64, at most 16777216; ceil(N / 128) <=
 *              16777215 (else VSA_ERR_UNSUPPORTED)
 *   y          [M, N] float32 (16-byte aligned when N % 4 == 0), fully written
 *   workspace  small_m_qmm_workspace_size(M, N, K) bytes, 256-byte aligned: partial sums
 *              of the input splits (no state kept between calls)
 * The inputs are split over workgroups for parallelism and the partials summed in a fixed
 * order, so the result is bitwise reproducible.
 * ------------------------------------------------------------------------------------ */
size_t small_m_qmm_workspace_size(int M, int N, int K);

vsa_status small_m_qmm(const void* x, const uint8_t* codes, const void* sb, int bits, int M,
                       int N, int K, float* y, void* workspace, size_t workspace_bytes,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
