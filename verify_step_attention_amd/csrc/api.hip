// C-ABI entry points: host-side validation, workspace layout and launches.
#include <math.h>
#include <stdlib.h>

#include <mutex>

#include "vsa_internal.h"

using namespace vsa;

namespace {

constexpr int kMaxRowsPerSeq = kMaxSeqRows;
constexpr int kMaxTopK = kKeep;
constexpr int kMaxTopLogprobs = 32;
constexpr int kMaxVocab = kMaxChunks * kChunk;

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

// Clears counters past the workspace's counter region (calls with that many of them).
hipError_t vsa::launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       p, n);
    return hipGetLastError();
}

extern "C" {

int vsa_version(void) { return 200; }

const char* vsa_status_string(vsa_status status) {
    switch (status) {
        case VSA_OK: return "VSA_OK";
        case VSA_ERR_INVALID_ARG: return "VSA_ERR_INVALID_ARG";
        case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED";
        case VSA_ERR_WORKSPACE: return "VSA_ERR_WORKSPACE";
        case VSA_ERR_LAUNCH: return "VSA_ERR_LAUNCH";
        default: return "VSA_ERR_UNKNOWN";  // any other int a caller passes
    }
}

size_t verify_attention_workspace_size(int B, int Hq, int Hkv, int D, int max_rows_per_seq,
                                       int max_kv_len) {
    if (B < 1 || B > kMaxBatch || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
        (long)B * Hkv > kMaxAttnUnits || (D != 64 && D != 128) || max_rows_per_seq < 1 ||
        max_rows_per_seq > kMaxRowsPerSeq || max_kv_len < 1 ||
        (long)(Hq / Hkv) * max_rows_per_seq > 128)
        return 0;
    return plan_attention(B, Hq, Hkv, D, max_rows_per_seq, max_kv_len).bytes;
}

vsa_status verify_attention(const void* q, const void* k_cache, const void* v_cache,
                            vsa_dtype dtype, const int32_t* cu_rows, const int32_t* ctx_lens,
                            int B, int total_rows, int Hq, int Hkv, int D, int S_max,
                            int max_rows_per_seq, int max_kv_len, float scale,
                            uint32_t flags, float* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (flags & ~VSA_ATTN_DYNAMIC_SPLITS) return VSA_ERR_INVALID_ARG;
    return block_attention(q, k_cache, v_cache, dtype, cu_rows, ctx_lens, B, total_rows, Hq,
                           Hkv, D, S_max, max_rows_per_seq, max_kv_len, scale, 0, flags, out,
                           workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The multi-row attention behind verify_attention, block_attention and
// verify_attention_noalloc. err_word receives the device error bits; NULL means the
// workspace's own error word (byte 0).
vsa_status attention_call(const void* q, const void* k_cache, const void* v_cache,
                          vsa_dtype dtype, const int32_t* cu_rows, const int32_t* ctx_lens,
                          int B, int total_rows, int Hq, int Hkv, int D, int S_max,
                          int max_rows_per_seq, int max_kv_len, float scale, int window,
                          uint32_t flags, float* out, void* workspace, size_t workspace_bytes,
                          uint32_t* err_word, void* stream) {
    if (!q || !k_cache || !v_cache || !cu_rows || !ctx_lens || !out) return VSA_ERR_INVALID_ARG;
    if (flags & ~(VSA_ATTN_DYNAMIC_SPLITS | VSA_ATTN_BIDIRECTIONAL | VSA_ATTN_SLIDING_WINDOW))
        return VSA_ERR_INVALID_ARG;
    if (window < 0 || ((flags & VSA_ATTN_SLIDING_WINDOW) && window == 0))
        return VSA_ERR_INVALID_ARG;
    if (dtype != VSA_F32 && dtype != VSA_BF16) return VSA_ERR_INVALID_ARG;
    if (B < 1 || total_rows < B || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S_max < 1 ||
        max_rows_per_seq < 1 || max_kv_len < 1 || max_kv_len > S_max ||
        (long)total_rows > (long)B * max_rows_per_seq || !(scale >= 0.f) || !isfinite(scale))
        return VSA_ERR_INVALID_ARG;
    if ((D != 64 && D != 128) || max_rows_per_seq > kMaxRowsPerSeq ||
        (long)(Hq / Hkv) * max_rows_per_seq > 128 || B > kMaxBatch ||
        (long)B * Hkv > kMaxAttnUnits)
        return VSA_ERR_UNSUPPORTED;
    // A window bounds the keys of every sequence by window + rows (plus one tile of
    // rounding), so the split count is planned for that; it never exceeds the one the
    // workspace size query plans for max_kv_len.
    int plan_len = max_kv_len;
    if (window > 0 && (long)window + max_rows_per_seq + 128 < (long)max_kv_len)
        plan_len = window + max_rows_per_seq + 128;
    const AttnPlan plan = plan_attention(B, Hq, Hkv, D, max_rows_per_seq, plan_len);
    if (!workspace || !aligned256(workspace) || workspace_bytes < plan.bytes)
        return VSA_ERR_WORKSPACE;

    char* ws = static_cast<char*>(workspace);
    AttnArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.cu_rows = cu_rows;
    a.ctx_lens = ctx_lens;
    a.out = out;
    a.part_o = reinterpret_cast<float*>(ws + plan.off_o);
    a.part_ml = reinterpret_cast<float2*>(ws + plan.off_ml);
    a.tile_ctr = reinterpret_cast<uint32_t*>(ws + kWsCounters);
    a.tile_ctr_x = reinterpret_cast<uint32_t*>(ws + plan.off_ctr_x);
    a.err = err_word ? err_word : reinterpret_cast<uint32_t*>(ws);
    a.batch = B;
    a.total_rows = total_rows;
    a.hq = Hq;
    a.hkv = Hkv;
    a.group = Hq / Hkv;
    a.d = D;
    a.s_max = S_max;
    a.max_rows = max_rows_per_seq;
    a.max_kv_len = max_kv_len;
    a.nsplit = plan.nsplit;
    a.dyn = (flags & VSA_ATTN_DYNAMIC_SPLITS) != 0 && plan.nsplit >= 2 && dtype == VSA_BF16;
    a.units = plan.units;
    a.mcap = plan.mcap;
    a.merge_kernel = plan.merge_kernel;
    const float sc = scale == 0.f ? 1.f / sqrtf((float)D) : scale;
    a.scale_log2 = sc * 1.4426950408889634f;
    a.window = window;
    a.mask = ((flags & VSA_ATTN_BIDIRECTIONAL) ? kMaskBidirectional : 0) |
             ((flags & VSA_ATTN_SLIDING_WINDOW) ? kMaskSliding : 0);
    if (plan.n_ctr_x &&
        launch_zero_u32(a.tile_ctr_x, plan.n_ctr_x, static_cast<hipStream_t>(stream)) != hipSuccess)
        return VSA_ERR_LAUNCH;
    if (launch_attention(a, plan, dtype, static_cast<hipStream_t>(stream)) != hipSuccess)
        return VSA_ERR_LAUNCH;
    return VSA_OK;
}

// Scratch of verify_attention_noalloc: one copy per GPU, zero when the code object loads,
// held until the process ends. Host code never passes `scratch` itself to a kernel (on the
// host it is only a stand-in for the symbol); it uses the per-device address that
// hipGetSymbolAddress returns.
constexpr size_t kNoallocScratchBytes = VSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address, looked up (and its header of error word and
// counters cleared, by a kernel on `stream`) on the first call on that device.
vsa_status device_scratch(hipStream_t stream, char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return VSA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr ||
            !aligned256(ptr))
            return VSA_ERR_LAUNCH;
        if (launch_zero_u32(static_cast<uint32_t*>(ptr), kWsHeader / 4, stream) != hipSuccess)
            return VSA_ERR_LAUNCH;
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<char*>(g_scratch_ptr[dev]);
    return VSA_OK;
}

}  // namespace

extern "C" {

vsa_status block_attention(const void* q, const void* k_cache, const void* v_cache,
                           vsa_dtype dtype, const int32_t* cu_rows, const int32_t* ctx_lens,
                           int B, int total_rows, int Hq, int Hkv, int D, int S_max,
                           int max_rows_per_seq, int max_kv_len, float scale, int window,
                           uint32_t flags, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return attention_call(q, k_cache, v_cache, dtype, cu_rows, ctx_lens, B, total_rows, Hq,
                          Hkv, D, S_max, max_rows_per_seq, max_kv_len, scale, window, flags,
                          out, workspace, workspace_bytes, nullptr, stream);
}

vsa_status verify_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    vsa_dtype dtype, const int32_t* cu_rows,
                                    const int32_t* ctx_lens, int B, int total_rows, int Hq,
                                    int Hkv, int D, int S_max, int max_rows_per_seq,
                                    int max_kv_len, float scale, uint32_t flags, float* out,
                                    uint32_t* device_error, void* stream) {
    if (!q || !k_cache || !v_cache || !cu_rows || !ctx_lens || !out) return VSA_ERR_INVALID_ARG;
    if (flags & ~VSA_ATTN_DYNAMIC_SPLITS) return VSA_ERR_INVALID_ARG;
    const size_t need = verify_attention_workspace_size(B, Hq, Hkv, D, max_rows_per_seq,
                                                        max_kv_len);
    if (need > kNoallocScratchBytes) return VSA_ERR_WORKSPACE;
    if (need == 0) {
        // Not a supported problem: the regular checks name the reason before any set-up.
        return attention_call(q, k_cache, v_cache, dtype, cu_rows, ctx_lens, B, total_rows,
                              Hq, Hkv, D, S_max, max_rows_per_seq, max_kv_len, scale, 0,
                              flags, out, nullptr, 0, device_error, stream);
    }
    char* ws = nullptr;
    const vsa_status st = device_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != VSA_OK) return st;
    return attention_call(q, k_cache, v_cache, dtype, cu_rows, ctx_lens, B, total_rows, Hq,
                          Hkv, D, S_max, max_rows_per_seq, max_kv_len, scale, 0, flags, out,
                          ws, kNoallocScratchBytes, device_error, stream);
}

vsa_status verify_attention_kvq(const void* q, const uint8_t* k_codes, const void* k_sb,
                                const uint8_t* v_codes, const void* v_sb, int bits,
                                const int32_t* cu_rows, const int32_t* ctx_lens, int B,
                                int total_rows, int Hq, int Hkv, int D, int S_max,
                                int max_rows_per_seq, int max_kv_len, float scale,
                                uint32_t flags, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (!q || !k_codes || !k_sb || !v_codes || !v_sb || !cu_rows || !ctx_lens || !out)
        return VSA_ERR_INVALID_ARG;
    if (bits != 8 && bits != 4) return VSA_ERR_INVALID_ARG;
    if (flags & ~VSA_ATTN_DYNAMIC_SPLITS) return VSA_ERR_INVALID_ARG;
    if (B < 1 || total_rows < B || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S_max < 1 ||
        max_rows_per_seq < 1 || max_kv_len < 1 || max_kv_len > S_max ||
        (long)total_rows > (long)B * max_rows_per_seq || !(scale >= 0.f) || !isfinite(scale))
        return VSA_ERR_INVALID_ARG;
    if ((D != 64 && D != 128) || max_rows_per_seq > kMaxRowsPerSeq ||
        (long)(Hq / Hkv) * max_rows_per_seq > 128 || B > kMaxBatch ||
        (long)B * Hkv > kMaxAttnUnits)
        return VSA_ERR_UNSUPPORTED;
    const AttnPlan plan = plan_attention(B, Hq, Hkv, D, max_rows_per_seq, max_kv_len);
    if (!workspace || !aligned256(workspace) || workspace_bytes < plan.bytes)
        return VSA_ERR_WORKSPACE;

    char* ws = static_cast<char*>(workspace);
    AttnArgs a{};
    a.q = q;
    a.k = k_codes;
    a.v = v_codes;
    a.ksb = k_sb;
    a.vsb = v_sb;
    a.bits = bits;
    a.cu_rows = cu_rows;
    a.ctx_lens = ctx_lens;
    a.out = out;
    a.part_o = reinterpret_cast<float*>(ws + plan.off_o);
    a.part_ml = reinterpret_cast<float2*>(ws + plan.off_ml);
    a.tile_ctr = reinterpret_cast<uint32_t*>(ws + kWsCounters);
    a.tile_ctr_x = reinterpret_cast<uint32_t*>(ws + plan.off_ctr_x);
    a.err = reinterpret_cast<uint32_t*>(ws);
    a.batch = B;
    a.total_rows = total_rows;
    a.hq = Hq;
    a.hkv = Hkv;
    a.group = Hq / Hkv;
    a.d = D;
    a.s_max = S_max;
    a.max_rows = max_rows_per_seq;
    a.max_kv_len = max_kv_len;
    a.nsplit = plan.nsplit;
    a.dyn = (flags & VSA_ATTN_DYNAMIC_SPLITS) != 0 && plan.nsplit >= 2;
    a.units = plan.units;
    a.mcap = plan.mcap;
    a.merge_kernel = plan.merge_kernel;
    const float sc = scale == 0.f ? 1.f / sqrtf((float)D) : scale;
    a.scale_log2 = sc * 1.4426950408889634f;
    if (plan.n_ctr_x &&
        launch_zero_u32(a.tile_ctr_x, plan.n_ctr_x, static_cast<hipStream_t>(stream)) != hipSuccess)
        return VSA_ERR_LAUNCH;
    if (launch_attention(a, plan, VSA_BF16, static_cast<hipStream_t>(stream)) != hipSuccess)
        return VSA_ERR_LAUNCH;
    return VSA_OK;
}

}  // extern "C"

namespace {
// The vocabulary stage launches up to B * ceil(V / 2048) workgroups (statistics, draws) and
// B * 3 * max_rows_per_seq (selections); both must fit one dispatch.
bool sample_grids_fit(int B, int V, int max_rows_per_seq) {
    return (long)B * ((V + kChunk - 1) / kChunk) <= kMaxGridWgs &&
           (long)B * 3 * max_rows_per_seq <= kMaxGridWgs;
}
}  // namespace

extern "C" {

size_t verify_sample_accept_workspace_size(int B, int total_rows, int V, int max_rows_per_seq,
                                           int max_top_k, int max_top_logprobs) {
    if (B < 1 || total_rows < B || V < 1 || V > kMaxVocab || max_rows_per_seq < 1 ||
        max_rows_per_seq > kMaxRowsPerSeq || (long)total_rows > (long)B * max_rows_per_seq ||
        B > kMaxBatch || !sample_grids_fit(B, V, max_rows_per_seq) || max_top_k < 0 ||
        max_top_k > kMaxTopK || max_top_logprobs < 0 ||
        max_top_logprobs > kMaxTopLogprobs)
        return 0;
    return plan_sample(B, total_rows, V, max_top_k, max_top_logprobs).bytes;
}

vsa_status verify_sample_accept(const float* target_logits, const float* draft_logits,
                                const int32_t* draft_tokens, const int32_t* cu_rows,
                                const int32_t* token_counts, const vsa_row_params* params,
                                const int32_t* positions, uint64_t seed, int B, int total_rows,
                                int V, int max_rows_per_seq, int max_top_k,
                                int max_top_logprobs, int32_t* accepted_len,
                                int32_t* out_tokens, float* chosen_logprob, float* top_lp_vals,
                                int32_t* top_lp_ids, float* diag_threshold, int32_t* diag_kept,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return verify_sample_accept_reduced_draft(
        target_logits, draft_logits, V, nullptr, draft_tokens, cu_rows, token_counts, params,
        positions, seed, B, total_rows, V, max_rows_per_seq, max_top_k, max_top_logprobs,
        accepted_len, out_tokens, chosen_logprob, top_lp_vals, top_lp_ids, diag_threshold,
        diag_kept, workspace, workspace_bytes, stream);
}

vsa_status draft_vocab_inverse(const int32_t* d2t, int draft_vocab, int V, int32_t* t2d,
                               void* stream) {
    if (!d2t || !t2d || draft_vocab < 1 || V < 1 || draft_vocab > V) return VSA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(t2d) & 15u) != 0) return VSA_ERR_INVALID_ARG;
    if (launch_draft_vocab_inverse(d2t, draft_vocab, V, t2d,
                                   static_cast<hipStream_t>(stream)) != hipSuccess)
        return VSA_ERR_LAUNCH;
    return VSA_OK;
}

}  // extern "C"

namespace {

// How long (microseconds) a fused-kernel workgroup waits for its sequence's statistics
// before it hands its chunk of the draw to the last arriver: VSA_FUSED_WAIT_US, else 2 ms.
// Tests set it to 0 to drive the hand-over path from the host.
uint32_t fused_wait_ticks() {
    const char* e = getenv("VSA_FUSED_WAIT_US");
    long us = 2000;
    if (e && *e) {
        char* end = nullptr;
        const long v = strtol(e, &end, 10);
        if (end && *end == '\0' && v >= 0 && v <= 10000000) us = v;
    }
    return (uint32_t)(us * 100);                  // s_memrealtime runs at 100 MHz
}

vsa_status sample_call(const float* target_logits, const float* draft_logits, int draft_vocab,
                       const int32_t* t2d, bool onehot, const int32_t* draft_tokens,
                       const int32_t* cu_rows, const int32_t* token_counts,
                       const vsa_row_params* params, const int32_t* positions, uint64_t seed,
                       int B, int total_rows, int V, int max_rows_per_seq, int max_top_k,
                       int max_top_logprobs, int32_t* accepted_len, int32_t* out_tokens,
                       float* chosen_logprob, float* top_lp_vals, int32_t* top_lp_ids,
                       float* diag_threshold, int32_t* diag_kept, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (!target_logits || !cu_rows || !params || !positions || !accepted_len || !out_tokens)
        return VSA_ERR_INVALID_ARG;
    if (B < 1 || total_rows < B || V < 1 || max_rows_per_seq < 1 || max_top_k < 0 ||
        max_top_logprobs < 0 || (long)total_rows > (long)B * max_rows_per_seq)
        return VSA_ERR_INVALID_ARG;
    if (total_rows > B && !draft_tokens) return VSA_ERR_INVALID_ARG;
    if (draft_vocab < 1 || draft_vocab > V || (draft_vocab != V && !t2d))
        return VSA_ERR_INVALID_ARG;
    if (t2d && (V % 4) == 0 && (reinterpret_cast<uintptr_t>(t2d) & 15u) != 0)
        return VSA_ERR_INVALID_ARG;
    if (V > kMaxVocab || max_rows_per_seq > kMaxRowsPerSeq || max_top_k > kMaxTopK ||
        max_top_logprobs > kMaxTopLogprobs || B > kMaxBatch ||
        !sample_grids_fit(B, V, max_rows_per_seq))
        return VSA_ERR_UNSUPPORTED;
    const SampPlan plan = plan_sample(B, total_rows, V, max_top_k, max_top_logprobs);
    if (!workspace || !aligned256(workspace) || workspace_bytes < plan.bytes)
        return VSA_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    SampArgs a{};
    a.tl = target_logits;
    a.dl = onehot ? nullptr : draft_logits;
    a.t2d = onehot ? nullptr : t2d;
    a.dvocab = (t2d && !onehot) ? draft_vocab : V;
    a.onehot = onehot ? 1 : 0;
    a.wait_ticks = fused_wait_ticks();
    a.drafts = draft_tokens;
    a.cu_rows = cu_rows;
    a.counts = token_counts;
    a.params = params;
    a.positions = positions;
    a.seed = seed;
    a.batch = B;
    a.total_rows = total_rows;
    a.vocab = V;
    a.max_rows = max_rows_per_seq;
    a.max_top_k = max_top_k;
    a.max_top_lp = max_top_logprobs;
    a.nchunk = plan.nchunk;
    a.capc = plan.capc;
    a.keepcap = plan.keepcap;
    a.accepted = accepted_len;
    a.out_tokens = out_tokens;
    a.chosen_lp = chosen_logprob;
    a.top_vals = top_lp_vals;
    a.top_ids = top_lp_ids;
    a.diag_thr = diag_threshold;
    a.diag_kept = diag_kept;
    a.err = reinterpret_cast<uint32_t*>(ws);
    a.ctr = reinterpret_cast<uint32_t*>(ws + kWsCounters);
    a.ctr_x = reinterpret_cast<uint32_t*>(ws + plan.off_ctr_x);
    a.stats = reinterpret_cast<float4*>(ws + plan.off_stats);
    a.cand = reinterpret_cast<uint2*>(ws + plan.off_cand);
    a.cand_meta = reinterpret_cast<uint2*>(ws + plan.off_meta);
    a.rows = reinterpret_cast<RowInfo*>(ws + plan.off_rows);
    a.keep = reinterpret_cast<KeepEntry*>(ws + plan.off_keep);
    a.race = reinterpret_cast<RaceReq*>(ws + plan.off_race);
    a.race_part = reinterpret_cast<float4*>(ws + plan.off_race_part);
    if (max_top_k > 0) {
        a.nuc_hm = reinterpret_cast<double*>(ws + plan.off_nuc_hm);
        a.nuc_hn = reinterpret_cast<uint32_t*>(ws + plan.off_nuc_hn);
        a.nuc_info = reinterpret_cast<NucInfo*>(ws + plan.off_nuc_info);
    }
    if (plan.n_ctr_x &&
        launch_zero_u32(a.ctr_x, plan.n_ctr_x, static_cast<hipStream_t>(stream)) != hipSuccess)
        return VSA_ERR_LAUNCH;
    if (launch_sample(a, static_cast<hipStream_t>(stream)) != hipSuccess) return VSA_ERR_LAUNCH;
    return VSA_OK;
}

}  // namespace

extern "C" {

vsa_status verify_sample_accept_reduced_draft(
    const float* target_logits, const float* draft_logits, int draft_vocab, const int32_t* t2d,
    const int32_t* draft_tokens, const int32_t* cu_rows, const int32_t* token_counts,
    const vsa_row_params* params, const int32_t* positions, uint64_t seed, int B,
    int total_rows, int V, int max_rows_per_seq, int max_top_k, int max_top_logprobs,
    int32_t* accepted_len, int32_t* out_tokens, float* chosen_logprob, float* top_lp_vals,
    int32_t* top_lp_ids, float* diag_threshold, int32_t* diag_kept, void* workspace,
    size_t workspace_bytes, void* stream) {
    return sample_call(target_logits, draft_logits, draft_vocab, t2d, false, draft_tokens,
                       cu_rows, token_counts, params, positions, seed, B, total_rows, V,
                       max_rows_per_seq, max_top_k, max_top_logprobs, accepted_len, out_tokens,
                       chosen_logprob, top_lp_vals, top_lp_ids, diag_threshold, diag_kept,
                       workspace, workspace_bytes, stream);
}

vsa_status verify_sample_accept_onehot(
    const float* target_logits, const int32_t* draft_tokens, const int32_t* cu_rows,
    const int32_t* token_counts, const vsa_row_params* params, const int32_t* positions,
    uint64_t seed, int B, int total_rows, int V, int max_rows_per_seq, int max_top_k,
    int max_top_logprobs, int32_t* accepted_len, int32_t* out_tokens, float* chosen_logprob,
    float* top_lp_vals, int32_t* top_lp_ids, float* diag_threshold, int32_t* diag_kept,
    void* workspace, size_t workspace_bytes, void* stream) {
    return sample_call(target_logits, nullptr, V, nullptr, true, draft_tokens, cu_rows,
                       token_counts, params, positions, seed, B, total_rows, V,
                       max_rows_per_seq, max_top_k, max_top_logprobs, accepted_len, out_tokens,
                       chosen_logprob, top_lp_vals, top_lp_ids, diag_threshold, diag_kept,
                       workspace, workspace_bytes, stream);
}

size_t small_m_qmm_workspace_size(int M, int N, int K) {
    if (M < 1 || M > 16 || N < 1 || K < 64 || K % 64 != 0 || K > kMaxQmmK) return 0;
    const QmmPlan p = plan_qmm(M, N, K);
    if ((long)p.tiles * p.nsplit > kMaxGridWgs) return 0;
    return p.bytes > 0 ? p.bytes : 256;
}

vsa_status small_m_qmm(const void* x, const uint8_t* codes, const void* sb, int bits, int M,
                       int N, int K, float* y, void* workspace, size_t workspace_bytes,
                       void* stream) {
    if (!x || !codes || !sb || !y) return VSA_ERR_INVALID_ARG;
    if (bits != 8 && bits != 4) return VSA_ERR_INVALID_ARG;
    if (M < 1 || N < 1 || K < 1) return VSA_ERR_INVALID_ARG;
    if (M > 16 || K % 64 != 0 || K > kMaxQmmK) return VSA_ERR_UNSUPPORTED;
    const uintptr_t ax = reinterpret_cast<uintptr_t>(x), ac = reinterpret_cast<uintptr_t>(codes);
    const uintptr_t as = reinterpret_cast<uintptr_t>(sb), ay = reinterpret_cast<uintptr_t>(y);
    if ((ax & 15u) || (ac & 15u) || (as & 3u) || (ay & ((N % 4) == 0 ? 15u : 3u)))
        return VSA_ERR_INVALID_ARG;
    const QmmPlan plan = plan_qmm(M, N, K);
    if ((long)plan.tiles * plan.nsplit > kMaxGridWgs) return VSA_ERR_UNSUPPORTED;
    if (plan.bytes > 0 && (!workspace || !aligned256(workspace) || workspace_bytes < plan.bytes))
        return VSA_ERR_WORKSPACE;
    QmmArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.codes = codes;
    a.sb = sb;
    a.y = y;
    a.part = plan.bytes > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kWsHeader)
                            : nullptr;
    a.M = M;
    a.N = N;
    a.K = K;
    a.bits = bits;
    a.rowbytes = K * bits / 8;
    a.sbrow = K / 64;
    a.nsplit = plan.nsplit;
    a.ksplit = plan.ksplit;
    a.tiles = plan.tiles;
    if (launch_qmm(a, static_cast<hipStream_t>(stream)) != hipSuccess) return VSA_ERR_LAUNCH;
    return VSA_OK;
}

}  // extern "C"
