// Internal declarations shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vsa.h"

namespace vsa {

// ---------------------------------------------------------------- vector types
typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;
// Every workspace starts with the same header: the device error word (byte 0), then from
// byte 256 a region of kCtrLines 256-byte lines of counters that workgroups update
// atomically. Every call returns its counters to zero and no call keeps anything else
// there, so any mix of calls and shapes can share one workspace in stream order. Counter i
// has a line of its own for i < kCtrLines (counters sharing a line serialize each other's
// atomics); beyond that, lines are shared round-robin.
// The last 8 bytes of each line are a 64-bit word of its own (word64_at), so 32-bit
// counters use the first 62 words of each line.
constexpr int kCtrLines = 256;
constexpr int kMaxCounters = kCtrLines * 62;
constexpr size_t kWsCounters = 256;                                // byte offset
constexpr size_t kWsHeader = kWsCounters + (size_t)kCtrLines * 256; // first data byte
__host__ __device__ __forceinline__ size_t ctr_slot(int i) {
    return (size_t)(i % kCtrLines) * 64 + (size_t)(i / kCtrLines);
}
// 64-bit word i (i < kCtrLines: one per line) of the counter region.
__device__ __forceinline__ unsigned long long* word64_at(uint32_t* head, int i) {
    return reinterpret_cast<unsigned long long*>(head + (size_t)(i % kCtrLines) * 64 + 62);
}
// A call that needs more than kMaxCounters counters keeps the rest in its own workspace
// area (`extra`, compact), which a fill kernel clears at the start of the call.
__device__ __forceinline__ uint32_t* counter_at(uint32_t* head, uint32_t* extra, int i) {
    return i < kMaxCounters ? head + ctr_slot(i) : extra + (i - kMaxCounters);
}
inline size_t extra_counters(long n) { return n > kMaxCounters ? (size_t)(n - kMaxCounters) : 0; }

// ---------------------------------------------------------------- small helpers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float -> bf16 bit pattern, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ void set_device_error(uint32_t* err, uint32_t bit) {
    if (err) atomicOr(err, bit);
}

// ---------------------------------------------------------------- wave reductions
// Wave-wide reductions on DPP cross-lane moves (plain VALU ops, no LDS round trip as with
// ds_bpermute): swap neighbours, swap pairs, mirror within 8, mirror within 16 (now every
// lane of each 16-lane row holds the row's result), then row_bcast:15 / row_bcast:31 fold
// the rows into lane 63, which is read back as a wave-uniform value.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v),
                                                      CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
constexpr int kDppSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

__device__ __forceinline__ float readlane63(float x) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f<kDppSwap1>(x, x));
    x = fmaxf(x, dpp_f<kDppSwap2>(x, x));
    x = fmaxf(x, dpp_f<kDppHalfMirror>(x, x));
    x = fmaxf(x, dpp_f<kDppMirror>(x, x));
    x = fmaxf(x, dpp_f<kDppBcast15, 0xA>(x, x));
    x = fmaxf(x, dpp_f<kDppBcast31, 0xC>(x, x));
    return readlane63(x);
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f<kDppSwap1>(0.f, x);
    x += dpp_f<kDppSwap2>(0.f, x);
    x += dpp_f<kDppHalfMirror>(0.f, x);
    x += dpp_f<kDppMirror>(0.f, x);
    x += dpp_f<kDppBcast15, 0xA>(0.f, x);
    x += dpp_f<kDppBcast31, 0xC>(0.f, x);
    return readlane63(x);
}

// (value, id) with the larger value, ties to the lower id; result in every lane
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
    const float ov = dpp_f<CTRL, ROWS>(v, v);
    const int oi = dpp_i<CTRL, ROWS>(i, i);
    const bool take = (ov > v) | ((ov == v) & (oi < i));  // selects, no divergent branch
    v = take ? ov : v;
    i = take ? oi : i;
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_step<kDppSwap1>(v, i);
    argmax_step<kDppSwap2>(v, i);
    argmax_step<kDppHalfMirror>(v, i);
    argmax_step<kDppMirror>(v, i);
    argmax_step<kDppBcast15, 0xA>(v, i);
    argmax_step<kDppBcast31, 0xC>(v, i);
    v = readlane63(v);
    i = __builtin_amdgcn_readlane(i, 63);
}

__device__ __forceinline__ double wave_sum_f64(double x) {
    // 64-bit values move as two 32-bit halves
#define VSA_DPP_F64(CTRL, ROWS)                                                             \
    {                                                                                       \
        const unsigned long long u = __double_as_longlong(x);                              \
        const int lo = __builtin_amdgcn_update_dpp(0, (int)(u & 0xFFFFFFFFull), CTRL, ROWS, \
                                                   0xF, false);                            \
        const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, ROWS, 0xF,       \
                                                   false);                                 \
        x += __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo); \
    }
    VSA_DPP_F64(kDppSwap1, 0xF)
    VSA_DPP_F64(kDppSwap2, 0xF)
    VSA_DPP_F64(kDppHalfMirror, 0xF)
    VSA_DPP_F64(kDppMirror, 0xF)
    VSA_DPP_F64(kDppBcast15, 0xA)
    VSA_DPP_F64(kDppBcast31, 0xC)
#undef VSA_DPP_F64
    const unsigned long long u = __double_as_longlong(x);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(u & 0xFFFFFFFFull), 63);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(u >> 32), 63);
    return __longlong_as_double(((unsigned long long)hi << 32) | lo);
}

// ---------------------------------------------------------------- workgroup hand-off
// Small results pass from many workgroups to the last one to finish without an
// agent-scope fence (on gfx950 that fence writes back and then invalidates the whole XCD
// L2, which costs tens of microseconds when hundreds of workgroups issue it). Instead the
// values themselves are stored with agent-scope atomic stores (global_store ... sc1:
// written through to the device-coherent level), every wave waits for its stores to
// complete (s_waitcnt), and only then is the arrival counter incremented. The last
// arriving workgroup reads the values with agent-scope atomic loads (global_load ... sc1),
// which do not hit stale L1/L2 lines.
__device__ __forceinline__ void handoff_store(float2* p, float2 v) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                       *reinterpret_cast<unsigned long long*>(&v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 handoff_load(const float2* p) {
    unsigned long long u = __hip_atomic_load(
        reinterpret_cast<unsigned long long*>(const_cast<float2*>(p)), __ATOMIC_RELAXED,
        __HIP_MEMORY_SCOPE_AGENT);
    return *reinterpret_cast<float2*>(&u);
}
__device__ __forceinline__ void handoff_store4(float4* p, float4 v) {
    float2* q = reinterpret_cast<float2*>(p);
    handoff_store(q, make_float2(v.x, v.y));
    handoff_store(q + 1, make_float2(v.z, v.w));
}
__device__ __forceinline__ float4 handoff_load4(const float4* p) {
    const float2* q = reinterpret_cast<const float2*>(p);
    const float2 a = handoff_load(q), b = handoff_load(q + 1);
    return make_float4(a.x, a.y, b.x, b.y);
}

// 16-byte hand-off loads and stores through a buffer resource, with the cache policy of
// the agent-scope atomic ones above (sc1): one instruction per float4 instead of two. They
// are not single-copy atomic across the 16 bytes, which a hand-off does not need (the
// values are complete before the counter says so). The resource's byte count bounds every
// access: a load past it returns 0 and a store past it is dropped.
typedef unsigned int vsa_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCpolSc1 = 16;                // cache-policy operand: sc1
constexpr int kRawBufferWord3 = 0x00020000; // raw (untyped) access, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t handoff_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRawBufferWord3);
}
__device__ __forceinline__ float4 handoff_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const vsa_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}
__device__ __forceinline__ void handoff_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
    vsa_u32x4 u;
    u.x = __float_as_uint(v.x);
    u.y = __float_as_uint(v.y);
    u.z = __float_as_uint(v.z);
    u.w = __float_as_uint(v.w);
    __builtin_amdgcn_raw_buffer_store_b128(u, r, off, 0, kCpolSc1);
}

// Every thread's hand-off stores are complete before thread 0 counts the workgroup in;
// returns true (in every thread) in the last of `total` workgroups to arrive, which also
// resets the counter for the next call unless `reset` is false (then whoever else reads
// the count clears it).
__device__ __forceinline__ bool handoff_arrive(uint32_t* counter, uint32_t total,
                                               int* s_flag, bool reset = true) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(counter, 1u);
        const bool last = prev == total - 1;
        if (last && reset)
            __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}

// ---------------------------------------------------------------- attention launch args
struct AttnArgs {
    // what the first tile's DMA and the sequence geometry need, in the first 64 bytes (one
    // scalar cache line of the kernel arguments)
    const void* k;
    const void* v;
    uint32_t* tile_ctr;     // counter region; unit u claims tiles at counter_at(u)
    const int32_t* cu_rows;
    const int32_t* ctx_lens;
    int nsplit, hkv, s_max, max_kv_len;
    int dyn;                // splits claim tiles from tile_ctr (needs nsplit >= 2)
    int max_rows;
    // the rest
    uint32_t* tile_ctr_x;   // tile claim counters past the counter region (or unused)
    const void* ksb;        // quantized caches: (scale, bias) fp16 pairs per 64 dims
    const void* vsb;
    int bits;               // 0: bf16 / fp32 K and V; 8 or 4: quantized codes in k / v
    const void* q;
    float* out;
    float* part_o;          // [units][nsplit][mcap][D]
    float2* part_ml;        // [units][nsplit][mcap]   (running max (log2 units), sum)
    uint32_t* err;
    int batch, total_rows, hq, group, d, units, mcap;
    float scale_log2;       // softmax scale * log2(e)
    int window;             // > 0: context keys seen per row are limited (see mask)
    int mask;               // kMaskBidirectional | kMaskSliding
    int merge_kernel;       // the splits are merged by attn_merge_kernel, not in the kernel
    int slice_merge;        // in-kernel merge split over the unit's splits (all resident)
    uint32_t merge_wait;    // real-time ticks a split waits for its slice of the merge
};
constexpr int kMaskBidirectional = 1;   // block rows see every block row
constexpr int kMaskSliding = 2;         // the window ends at each row's own position

// Host-side plan shared by the size query and the launcher.
struct AttnPlan {
    int nb;          // 32-column blocks of the (row x head) query matrix per KV head
    int mcap;        // 32 * nb
    int nsplit;      // key splits per (sequence, KV head)
    int units;       // B * Hkv
    int tile;        // keys per workgroup tile
    int merge_kernel;  // 1: a separate kernel merges the splits (see plan_attention)
    size_t off_ctr_x, n_ctr_x, off_ml, off_o, bytes;
};

AttnPlan plan_attention(int B, int Hq, int Hkv, int D, int max_rows, int max_kv_len);
hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, vsa_dtype dtype,
                            hipStream_t stream);

// ---------------------------------------------------------------- few-row quantized matmul
struct QmmArgs {
    const uint16_t* x;      // [M, K] bf16
    const uint8_t* codes;   // [N, rowbytes]
    const void* sb;         // [N, sbrow] fp16 (scale, bias) pairs
    float* y;               // [M, N]
    float* part;            // [nsplit, M, N] partials (nsplit > 1)
    int M, N, K, bits, rowbytes, sbrow, nsplit, ksplit, tiles;
};
struct QmmPlan {
    int tiles, nsplit, ksplit;
    size_t bytes;           // workspace (partials), 0 with one split
};
QmmPlan plan_qmm(int M, int N, int K);
hipError_t launch_qmm(const QmmArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- vocabulary stage
constexpr int kChunk = 2048;         // vocabulary ids per workgroup chunk (8 per thread)
constexpr int kMaxBatch = 1 << 22;  // sequences per call
constexpr int kMaxQmmK = 1 << 24;   // inner dimension of small_m_qmm
constexpr long kMaxAttnUnits = 1L << 22;  // (sequence, KV head) pairs per attention call
// Workgroups of 256 threads in one launch: a dispatch's grid size counts work-items in 32 bits.
constexpr long kMaxGridWgs = (1L << 24) - 1;
constexpr int kMaxChunks = 256;      // chunks per row (vocabulary <= kMaxChunks * kChunk)
constexpr int kChunkLoads = kMaxChunks / 64;   // per-lane loads when a wave reads a row's chunks
constexpr int kKeep = 256;           // kept-set capacity of one truncated row
constexpr int kMaxSeqRows = 32;      // verify rows per sequence (K <= 31)

// Merged statistics of one row (finalize results, also handed to the race kernel).
struct RowInfo {
    double z;          // sum of exp((v - m) / T) over the row (softmax normalizer)
    float m;           // max of v over the row
    int argmax;        // greedy argmax (lowest id on ties)
    float theta;       // top-k threshold (value of the k-th largest)
    int kept_k, kept_p;
    // nucleus without top-k: the kept set is {v >= ythr}, with mass zk = sum over it of
    // e^((v - ymax) / T), ymax the row's max of v; ythr = -inf otherwise
    float ythr;
    float ymax;
    int pad;
    double zk;
};

// Nucleus rows without top-k: bins of (vmax - v) / T in steps of 1/16 (the last bin holds
// every lower value), filled by several workgroups per row; the last to finish finds the
// bin where the mass from the top reaches top_p of the row's mass.
constexpr int kNucBins = 512;
struct NucInfo {       // one nucleus row: its crossing bin, for the listing of that bin's ids
    double mass_before;    // mass of the bins above the crossing bin
    double target;         // top_p times the row's mass
    float vmax;            // the row's max of v (the bins' origin)
    int bstar;             // the crossing bin; -1: the row is resolved already
    int cnt_before;        // ids in the bins above it
    int nb;                // ids in it
    int listed;            // ids listed so far by the listing pass (reservations)
    int pad;
};

struct KeepEntry {     // one id of a truncated, renormalized distribution
    int idx;
    int pad;
    double p;
};

struct RaceReq {       // a categorical draw over the whole vocabulary, done by race_kernel
    int kind;          // 0 none, 1 residual max(0, p - q), 2 bonus (p)
    int onehot_d;      // kind 1 with a one-hot proposal: q = 1 at this id, 0 elsewhere; else -1
    int a;             // accepted drafts (the draw decides row a)
    int pos;           // absolute position of the draw
    int logprobs;
    float m_p, m_q, m_x;
    int nucleus;       // p and q are nucleus rows: (ythr, ymax) below, z_p / z_q their kept mass
    double z_p, z_q, z_x;
    float ythr_p, ymax_p, ythr_q, ymax_q;
};

struct SampArgs {
    const float* tl;               // target logits [T, V]
    const float* dl;               // draft logits [T - B, dvocab] or null
    const int32_t* drafts;         // [T - B]
    const int32_t* cu_rows;        // [B + 1]
    const int32_t* counts;         // [B, V] or null
    const vsa_row_params* params;  // [B]
    const int32_t* positions;      // [B]
    uint64_t seed;
    int batch, total_rows, vocab, max_rows, max_top_k, max_top_lp, nchunk, capc, keepcap;
    int32_t* accepted;
    int32_t* out_tokens;
    float* chosen_lp;
    float* top_vals;
    int32_t* top_ids;
    float* diag_thr;
    int32_t* diag_kept;
    uint32_t* err;
    uint32_t* ctr;                 // counter region: sequence b's arrivals at counter_at(4b)
                                   // and counter_at(4b + 1) (see the kernels)
    uint32_t* ctr_x;               // counters past the region (or unused)
    float4* stats;                 // [slots][nchunk] (m, s, best value, best id bits)
    uint2* cand;                   // [slots][nchunk][capc] (ordered key, id)
    uint2* cand_meta;              // [slots][nchunk] (count, k-th key)
    RowInfo* rows;                 // [slots]
    KeepEntry* keep;               // [2T - B][keepcap]
    RaceReq* race;                 // [B]
    float4* race_part;             // [B][nchunk][4] race winners per (chunk, wave)
    // reduced draft vocabulary (after the rest, so the common fields keep their offsets)
    const int32_t* t2d;            // [V] draft id of each target id (-1: none) or null
    int dvocab;                    // draft vocabulary (V unless t2d is given)
    int onehot;                    // the drafts are one-hot proposals (no draft rows)
    uint32_t wait_ticks;           // fused kernel: how long (100 MHz ticks) a workgroup waits
                                   // for its sequence's statistics before it hands its chunk
                                   // of the draw to the last arriver
    int rsplit;                    // sweep: workgroups sharing a (sequence, chunk)'s rows
    // nucleus rows without top-k (null when max_top_k is 0)
    double* nuc_hm;                // [slots][kNucBins] mass per bin (zero between calls)
    uint32_t* nuc_hn;              // [slots][kNucBins] ids per bin (zero between calls)
    NucInfo* nuc_info;             // [slots]
    int nsel;                      // select: workgroups per nucleus row (histogram pass)
    int nfin;                      // finalize: workgroups per sequence (listing pass)
};
// The fused kernel keeps each sequence's counters and race words on lines 4b .. 4b + 3 and
// its claim words on the lines after the first 4B.
constexpr int kFusedMaxBatch = 60;

// Every kernel argument in one round of scalar loads: the compiler otherwise spreads them
// over several dependent round trips ahead of the first memory request.
__device__ __forceinline__ void preload_args(const SampArgs& a) {
    asm volatile("" ::"s"(a.tl), "s"(a.dl), "s"(a.drafts), "s"(a.cu_rows), "s"(a.counts),
                 "s"(a.params), "s"(a.positions), "s"(a.seed), "s"(a.batch),
                 "s"(a.total_rows), "s"(a.vocab), "s"(a.max_rows), "s"(a.max_top_k),
                 "s"(a.max_top_lp), "s"(a.nchunk), "s"(a.capc), "s"(a.keepcap));
    asm volatile("" ::"s"(a.accepted), "s"(a.out_tokens), "s"(a.chosen_lp), "s"(a.top_vals),
                 "s"(a.top_ids), "s"(a.diag_thr), "s"(a.diag_kept), "s"(a.err),
                 "s"(a.ctr), "s"(a.ctr_x), "s"(a.stats), "s"(a.cand),
                 "s"(a.cand_meta), "s"(a.rows), "s"(a.keep), "s"(a.race), "s"(a.race_part),
                 "s"(a.onehot), "s"(a.wait_ticks));
}

struct SampPlan {
    int nchunk, capc, keepcap, slots;
    size_t off_ctr_x, n_ctr_x, off_stats, off_cand, off_meta, off_rows, off_keep,
        off_race, off_race_part, off_nuc_hm, off_nuc_hn, off_nuc_info, bytes;
};

SampPlan plan_sample(int B, int total_rows, int V, int max_top_k, int max_top_lp);
hipError_t launch_sample(const SampArgs& a, hipStream_t stream);
bool fused_fits(const SampArgs& a);
hipError_t launch_fused(const SampArgs& a, hipStream_t stream);
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t stream);
hipError_t launch_draft_vocab_inverse(const int32_t* d2t, int dvocab, int vocab, int32_t* t2d,
                                      hipStream_t stream);

}  // namespace vsa
