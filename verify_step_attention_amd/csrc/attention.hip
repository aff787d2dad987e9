// Split-KV multi-row causal GQA attention for the verify step (gfx950).
//
// One workgroup handles one (sequence b, KV head g, key split). The query matrix of a KV
// head is every verify row of the sequence times every query head of the group
// (M = R_b * G columns, column n = i * G + hh), so each K/V tile staged in LDS is read from
// HBM once and consumed by all rows and heads of the group (mlx-dspark Changelog [0.20.0]
// "Added": the multi-row kernel packs every GQA head x query row of a KV head so each KV
// tile is read once; [0.3.1]: K/V stay at n_kv heads). Splitting the keys and merging the
// partial softmax states afterwards follows the same passage (split over keys + a merge).
//
// bf16 path: QK^T and PV on v_mfma_f32_32x32x16_bf16 in the transposed orientation
//   S^T[32 keys x 32 cols] = K[32 x D] * Q^T[D x 32]       (K from LDS, Q^T in registers)
//   O^T[32 d x 32 cols]   += V^T[32 x 32 keys] * P^T[32 keys x 32 cols]   (P as bf16 hi+lo)
// so every lane owns one column n for all of its accumulators: the online softmax rescale
// is lane-local, and P^T goes from the S^T accumulators straight into the B operand.
// V^T comes out of the row-major LDS tile with ds_read_b64_tr_b16.
// fp32 path: the same tiling and merge with plain FMA arithmetic.
#include "vsa_internal.h"

#include <mutex>

namespace vsa {

namespace {

constexpr float kNegInf = -__builtin_inff();

#ifndef VSA_ATTN_TARGET_WGS
#define VSA_ATTN_TARGET_WGS 256      // workgroups the key split aims for (one per CU)
#endif
constexpr int kThreads = 256;        // threads per workgroup (every kernel here; a constant,
                                     // so loops do not load the size from the dispatch packet)
constexpr int kMaxSplits = 32;       // key splits per (sequence, KV head)
constexpr int kMergeGroup = 8;       // splits whose partials a merge thread loads together
constexpr uint32_t kMergeWaitTicks = 20000;  // 200 us of the 100 MHz real-time clock
constexpr float kLazyLog2 = 8.f;     // online softmax: rescale only past this growth (log2)
#ifndef VSA_ATTN_DMA_CPOL
#define VSA_ATTN_DMA_CPOL 2
#endif
// Cache policy of the K/V tile DMAs: 2 = nt (streaming; each byte is read once per call).
constexpr int kKvPolicy = VSA_ATTN_DMA_CPOL;

// Block index -> (unit, split). Consecutive block ids go to different XCDs (round-robin
// dispatch), so the splits of one unit are spread over the XCDs: the XCDs start their
// workgroups microseconds apart, and splits that start early claim more of the unit's
// tiles (see the tile loop of the bf16 kernel).
__device__ __forceinline__ void map_block(int bid, int nsplit, int* unit, int* split) {
    *unit = bid / nsplit;
    *split = bid % nsplit;
}

// One tile claim of the dynamic schedule: thread 0 reads the result only at the next
// barrier, so the claim's round trip overlaps the tile in flight. atomicInc with the
// largest limit is a plain increment; unlike atomicAdd, the compiler does not rewrite it
// into a wave-wide form that reads the result (and so waits for every earlier load of the
// wave, DMAs included, which complete in issue order) right after issuing it.
__device__ __forceinline__ uint32_t claim_tile(uint32_t* ctr) {
    return atomicInc(ctr, 0xFFFFFFFFu);
}

struct SeqGeom {
    int r0, rows, ctx;
    bool ok;
};

// The raw geometry words of sequence b: cu_rows[b], cu_rows[b + 1], ctx_lens[b].
struct GeomWords {
    int r0, r1, ctx;
};

// Read through the constant address space: scalar loads, whose completion does not wait
// for the vector loads and DMAs issued before them (those complete in issue order). The
// arrays are inputs that no kernel of the call writes.
typedef __attribute__((address_space(4))) const int const_int;

__device__ __forceinline__ GeomWords load_geometry(const AttnArgs& a, int b) {
    const const_int* cu = (const const_int*)a.cu_rows;
    const const_int* cl = (const const_int*)a.ctx_lens;
    return GeomWords{cu[b], cu[b + 1], cl[b]};
}

__device__ __forceinline__ SeqGeom seq_geometry(const AttnArgs& a, GeomWords w, bool report) {
    SeqGeom s;
    s.r0 = w.r0;
    s.rows = w.r1 - w.r0;
    s.ctx = w.ctx;
    bool bad = false;
    if (s.rows > a.max_rows) { s.rows = a.max_rows; bad = true; }
    if (s.ctx < 0) { s.ctx = 0; bad = true; }
    const int kv_cap = a.max_kv_len < a.s_max ? a.max_kv_len : a.s_max;
    if (s.rows > kv_cap) { s.rows = kv_cap; bad = true; }
    if (s.ctx + s.rows > kv_cap) { s.ctx = kv_cap - s.rows; bad = true; }
    // rows must lie inside q / out: a malformed cu_rows skips the sequence
    s.ok = s.rows >= 1 && s.r0 >= 0 && s.r0 + s.rows <= a.total_rows;
    if (!s.ok) bad = true;
    if (bad && report) set_device_error(a.err, VSA_DEVERR_SEQ_SHAPE);
    return s;
}

__device__ __forceinline__ SeqGeom seq_geometry(const AttnArgs& a, int b, bool report) {
    return seq_geometry(a, load_geometry(a, b), report);
}

// Keys a block row sees. Verify: window 0, causal, so row i sees keys 0 .. ctx + i. A
// drafter's block (mlx-dspark Changelog [0.20.0] "Changed": only the last `window` context
// rows, or a trained sliding window; [0.8.1] "Changed": causal or bidirectional in the
// block): row i at position p = ctx + i sees keys key_lo .. key_hi,
//   key_lo = 0 | max(0, ctx - window) | max(0, p - window + 1) (sliding),
//   key_hi = p | ctx + rows - 1 (bidirectional).
__device__ __forceinline__ int key_lo(const AttnArgs& a, const SeqGeom& s, int i) {
    if (a.window <= 0) return 0;
    const int lo = (a.mask & kMaskSliding) ? s.ctx + i - a.window + 1 : s.ctx - a.window;
    return lo > 0 ? lo : 0;
}
__device__ __forceinline__ int key_hi(const AttnArgs& a, const SeqGeom& s, int i) {
    return (a.mask & kMaskBidirectional) ? s.ctx + s.rows - 1 : s.ctx + i;
}

// Workgroup statistics of the epilogue, in LDS: kStatCap floats each of
//   gm[KGX][MC] key-group running max (log2 units) | gl[KGX][MC] key-group sum
//   | fac[KGX][MC] factor 2^(m_kg - m_wg) | wm[MC] workgroup max | wl[MC] workgroup sum
constexpr int kStatCap = 128;
constexpr int kStatFloats = 5 * kStatCap;

// Four LDS regions, picked by a runtime index (an array of LDS pointers would become a
// static initializer, which the target does not support).
struct LdsQuad {
    float* p0;
    float* p1;
    float* p2;
    float* p3;
    __device__ __forceinline__ float* operator[](int i) const {
        return i == 0 ? p0 : i == 1 ? p1 : i == 2 ? p2 : p3;
    }
};

// Merges output float4s [e_begin, e_end) of the unit (of M * D/4). Thread tasks: float4s
// e, e + 256, ... (TPT of them; column e / (D/4), consecutive lanes on consecutive
// float4s); the loads of all TPT tasks and up to kMergeGroup splits are in flight together
// (a task past the range loads in bounds and is dropped, so TPT fits the range).
template <int D, int TPT>
__device__ void attn_merge_range(const AttnArgs& a, int unit, int g, const SeqGeom& s,
                                 int e_begin, int e_end) {
    constexpr int D4 = D / 4;
    constexpr int SG = kMergeGroup;
    const int ntask = e_end;
    const int ns = a.nsplit;
    const size_t base = (size_t)unit * ns;
    const uint32_t sstride = (uint32_t)a.mcap * D4;          // float4s between splits
    const float2* pml = a.part_ml + base * a.mcap;
    // the unit's partial outputs (ns * mcap * D floats; a few MB at most)
    const __amdgpu_buffer_rsrc_t po =
        handoff_rsrc(a.part_o + base * a.mcap * D, (uint32_t)ns * sstride * 16u);
    for (int e0 = e_begin + (int)threadIdx.x; e0 < ntask; e0 += TPT * kThreads) {
        float m_run[TPT], l_run[TPT];
        float4 acc[TPT];
#pragma unroll
        for (int t = 0; t < TPT; ++t) {
            m_run[t] = kNegInf;
            l_run[t] = 0.f;
            acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int s0 = 0; s0 < ns; s0 += SG) {
            float2 ml[TPT][SG];
            float4 v[TPT][SG];
#pragma unroll
            for (int t = 0; t < TPT; ++t) {
                int e = e0 + t * kThreads;
                e = e < ntask ? e : ntask - 1;                   // in bounds; dropped below
#pragma unroll
                for (int u = 0; u < SG; ++u) {
                    const int sp = s0 + u < ns ? s0 + u : ns - 1;
                    ml[t][u] = handoff_load(pml + (size_t)sp * a.mcap + e / D4);
                }
            }
#pragma unroll
            for (int t = 0; t < TPT; ++t) {
                int e = e0 + t * kThreads;
                e = e < ntask ? e : ntask - 1;
#pragma unroll
                for (int u = 0; u < SG; ++u) {
                    const int sp = s0 + u < ns ? s0 + u : ns - 1;
                    v[t][u] = handoff_load16(po, ((uint32_t)sp * sstride + (uint32_t)e) * 16u);
                }
            }
#pragma unroll
            for (int t = 0; t < TPT; ++t) {
                float m = m_run[t];
#pragma unroll
                for (int u = 0; u < SG; ++u)
                    if (s0 + u < ns) m = fmaxf(m, ml[t][u].x);
                if (m == kNegInf) continue;
                const float c = exp2f(m_run[t] - m);             // m_run = -inf gives 0
                l_run[t] *= c;
                acc[t] = make_float4(acc[t].x * c, acc[t].y * c, acc[t].z * c, acc[t].w * c);
#pragma unroll
                for (int u = 0; u < SG; ++u) {
                    const float f =
                        (s0 + u < ns && ml[t][u].x != kNegInf) ? exp2f(ml[t][u].x - m) : 0.f;
                    l_run[t] += f * ml[t][u].y;
                    acc[t].x += f * v[t][u].x;
                    acc[t].y += f * v[t][u].y;
                    acc[t].z += f * v[t][u].z;
                    acc[t].w += f * v[t][u].w;
                }
                m_run[t] = m;
            }
        }
#pragma unroll
        for (int t = 0; t < TPT; ++t) {
            const int e = e0 + t * kThreads;
            if (e >= ntask) break;
            const int n = e / D4, d4 = e % D4;
            const float il = 1.f / l_run[t];
            const int row = s.r0 + n / a.group, head = g * a.group + n % a.group;
            *(reinterpret_cast<float4*>(a.out + ((size_t)row * a.hq + head) * D) + d4) =
                make_float4(acc[t].x * il, acc[t].y * il, acc[t].z * il, acc[t].w * il);
        }
    }
}

// Arrival of a split, and the merge of the unit's splits once all have arrived. Each split
// has stored its partial state (O relative to the split's max, unnormalized; max in log2
// units; sum) with the hand-off stores (written through to the device-coherent level);
//   out = sum_s w_s O_s,   w_s = 2^(m_s - m) / sum_s' 2^(m_s' - m) l_s',   m = max_s m_s.
// Sliced (a.slice_merge: every split of the grid is resident at once): the split that
// arrives r-th merges the r-th of nsplit slices of the output. The last to arrive merges
// its slice at once and hands every other slice to its owner through the owner's slot
// (0 -> 1, go); an owner waits for the go (bounded), merges and returns the slot to 0. An
// owner that times out marks its slot abandoned (0 -> 2, by compare-and-swap, so exactly
// one of the two wins) and the last arriver merges that slice too. Otherwise the last to
// arrive merges all of it. The unit's tile-claim and arrival counters return to zero; a
// unit whose geometry is invalid (merge = false) only counts in.
template <int D>
__device__ void attn_finish_unit(const AttnArgs& a, int unit, int g, const SeqGeom& s,
                                 bool merge) {
    constexpr int D4 = D / 4;
    __shared__ int s_rank, s_go;
    __shared__ uint32_t s_slot[kMaxSplits];
    const int ns = a.nsplit;
    uint32_t* const arrive = counter_at(a.tile_ctr, a.tile_ctr_x, a.units + unit);
    __builtin_amdgcn_s_waitcnt(0);                     // this workgroup's stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(arrive, 1u);
        if (prev == (uint32_t)ns - 1u) {
            __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (a.dyn)
                __hip_atomic_store(counter_at(a.tile_ctr, a.tile_ctr_x, unit), 0u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        s_rank = (int)prev;
    }
    __syncthreads();
    const int rank = s_rank;
    const bool last = rank == ns - 1;
    if (!merge) return;
    const int ntask = s.rows * a.group * D4;
    if (!a.slice_merge) {
        if (last) attn_merge_range<D, 3>(a, unit, g, s, 0, ntask);
        return;
    }
    // one slice: up to kThreads float4s a pass
    auto merge_slice = [&](int lo, int hi) __attribute__((always_inline)) {
        if (hi - lo <= kThreads) attn_merge_range<D, 1>(a, unit, g, s, lo, hi);
        else attn_merge_range<D, 3>(a, unit, g, s, lo, hi);
    };
    auto slot = [&](int r) __attribute__((always_inline)) {
        return counter_at(a.tile_ctr, a.tile_ctr_x, 2 * a.units + unit * ns + r);
    };
    auto slice_lo = [&](int r) __attribute__((always_inline)) {
        return (int)((uint32_t)(r * ntask) / (uint32_t)ns);
    };
    if (!last) {
        if (threadIdx.x == 0) {
            uint32_t* const sl = slot(rank);
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            uint32_t v;
            for (;;) {
                v = __hip_atomic_load(sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v == 1u) break;
                if (__builtin_amdgcn_s_memrealtime() - t0 >= (uint64_t)a.merge_wait) {
                    // give the slice up, unless the go came in the meantime
                    v = atomicCAS(sl, 0u, 2u);
                    if (v == 0u) v = 2u;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            s_go = (int)v;
        }
        __syncthreads();
        if (s_go != 1) return;                         // abandoned to the last arriver
        merge_slice(slice_lo(rank), slice_lo(rank + 1));
        if (threadIdx.x == 0)
            __hip_atomic_store(slot(rank), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    // the last arriver: every other slice's go, then its own slice, then any abandoned one
    if (threadIdx.x < ns - 1) s_slot[threadIdx.x] = atomicCAS(slot(threadIdx.x), 0u, 1u);
    merge_slice(slice_lo(ns - 1), ntask);
    __syncthreads();
    for (int r = 0; r < ns - 1; ++r) {
        if (s_slot[r] != 2u) continue;
        merge_slice(slice_lo(r), slice_lo(r + 1));
        if (threadIdx.x == 0)
            __hip_atomic_store(slot(r), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Combines the key groups of one workgroup and writes either the final output (single
// split) or this split's partial state (O relative to the split's max, unnormalized; max in
// log2 units; sum), which the unit's last split to finish merges (attn_finish_unit). The
// O of key group k (relative to its own max) for columns 32 j .. 32 j + 31 is at
// ob[k * NBX + j], rows OS floats apart.
template <int D, int KGX, int NBX>
__device__ void attn_epilogue(const AttnArgs& a, LdsQuad ob, float* st, int unit, int split,
                              int g, const SeqGeom& s, int OS) {
    const int tid = threadIdx.x;
    const int M = s.rows * a.group;
    const int MC = a.mcap;
    float* gm = st;
    float* gl = st + kStatCap;
    float* fac = st + 2 * kStatCap;
    float* wm = st + 3 * kStatCap;
    float* wl = st + 4 * kStatCap;

    for (int n = tid; n < M; n += kThreads) {
        float m = kNegInf;
        for (int k = 0; k < KGX; ++k) m = fmaxf(m, gm[k * MC + n]);
        float l = 0.f;
        for (int k = 0; k < KGX; ++k) {
            const float mk = gm[k * MC + n];
            const float f = (mk == kNegInf) ? 0.f : exp2f(mk - m);
            fac[k * MC + n] = f;
            l += f * gl[k * MC + n];
        }
        wm[n] = m;
        wl[n] = l;
    }
    __syncthreads();

    const size_t pslot = (size_t)unit * a.nsplit + split;
    // this split's partial output (mcap * D floats)
    const __amdgpu_buffer_rsrc_t po =
        handoff_rsrc(a.part_o + pslot * a.mcap * D, (uint32_t)(MC * D * 4));
    // at most 32 NBX rows of D / 4 float4s; with one column block (at most four passes)
    // every pass is unrolled, so their LDS reads overlap (more passes would spill)
    constexpr int kPasses = (32 * NBX * (D / 4) + kThreads - 1) / kThreads;
    constexpr int kUnroll = NBX == 1 ? kPasses : 1;
#pragma unroll kUnroll
    for (int pass = 0; pass < kPasses; ++pass) {
        const int e = tid + pass * kThreads;
        if (e >= M * (D / 4)) continue;
        const int n = e / (D / 4), d = 4 * (e % (D / 4));
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < KGX; ++k) {
            const float f = fac[k * MC + n];
            const float4 v = *reinterpret_cast<const float4*>(ob[k * NBX + (n >> 5)] +
                                                              (n & 31) * OS + d);
            o.x += f * v.x;
            o.y += f * v.y;
            o.z += f * v.z;
            o.w += f * v.w;
        }
        if (a.nsplit == 1) {
            const float il = 1.f / wl[n];
            const int row = s.r0 + n / a.group, head = g * a.group + n % a.group;
            *reinterpret_cast<float4*>(a.out + ((size_t)row * a.hq + head) * D + d) =
                make_float4(o.x * il, o.y * il, o.z * il, o.w * il);
        } else if (a.merge_kernel) {
            *reinterpret_cast<float4*>(a.part_o + (pslot * a.mcap + n) * D + d) = o;
        } else {
            handoff_store16(po, (uint32_t)(n * D + d) * 4u, o);
        }
    }
    if (a.nsplit == 1) return;
    if (a.merge_kernel) {
        for (int n = tid; n < M; n += kThreads)
            a.part_ml[pslot * a.mcap + n] = make_float2(wm[n], wl[n]);
        return;
    }
    for (int n = tid; n < M; n += kThreads)
        handoff_store(a.part_ml + pslot * a.mcap + n, make_float2(wm[n], wl[n]));
    attn_finish_unit<D>(a, unit, g, s, true);
}

// A split that owns no tile publishes an empty state (m = -inf, l = 0, O = 0), which
// adds nothing in the merge.
template <int D>
__device__ void attn_empty_split(const AttnArgs& a, int unit, int split, int g,
                                 const SeqGeom& s) {
    const int M = s.rows * a.group;
    const size_t pslot = (size_t)unit * a.nsplit + split;
    const __amdgpu_buffer_rsrc_t po =
        handoff_rsrc(a.part_o + pslot * a.mcap * D, (uint32_t)(a.mcap * D * 4));
    for (int e = threadIdx.x; e < M * (D / 4); e += kThreads)
        handoff_store16(po, (uint32_t)e * 16u, make_float4(0.f, 0.f, 0.f, 0.f));
    for (int n = threadIdx.x; n < M; n += kThreads)
        handoff_store(a.part_ml + pslot * a.mcap + n, make_float2(kNegInf, 0.f));
    if (!a.merge_kernel) attn_finish_unit<D>(a, unit, g, s, true);
}

// -------------------------------------------------------------------------- bf16 / MFMA
// K/V tiles of TK keys go straight from HBM into LDS (global_load_lds_dwordx4: lane l of a
// wave writes bytes [16 l, 16 l + 16) of the wave's 1 KB destination block), two buffers
// deep: while the waves compute on one tile, the next one is in flight. Rows are stored
// unpadded, so the 16-byte chunks of row r are permuted (chunk c at position c ^ swz(r))
// to keep both LDS read patterns free of bank conflicts:
//   QK^T A operand: 16 lanes read one chunk of 16 consecutive rows  -> swz bijective on
//                   16 consecutive rows;
//   V^T (ds_read_b64_tr_b16): 32 lanes read 4 chunks of 4 consecutive rows -> the 4 rows
//                   map the 4 chunks to different 64-byte blocks of the bank space.
// A row of D = 128 bf16 is 256 bytes (all 64 banks); D = 64 packs two rows per bank span.
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// WIN: the call has a window or a bidirectional block (block_attention); without it the
// kernel is compiled for window 0, causal (verify) and carries none of the extra bounds.
template <int D, int NB, bool WIN>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(const AttnArgs a) {
    constexpr int TK = 128;                  // keys per tile
    constexpr int ROWB = D * 2;              // LDS bytes per key row
    constexpr int CH = ROWB / 16;            // 16-byte chunks per row
    constexpr int RPI = 1024 / ROWB;         // rows per 1 KB wave DMA block
    constexpr int BLOCKS = TK * ROWB / 1024; // DMA blocks per matrix tile
    constexpr int BPW = BLOCKS / 4;          // ... per wave
    constexpr int TILEB = TK * ROWB;         // bytes of one matrix tile
    constexpr int KSTEPS = D / 16;           // k-steps of QK^T
    constexpr int DB = D / 32;               // 32-wide d blocks of PV
    constexpr int KG = 4 / NB;               // key groups (waves sharing a column block)
    constexpr int OS = D + 4;                // epilogue row stride (floats)
    static_assert(32 * OS * 4 <= TILEB, "a wave's O fits in one tile buffer");
    static_assert(BLOCKS % 4 == 0, "whole DMA blocks per wave");
    // Two tile buffers (K, V each) as four distinct LDS objects: the compiler then knows
    // that the DMA into one buffer does not alias the reads of the other and does not wait
    // for it before computing.
    __shared__ __attribute__((aligned(1024))) char k0s[TILEB];
    __shared__ __attribute__((aligned(1024))) char v0s[TILEB];
    __shared__ __attribute__((aligned(1024))) char k1s[TILEB];
    __shared__ __attribute__((aligned(1024))) char v1s[TILEB];
    // tail: the last L mod TK keys of a sequence, <= 32 per split (see below)
    constexpr int TAILB = 32 * ROWB;
    constexpr int TPW = TAILB / 1024 / 4 > 0 ? TAILB / 1024 / 4 : 1;   // tail blocks per wave
    __shared__ __attribute__((aligned(1024))) char kts[TAILB];
    __shared__ __attribute__((aligned(1024))) char vts[TAILB];
    __shared__ float stats[kStatFloats];

    // every kernel argument in one round of scalar loads (the compiler would otherwise
    // spread them over several dependent round trips before the first DMA)
    asm volatile("" ::"s"(a.k), "s"(a.v), "s"(a.tile_ctr), "s"(a.cu_rows), "s"(a.ctx_lens),
                 "s"(a.nsplit), "s"(a.hkv), "s"(a.s_max), "s"(a.max_kv_len), "s"(a.dyn),
                 "s"(a.max_rows), "s"(a.q), "s"(a.out), "s"(a.part_o), "s"(a.part_ml),
                 "s"(a.err), "s"(a.total_rows), "s"(a.group), "s"(a.mcap), "s"(a.scale_log2),
                 "s"(a.window), "s"(a.mask));
    int unit, split;
    map_block(blockIdx.x, a.nsplit, &unit, &split);    // the grid is units x nsplit
    const int b = unit / a.hkv, g = unit % a.hkv;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const size_t kv_off = ((size_t)b * a.hkv + g) * (size_t)a.s_max * D;
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + kv_off;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + kv_off;
    // The geometry words go out before the first tile's DMA: vector loads complete in
    // issue order, so issued after it they would wait for the whole tile.
    const GeomWords geo = load_geometry(a, b);

    // DMA of tile t: wave w fills blocks w, w + 4, ... of K and of V (so a wave only ever
    // waits for its own blocks). Keys at or past key_lim read key key_lim - 1.
    const int dma_ri = lane / CH, dma_pos = lane % CH;
    // the permutation of a row depends only on its index mod 16, which for the rows this
    // lane fills (blocks wave, wave + 4, ...) is the same in every block
    const int dma_off = dma_ri * ROWB + ((dma_pos ^ kv_swz<D>(wave * RPI + dma_ri)) << 4);
    int key_lim;
    auto issue_tile = [&](int t, char* kt, char* vt) __attribute__((always_inline)) {
        if ((t + 1) * TK <= key_lim) {
            // whole tile inside the sequence: uniform base + the lane's fixed offset
            const char* kb = reinterpret_cast<const char*>(kbase) + (size_t)t * TILEB;
            const char* vb = reinterpret_cast<const char*>(vbase) + (size_t)t * TILEB;
#pragma unroll
            for (int i = 0; i < BPW; ++i) {
                const int blk = i * 4 + wave;
                __builtin_amdgcn_global_load_lds(kb + blk * 1024 + dma_off,
                                                 (lds_void*)(kt + blk * 1024), 16, 0, kKvPolicy);
                __builtin_amdgcn_global_load_lds(vb + blk * 1024 + dma_off,
                                                 (lds_void*)(vt + blk * 1024), 16, 0, kKvPolicy);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int blk = i * 4 + wave;
            const int r = blk * RPI + dma_ri;
            int key = t * TK + r;
            key = key < key_lim ? key : key_lim - 1;
            const size_t src = (size_t)key * D + (size_t)((dma_pos ^ kv_swz<D>(r)) * 8);
            __builtin_amdgcn_global_load_lds(kbase + src, (lds_void*)(kt + blk * 1024), 16, 0, kKvPolicy);
            __builtin_amdgcn_global_load_lds(vbase + src, (lds_void*)(vt + blk * 1024), 16, 0, kKvPolicy);
        }
    };
    // Tiles. With >= 4 splits the streamed tiles are the F = L / TK full ones, and the last
    // L mod TK keys form a tail spread so that each split gets <= 32 of them (prefetched
    // into a small buffer and computed alongside its first tile); with fewer splits the
    // tiles are ceil(L / TK), the last one partial, and there is no tail.
    // Static schedule: split s streams tiles [nt s / n, nt (s + 1) / n) in order, so the
    // result does not depend on timing. Dynamic schedule (a.dyn): split s streams tile s
    // first, and every later tile is claimed from the unit's counter (tile nsplit + the
    // counter's old value), one claim ahead of the DMA, so splits that start early or
    // stream fast take more tiles and the splits of a unit end together; the partial states
    // then cover timing-dependent tile sets and the merged output varies in rounding only.
    const bool tails = a.nsplit >= 4;
    const bool dyn = a.dyn != 0;
    auto tile_count = [&](int len) __attribute__((always_inline)) {
        return tails ? len / TK : (len + TK - 1) / TK;
    };
    auto static_end = [&](int nt) __attribute__((always_inline)) {
        return (int)((uint32_t)((split + 1) * nt) / (uint32_t)a.nsplit);
    };
    auto first_tile = [&](int nt) __attribute__((always_inline)) {
        const int t = dyn ? split : (int)((uint32_t)(split * nt) / (uint32_t)a.nsplit);
        return t < (dyn ? nt : static_end(nt)) ? t : -1;
    };
    // The first tile is requested before the sequence geometry arrives, as if the sequence
    // held all kv_cap keys (the split's first tile is then the same whenever the sequence
    // spans as many tiles as kv_cap, and always in the dynamic schedule). Rows past the
    // true end are fixed up below.
    const int kv_cap = a.max_kv_len < a.s_max ? a.max_kv_len : a.s_max;
    const int t_spec = first_tile(tile_count(kv_cap));
    key_lim = kv_cap;
    if (t_spec >= 0) issue_tile(t_spec, k0s, v0s);
    uint32_t* const ctr = counter_at(a.tile_ctr, a.tile_ctr_x, unit);
    // thread 0: the pending claim. Left undefined in the other threads (which never read
    // it): a constant there would be a second write to the register the atomic returns
    // into, and the compiler would wait for the atomic (queued behind the DMA) at once.
    uint32_t claim;
    if (dyn && tid == 0) claim = claim_tile(ctr);
    __shared__ int s_next[2];

    const SeqGeom s = seq_geometry(a, geo, tid == 0 && split == 0 && g == 0);
    if (!s.ok) {
        __builtin_amdgcn_s_waitcnt(0);                 // no DMA outlives the workgroup
        if (a.nsplit > 1 && !a.merge_kernel) attn_finish_unit<D>(a, unit, g, s, false);
        return;
    }
    const int L = s.ctx + s.rows;                      // keys of this sequence
    // Streamed keys: from the first key any row sees, rounded down to a tile (key tile t0),
    // to L; schedule tile t is key tile t0 + t.
    const int lo_first = WIN ? key_lo(a, s, 0) : 0;
    const int lo_all = WIN ? key_lo(a, s, s.rows - 1) : 0;
    const int hi_all = WIN ? key_hi(a, s, 0) : s.ctx;  // every row sees lo_all .. hi_all
    const int t0 = lo_first / TK;
    const int nt = tile_count(L - t0 * TK);
    const int t_first = first_tile(nt);
    const int t_last = dyn ? nt : static_end(nt);      // tiles below this one are streamed
    int tail_b = 0, tail_e = 0;
    if (tails) {
        const int f = t0 * TK + (L - t0 * TK) / TK * TK, rem = L - f;
        tail_b = f + (int)((uint32_t)(split * rem) / (uint32_t)a.nsplit);
        tail_e = f + (int)((uint32_t)((split + 1) * rem) / (uint32_t)a.nsplit);
    }
    key_lim = L;
    // a split without a first tile has no tile at all (dynamic: nsplit + c > split >= nt)
    if (t_first < 0 && tail_b >= tail_e) {
        __builtin_amdgcn_s_waitcnt(0);                 // no DMA outlives the workgroup
        attn_empty_split<D>(a, unit, split, g, s);
        return;
    }
    if (t_first >= 0 && (t0 != 0 || t_first != t_spec)) {
        __builtin_amdgcn_s_waitcnt(0);                 // this wave's blocks are free again
        issue_tile(t0 + t_first, k0s, v0s);
    } else if (t_first >= 0 && (t_first + 1) * TK > L) {
        // the speculative tile runs past the sequence end: rows from L on may hold
        // anything, and a V row is multiplied by P = 0, so those rows become zeros
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int r0 = L - t_first * TK;
        for (int e = r0 * CH + tid; e < TK * CH; e += kThreads)
            *reinterpret_cast<uint4*>(v0s + (size_t)e * 16) = make_uint4(0, 0, 0, 0);
    }

    if (tail_b < tail_e) {
        // rows past the tail end read its last key (finite data, masked)
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int blk = i * 4 + wave;
            if (blk * 1024 >= TAILB) break;
            const int r = blk * RPI + dma_ri;
            int key = tail_b + r;
            key = key < tail_e ? key : tail_e - 1;
            const size_t src = (size_t)key * D + (size_t)((dma_pos ^ kv_swz<D>(r)) * 8);
            __builtin_amdgcn_global_load_lds(kbase + src, (lds_void*)(kts + blk * 1024), 16, 0, kKvPolicy);
            __builtin_amdgcn_global_load_lds(vbase + src, (lds_void*)(vts + blk * 1024), 16, 0, kKvPolicy);
        }
    }
    // Keys below the first one any row sees (a window) may share its tile; a V row is
    // multiplied by P = 0 there, so those rows become zeros whatever they hold.
    const bool tail_low = tail_b < tail_e && tail_b < lo_first;
    if (WIN && lo_first > t0 * TK && (t_first == 0 || tail_low)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t_first == 0)
            for (int e = tid; e < (lo_first - t0 * TK) * CH; e += kThreads)
                *reinterpret_cast<uint4*>(v0s + (size_t)e * 16) = make_uint4(0, 0, 0, 0);
        if (tail_low)
            for (int e = tid; e < (lo_first - tail_b) * CH && e < 32 * CH; e += kThreads)
                *reinterpret_cast<uint4*>(vts + (size_t)e * 16) = make_uint4(0, 0, 0, 0);
    }

    const int nb = wave % NB, kg = wave / NB;
    const int h = lane >> 5, col = lane & 31;
    const int n = nb * 32 + col;
    const int M = s.rows * a.group;
    const bool col_valid = n < M;
    const int ri = col_valid ? n / a.group : 0;
    const int hh = col_valid ? n % a.group : 0;
    const int lo_c = WIN ? key_lo(a, s, ri) : 0;                  // this column's keys
    const int hi_c = WIN ? key_hi(a, s, ri) : s.ctx + ri;

    // Q^T fragment (B operand): lane holds column n, dims 16*kk + 8*h .. +8
    bf16x8 qf[KSTEPS];
    {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                             ((size_t)(s.r0 + ri) * a.hq + g * a.group + hh) * D;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            if (col_valid)
                qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk + 8 * h);
            else
                qf[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;
    const int i16 = lane & 15;
    const int half = (lane >> 4) & 1;

    // One 32-key sub-tile: buffer rows kl0 .. kl0 + 31 hold keys kbase0 + row; keys at or
    // past khi are masked.
    auto compute_sub = [&](const char* ktile, const char* vtile, int kl0, int kbase0,
                           int khi) __attribute__((always_inline)) {
        {
            // ---- S^T = K Q^T  (A operand: row kl0 + col, chunk 2 kk + h)
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
            {
                const int krow = kl0 + col;
                const int ksw = kv_swz<D>(krow);
                const char* kr = ktile + krow * ROWB;
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk) {
                    const bf16x8 ka =
                        *reinterpret_cast<const bf16x8*>(kr + (((2 * kk + h) ^ ksw) << 4));
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], sacc, 0, 0, 0);
                }
            }
            // ---- mask + online softmax (lane owns column n; keys 8(r/4)+4h+r%4). A
            // sub-tile whose keys every row sees needs no mask.
            float sv[16];
            float mt = kNegInf;
            if ((!WIN || kbase0 + kl0 >= lo_all) && kbase0 + kl0 + 31 <= hi_all &&
                kbase0 + kl0 + 31 < khi) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sv[r] = sacc[r] * a.scale_log2;
                    mt = fmaxf(mt, sv[r]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tg = kbase0 + kl0 + 8 * (r >> 2) + 4 * h + (r & 3);
                    const bool vis = col_valid && tg < khi && tg <= hi_c && (!WIN || tg >= lo_c);
                    sv[r] = vis ? sacc[r] * a.scale_log2 : kNegInf;
                    mt = fmaxf(mt, sv[r]);
                }
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            // Lazy rescale: the reference max m_run moves only when a score exceeds it by
            // more than kLazyLog2 (or at the first finite score), so P stays <= 2^kLazyLog2
            // and the O rescale (64 accumulators) runs rarely instead of at most tiles.
            const bool grow = mt > m_run + kLazyLog2;
            if (__ballot(grow)) {
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;  // -inf -> 0
                if (grow) m_run = mt;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            }
            // P goes into the PV product as a bf16 pair hi + lo (about 16 significant
            // bits): a single bf16 rounding of P would perturb the weights by up to 2^-8.
            bf16x8 pb_hi[2], pb_lo[2];
            float ls = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pf = (sv[r] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m_run);
                const __bf16 hi = (__bf16)pf;
                const __bf16 lo = (__bf16)(pf - (float)hi);
                ls += pf;
                pb_hi[r >> 3][r & 7] = __builtin_bit_cast(short, hi);
                pb_lo[r >> 3][r & 7] = __builtin_bit_cast(short, lo);
            }
            l_run += ls;
            // ---- O^T += V^T P^T  (two 16-key k-steps; rows vrow and vrow + 8)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int vrow = kl0 + 16 * s2 + 4 * h + (i16 >> 2);
                const int sw0 = kv_swz<D>(vrow), sw1 = kv_swz<D>(vrow + 8);
                const char* r0p = vtile + vrow * ROWB + 8 * (i16 & 1);
                const char* r1p = r0p + 8 * ROWB;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int chunk = 4 * db + 2 * half + ((i16 & 3) >> 1);
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_bf16x4*)(const lds_char*)(r0p + ((chunk ^ sw0) << 4)));
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_bf16x4*)(const lds_char*)(r1p + ((chunk ^ sw1) << 4)));
                    const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_hi[s2], o[db], 0, 0, 0);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_lo[s2], o[db], 0, 0, 0);
                }
            }
        }
    };
    auto compute_tile = [&](int t, const char* ktile,
                            const char* vtile) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < NB; ++st) compute_sub(ktile, vtile, kg * (TK / KG) + st * 32, t * TK, L);
    };
    // the tail (<= 32 keys) is one sub-tile, for the waves of key group 0
    auto compute_tail = [&]() __attribute__((always_inline)) {
        if (tail_b < tail_e && kg == 0) compute_sub(kts, vts, 0, tail_b, tail_e);
    };

    // Tile t + 1 is in flight while tile t is computed. Before each tile: this wave's DMA
    // landed (s_waitcnt), then every wave's, and every wave is done with the other buffer.
    // Thread 0 publishes the next tile (its claim has returned by then) in s_next[parity]:
    // a slot is rewritten only two barriers after it was read.
    auto next_tile = [&](int t, int par) __attribute__((always_inline)) {
        if (tid == 0) s_next[par] = dyn ? a.nsplit + (int)claim : t + 1;
        __syncthreads();
        const int tn = s_next[par];
        if (tn >= t_last) return -1;
        if (dyn && tid == 0) claim = claim_tile(ctr);
        return tn;
    };
    if (t_first < 0) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        compute_tail();
    }
    for (int t = t_first; t >= 0;) {
        __builtin_amdgcn_s_waitcnt(0);                 // first time: the tail landed too
        const int t1 = next_tile(t, 0);
        if (t1 >= 0) issue_tile(t0 + t1, k1s, v1s);
        compute_tile(t0 + t, k0s, v0s);
        if (t == t_first) compute_tail();
        if (t1 < 0) break;
        __builtin_amdgcn_s_waitcnt(0);
        const int t2 = next_tile(t1, 1);
        if (t2 >= 0) issue_tile(t0 + t2, k0s, v0s);
        compute_tile(t0 + t1, k1s, v1s);
        t = t2;
    }

    // ---- combine the key groups: wave w stores its 32 columns of O in tile buffer w,
    // rows padded to OS floats so the 32 columns of one store hit different banks.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    __syncthreads();                                    // tiles no longer needed
    LdsQuad ob;
    ob.p0 = reinterpret_cast<float*>(k0s);
    ob.p1 = reinterpret_cast<float*>(v0s);
    ob.p2 = reinterpret_cast<float*>(k1s);
    ob.p3 = reinterpret_cast<float*>(v1s);
    float* mine = ob[wave];
    if (h == 0) {
        stats[kg * a.mcap + n] = m_run;
        stats[kStatCap + kg * a.mcap + n] = l_tot;
    }
    // accumulator entries r = 4 i .. 4 i + 3 are 4 consecutive d: one 16-byte store each
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 32 * db + 8 * i + 4 * h;
            *reinterpret_cast<float4*>(mine + col * OS + d) =
                make_float4(o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]);
        }
    __syncthreads();
    attn_epilogue<D, KG, NB>(a, ob, stats, unit, split, g, s, OS);
}

// ------------------------------------------------------------- bf16 Q x quantized K / V
// K and V arrive as unsigned codes (8 or 4 bits) with an fp16 (scale, bias) pair per group
// of 64 dimensions: value = scale * code + bias. The codes go to the MFMAs as exact
// integers (at most 255), so no dequantized value is ever rounded:
//   S[t][n] = sum_g ( s_g[t] * sum_{d in g} code[t][d] q[n][d] + b_g[t] * sum_{d in g} q[n][d] )
//   O[n][d] = sum_t (P[n][t] s_g[t]) code[t][d] + sum_t P[n][t] b_g[t]      (g = group of d)
// QK^T runs in fp16 (K codes built from their bits, q scaled by a power of two per column
// so that it converts exactly); PV runs in bf16 on P s_g split into two bf16 terms (16
// significant bits). The fp16 (scale, bias) enter fp32 arithmetic through mixed fma.
// The same tile schedule as the bf16 kernel (static or claimed tiles, tails, speculative
// first tile). Code rows (D * bits / 8 bytes) are staged by DMA with their 16-byte chunks
// permuted per row (chunk c at c ^ swz(r)) so the QK^T operand reads (32 lanes, 8 codes of
// 32 consecutive rows) hit at most two lanes per bank; the (scale, bias) rows follow the
// codes of each buffer. V codes are expanded once per tile into bf16 integers in the bf16
// kernel's V layout, so the transposed PV operand reads are the same.
template <int ROWB>
__device__ __forceinline__ int code_swz(int r) {
    return (r / (256 / ROWB)) & (ROWB / 16 - 1);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// K codes -> fp16 operands of the QK^T MFMA, exact: a code c (< 1024) under the exponent
// bits of 1024 is the fp16 number 1024 + c, and one packed subtraction of 1024 leaves c.
// 8-bit: dwords w0, w1 hold codes 0..7 in byte order. 4-bit: dword w holds codes 0..7 in
// nibble order; the result holds them as (0, 4, 1, 5, 2, 6, 3, 7), and the Q operand is
// permuted the same way.
__device__ __forceinline__ f16x2 f16_pair_minus_1024(uint32_t d) {
    return __builtin_bit_cast(f16x2, d) - f16x2{(_Float16)1024.f, (_Float16)1024.f};
}
__device__ __forceinline__ f16x8 kcodes8_to_f16(uint32_t w0, uint32_t w1) {
    // byte select over {0x64646464 : w}: selectors 0..3 pick bytes of w, 4 picks 0x64
    constexpr uint32_t kExp = 0x64646464u;
    const f16x2 p0 = f16_pair_minus_1024(__builtin_amdgcn_perm(kExp, w0, 0x04010400u));
    const f16x2 p1 = f16_pair_minus_1024(__builtin_amdgcn_perm(kExp, w0, 0x04030402u));
    const f16x2 p2 = f16_pair_minus_1024(__builtin_amdgcn_perm(kExp, w1, 0x04010400u));
    const f16x2 p3 = f16_pair_minus_1024(__builtin_amdgcn_perm(kExp, w1, 0x04030402u));
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
__device__ __forceinline__ f16x8 kcodes4_to_f16(uint32_t w) {
    const f16x2 p0 = f16_pair_minus_1024((w & 0x000F000Fu) | 0x64006400u);
    const f16x2 p1 = f16_pair_minus_1024(((w >> 4) & 0x000F000Fu) | 0x64006400u);
    const f16x2 p2 = f16_pair_minus_1024(((w >> 8) & 0x000F000Fu) | 0x64006400u);
    const f16x2 p3 = f16_pair_minus_1024(((w >> 12) & 0x000F000Fu) | 0x64006400u);
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// V codes -> 8 bf16 (exact small integers). 8-bit: two dwords; 4-bit: one dword, element
// 2i in the low nibble of byte i.
__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t w0, uint32_t w1) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = __builtin_bit_cast(short, (__bf16)(float)((w0 >> (8 * i)) & 0xFFu));
        r[4 + i] = __builtin_bit_cast(short, (__bf16)(float)((w1 >> (8 * i)) & 0xFFu));
    }
    return r;
}
__device__ __forceinline__ bf16x8 codes4_to_bf16(uint32_t w) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        r[i] = __builtin_bit_cast(short, (__bf16)(float)((w >> (4 * i)) & 0xFu));
    return r;
}

template <int D, int NB, int BITS>
__global__ __launch_bounds__(256, 1) void attn_kvq_kernel(const AttnArgs a) {
    constexpr int TK = 128;                  // keys per tile
    constexpr int NG = D / 64;               // quantization groups per row
    constexpr int KPG = 4;                   // QK^T k-steps (16 dims) per group
    constexpr int ROWB = D * BITS / 8;       // code bytes per key row
    constexpr int CH = ROWB / 16;            // 16-byte chunks per code row
    constexpr int RPI = 1024 / ROWB;         // rows per 1 KB DMA block
    constexpr int CODEB = TK * ROWB;         // code bytes of one matrix tile
    constexpr int BPW = CODEB / 1024 / 4;    // DMA blocks per wave
    constexpr int SBROW = NG * 4;            // (scale, bias) bytes per row
    constexpr int SBB = TK * SBROW;          // ... per tile
    constexpr int VROWB = D * 2;             // expanded V row (bf16)
    constexpr int KSTEPS = D / 16;
    constexpr int DB = D / 32;
    constexpr int KG = 4 / NB;
    constexpr int OS = D + 4;
    constexpr int OBB = 32 * OS * 4;         // one wave's O in the epilogue
    constexpr int BUFB0 = CODEB + SBB;
    constexpr int BUFB = ((BUFB0 > OBB ? BUFB0 : OBB) + 1023) / 1024 * 1024;
    static_assert(CODEB % 4096 == 0 && SBB % 256 == 0, "whole DMA blocks per wave");
    // two stages of (K codes + sb), (V codes + sb): four distinct LDS objects
    __shared__ __attribute__((aligned(1024))) char k0s[BUFB];
    __shared__ __attribute__((aligned(1024))) char v0s[BUFB];
    __shared__ __attribute__((aligned(1024))) char k1s[BUFB];
    __shared__ __attribute__((aligned(1024))) char v1s[BUFB];
    __shared__ __attribute__((aligned(1024))) char vdq[TK * VROWB];   // expanded V tile
    // tail (<= 32 keys per split): codes + sb of K and V, and its expanded V
    constexpr int TCODEB = 32 * ROWB, TSBB = 32 * SBROW;
    __shared__ __attribute__((aligned(1024))) char kts[TCODEB + TSBB];
    __shared__ __attribute__((aligned(1024))) char vts[TCODEB + TSBB];
    __shared__ __attribute__((aligned(1024))) char vtdq[32 * VROWB];
    __shared__ float stats[kStatFloats];
    __shared__ int s_next[2];

    asm volatile("" ::"s"(a.k), "s"(a.v), "s"(a.tile_ctr), "s"(a.cu_rows), "s"(a.ctx_lens),
                 "s"(a.nsplit), "s"(a.hkv), "s"(a.s_max), "s"(a.max_kv_len), "s"(a.dyn),
                 "s"(a.max_rows), "s"(a.ksb), "s"(a.vsb), "s"(a.q), "s"(a.out),
                 "s"(a.part_o), "s"(a.part_ml), "s"(a.err), "s"(a.total_rows), "s"(a.group),
                 "s"(a.mcap), "s"(a.scale_log2));
    int unit, split;
    map_block(blockIdx.x, a.nsplit, &unit, &split);    // the grid is units x nsplit
    const int b = unit / a.hkv, g = unit % a.hkv;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const size_t row0 = ((size_t)b * a.hkv + g) * (size_t)a.s_max;     // first key row
    const char* kbase = reinterpret_cast<const char*>(a.k) + row0 * ROWB;
    const char* vbase = reinterpret_cast<const char*>(a.v) + row0 * ROWB;
    const char* ksbase = reinterpret_cast<const char*>(a.ksb) + row0 * SBROW;
    const char* vsbase = reinterpret_cast<const char*>(a.vsb) + row0 * SBROW;

    // DMA of tile t: wave w fills code blocks w, w + 4, ... of K and of V and the dwords
    // [256 w, 256 w + 256) of each (scale, bias) tile. Keys at or past key_lim read key
    // key_lim - 1.
    const int dma_ri = lane / CH, dma_pos = lane % CH;
    const int dma_off = dma_ri * ROWB + ((dma_pos ^ code_swz<ROWB>(wave * RPI + dma_ri)) << 4);
    const int sb_byte = wave * 256 + lane * 4;         // this lane's dword of an sb tile
    int key_lim;
    auto issue_tile = [&](int t, char* kt, char* vt) __attribute__((always_inline)) {
        if ((t + 1) * TK <= key_lim) {
            const char* kb = kbase + (size_t)t * CODEB;
            const char* vb = vbase + (size_t)t * CODEB;
#pragma unroll
            for (int i = 0; i < BPW; ++i) {
                const int blk = i * 4 + wave;
                __builtin_amdgcn_global_load_lds(kb + blk * 1024 + dma_off,
                                                 (lds_void*)(kt + blk * 1024), 16, 0, kKvPolicy);
                __builtin_amdgcn_global_load_lds(vb + blk * 1024 + dma_off,
                                                 (lds_void*)(vt + blk * 1024), 16, 0, kKvPolicy);
            }
        } else {
#pragma unroll
            for (int i = 0; i < BPW; ++i) {
                const int blk = i * 4 + wave;
                const int r = blk * RPI + dma_ri;
                int key = t * TK + r;
                key = key < key_lim ? key : key_lim - 1;
                const size_t src = (size_t)key * ROWB + (size_t)((dma_pos ^ code_swz<ROWB>(r)) << 4);
                __builtin_amdgcn_global_load_lds(kbase + src, (lds_void*)(kt + blk * 1024), 16, 0, kKvPolicy);
                __builtin_amdgcn_global_load_lds(vbase + src, (lds_void*)(vt + blk * 1024), 16, 0, kKvPolicy);
            }
        }
        if (wave * 256 < SBB) {
            const int r = sb_byte / SBROW;
            int key = t * TK + r;
            key = key < key_lim ? key : key_lim - 1;
            const size_t src = (size_t)key * SBROW + sb_byte % SBROW;
            __builtin_amdgcn_global_load_lds(ksbase + src, (lds_void*)(kt + CODEB + wave * 256), 4, 0, kKvPolicy);
            __builtin_amdgcn_global_load_lds(vsbase + src, (lds_void*)(vt + CODEB + wave * 256), 4, 0, kKvPolicy);
        }
    };

    const bool tails = a.nsplit >= 4;
    const bool dyn = a.dyn != 0;
    auto tile_count = [&](int len) __attribute__((always_inline)) {
        return tails ? len / TK : (len + TK - 1) / TK;
    };
    auto static_end = [&](int nt) __attribute__((always_inline)) {
        return (int)((uint32_t)((split + 1) * nt) / (uint32_t)a.nsplit);
    };
    auto first_tile = [&](int nt) __attribute__((always_inline)) {
        const int t = dyn ? split : (int)((uint32_t)(split * nt) / (uint32_t)a.nsplit);
        return t < (dyn ? nt : static_end(nt)) ? t : -1;
    };
    const int kv_cap = a.max_kv_len < a.s_max ? a.max_kv_len : a.s_max;
    const int t_spec = first_tile(tile_count(kv_cap));
    key_lim = kv_cap;
    if (t_spec >= 0) issue_tile(t_spec, k0s, v0s);
    uint32_t* const ctr = counter_at(a.tile_ctr, a.tile_ctr_x, unit);
    uint32_t claim;                                    // thread 0 only (see the bf16 kernel)
    if (dyn && tid == 0) claim = claim_tile(ctr);

    const SeqGeom s = seq_geometry(a, b, tid == 0 && split == 0 && g == 0);
    if (!s.ok) {
        __builtin_amdgcn_s_waitcnt(0);
        if (a.nsplit > 1 && !a.merge_kernel) attn_finish_unit<D>(a, unit, g, s, false);
        return;
    }
    const int L = s.ctx + s.rows;
    const int nt = tile_count(L);
    const int t_first = first_tile(nt);
    const int t_last = dyn ? nt : static_end(nt);
    int tail_b = 0, tail_e = 0;
    if (tails) {
        const int f = L / TK * TK, rem = L - f;
        tail_b = f + (int)((uint32_t)(split * rem) / (uint32_t)a.nsplit);
        tail_e = f + (int)((uint32_t)((split + 1) * rem) / (uint32_t)a.nsplit);
    }
    key_lim = L;
    if (t_first < 0 && tail_b >= tail_e) {
        __builtin_amdgcn_s_waitcnt(0);
        attn_empty_split<D>(a, unit, split, g, s);
        return;
    }
    // The speculative tile is kept as it landed: rows past the sequence hold finite codes
    // (any byte is a code), and their (scale, bias), which may not be finite, are zeroed
    // before use. Every other DMA repeats the last key of its range in such rows.
    if (t_first >= 0 && t_first != t_spec) {
        __builtin_amdgcn_s_waitcnt(0);
        issue_tile(t_first, k0s, v0s);
    }
    if (tail_b < tail_e) {
        // rows past the tail end read its last key
        if (wave * 1024 < TCODEB) {
            const int r = wave * RPI + dma_ri;
            int key = tail_b + r;
            key = key < tail_e ? key : tail_e - 1;
            const size_t src = (size_t)key * ROWB + (size_t)((dma_pos ^ code_swz<ROWB>(r)) << 4);
            __builtin_amdgcn_global_load_lds(kbase + src, (lds_void*)(kts + wave * 1024), 16, 0, kKvPolicy);
            __builtin_amdgcn_global_load_lds(vbase + src, (lds_void*)(vts + wave * 1024), 16, 0, kKvPolicy);
        }
        if (wave == 0 && lane * 4 < TSBB) {
            int key = tail_b + lane * 4 / SBROW;
            key = key < tail_e ? key : tail_e - 1;
            const size_t src = (size_t)key * SBROW + (lane * 4) % SBROW;
            __builtin_amdgcn_global_load_lds(ksbase + src, (lds_void*)(kts + TCODEB), 4, 0, kKvPolicy);
            __builtin_amdgcn_global_load_lds(vsbase + src, (lds_void*)(vts + TCODEB), 4, 0, kKvPolicy);
        }
    }

    const int nb = wave % NB, kg = wave / NB;
    const int h = lane >> 5, col = lane & 31;
    const int n = nb * 32 + col;
    const int M = s.rows * a.group;
    const bool col_valid = n < M;
    const int ri = col_valid ? n / a.group : 0;
    const int hh = col_valid ? n % a.group : 0;
    const int causal_lim = s.ctx + ri;

    // This column's q as fp16, scaled by 2^qe so that its largest magnitude lies in
    // [2^14, 2^15): every bf16 value within 2^24 of that maximum converts exactly (the
    // smaller ones, if any, round at 2^-24 of the fp16 range, far below the score
    // tolerance); the scores are scaled back by 2^-qe, folded into qfac.
    f16x8 qh[KSTEPS];
    float qfac;
    {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                             ((size_t)(s.r0 + ri) * a.hq + g * a.group + hh) * D;
        float qv[KSTEPS][8];
        float qmax = 0.f;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            bf16x8 w = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (col_valid) w = *reinterpret_cast<const bf16x8*>(qp + 16 * kk + 8 * h);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qv[kk][e] = (float)__builtin_bit_cast(__bf16, (short)w[e]);
                qmax = fmaxf(qmax, fabsf(qv[kk][e]));
            }
        }
        qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
        int qe = 0;
        if (qmax > 0.f && qmax <= 3.0e38f) {
            int ex;
            (void)__builtin_frexpf(qmax, &ex);
            qe = 15 - ex;
        }
        qfac = __builtin_ldexpf(a.scale_log2, -qe);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // 4-bit K operands hold dims (0, 4, 1, 5, 2, 6, 3, 7) of each 8
                const int pos = BITS == 4 ? (e < 4 ? 2 * e : 2 * (e - 4) + 1) : e;
                qh[kk][pos] = (_Float16)__builtin_ldexpf(qv[kk][e], qe);
            }
    }
    // per-group sums of this column's (scaled, fp16) q: the bias term of the scores
    float qsum[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        float sm = 0.f;
#pragma unroll
        for (int kk = gi * KPG; kk < (gi + 1) * KPG; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm += (float)qh[kk][e];
        qsum[gi] = sm + __shfl_xor(sm, 32);
    }

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;
    const int i16 = lane & 15;
    const int half = (lane >> 4) & 1;

    // The bias term of O, sum_t P[n][t] b_g[t], is kept per group as one running value per
    // lane (column n), rescaled with O, and added to O once after the last tile.
    float bacc[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) bacc[gi] = 0.f;

    // (scale, bias) fp16 pairs of group gi for this lane's keys kl0 + 8 j + 4 h + (0..3),
    // as packed dwords (every lane of a half-wave reads the same ones)
    auto load_sb = [&](const char* sbt, int kl0, int gi, uint32_t (&w)[16])
        __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
                w[4 * j + k4] = *reinterpret_cast<const uint32_t*>(
                    sbt + (kl0 + 8 * j + 4 * h + k4) * SBROW + gi * 4);
    };
    auto lo_f16 = [](uint32_t w) __attribute__((always_inline)) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
    };
    auto hi_f16 = [](uint32_t w) __attribute__((always_inline)) {
        return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
    };

    // One 32-key sub-tile: code rows kl0 .. kl0 + 31 of ktile (their (scale, bias) rows in
    // ksbt) and expanded V rows of vtile (scale, bias in vsbt) hold keys kbase0 + row; keys
    // at or past khi are masked.
    auto compute_sub = [&](const char* ktile, const char* ksbt, const char* vtile,
                           const char* vsbt, int kl0, int kbase0, int khi)
        __attribute__((always_inline)) {
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        {
            const int krow = kl0 + col;
            const int ksw = code_swz<ROWB>(krow);
            const char* kr = ktile + krow * ROWB;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                f32x16 acc;
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
                for (int kk = gi * KPG; kk < (gi + 1) * KPG; ++kk) {
                    f16x8 ka;
                    if constexpr (BITS == 8) {
                        // dims 16 kk + 8 h .. + 8: half h of chunk kk
                        const uint2 w = *reinterpret_cast<const uint2*>(
                            kr + ((kk ^ ksw) << 4) + 8 * h);
                        ka = kcodes8_to_f16(w.x, w.y);
                    } else {
                        // 4 bytes at 8 kk + 4 h: chunk kk / 2, byte 8 (kk & 1) + 4 h
                        const uint32_t w = *reinterpret_cast<const uint32_t*>(
                            kr + (((kk >> 1) ^ ksw) << 4) + 8 * (kk & 1) + 4 * h);
                        ka = kcodes4_to_f16(w);
                    }
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qh[kk], acc, 0, 0, 0);
                }
                uint32_t sbw[16];
                load_sb(ksbt, kl0, gi, sbw);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sacc[r] = __builtin_fmaf(lo_f16(sbw[r]), acc[r],
                                             __builtin_fmaf(hi_f16(sbw[r]), qsum[gi], sacc[r]));
            }
        }
        float sv[16];
        float mt = kNegInf;
        if (kbase0 + kl0 + 31 <= s.ctx && kbase0 + kl0 + 31 < khi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sv[r] = sacc[r] * qfac;
                mt = fmaxf(mt, sv[r]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tg = kbase0 + kl0 + 8 * (r >> 2) + 4 * h + (r & 3);
                const bool vis = col_valid && tg < khi && tg <= causal_lim;
                sv[r] = vis ? sacc[r] * qfac : kNegInf;
                mt = fmaxf(mt, sv[r]);
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const bool grow = mt > m_run + kLazyLog2;
        if (__ballot(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
            if (grow) m_run = mt;
            l_run *= alpha;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) bacc[gi] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
        float pf[16];
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            pf[r] = (sv[r] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m_run);
            ls += pf[r];
        }
        l_run += ls;
        // ---- O^T += V^T (P s_g)^T per group; the bias term into bacc (every (scale, bias)
        // of the tile is finite: rows past the sequence were zeroed or repeat a key of it)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            uint32_t sbw[16];
            load_sb(vsbt, kl0, gi, sbw);
            bf16x8 pb_hi[2], pb_lo[2];
            float bsum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pw = __builtin_fmaf(pf[r], lo_f16(sbw[r]), 0.f);
                bsum = __builtin_fmaf(pf[r], hi_f16(sbw[r]), bsum);
                const __bf16 hi = (__bf16)pw;
                const __bf16 lo = (__bf16)(pw - (float)hi);
                pb_hi[r >> 3][r & 7] = __builtin_bit_cast(short, hi);
                pb_lo[r >> 3][r & 7] = __builtin_bit_cast(short, lo);
            }
            bacc[gi] += bsum;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int vrow = kl0 + 16 * s2 + 4 * h + (i16 >> 2);
                const int sw0 = kv_swz<D>(vrow), sw1 = kv_swz<D>(vrow + 8);
                const char* r0p = vtile + vrow * VROWB + 8 * (i16 & 1);
                const char* r1p = r0p + 8 * VROWB;
#pragma unroll
                for (int db = gi * (DB / NG); db < (gi + 1) * (DB / NG); ++db) {
                    const int chunk = 4 * db + 2 * half + ((i16 & 3) >> 1);
                    const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_bf16x4*)(const lds_char*)(r0p + ((chunk ^ sw0) << 4)));
                    const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_bf16x4*)(const lds_char*)(r1p + ((chunk ^ sw1) << 4)));
                    const bf16x8 va = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_hi[s2], o[db], 0, 0, 0);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_lo[s2], o[db], 0, 0, 0);
                }
            }
        }
    };

    // (scale, bias) rows of keys at or past L in the speculative tile t -> 0 (after every
    // wave's DMA of the tile landed)
    auto zero_sb = [&](int t, char* kt, char* vt) __attribute__((always_inline)) {
        if (t == t_spec && (t + 1) * TK > L && tid < TK && t * TK + tid >= L) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                *reinterpret_cast<uint32_t*>(kt + CODEB + tid * SBROW + gi * 4) = 0u;
                *reinterpret_cast<uint32_t*>(vt + CODEB + tid * SBROW + gi * 4) = 0u;
            }
        }
    };
    // V codes of `rows` rows -> bf16 integers in the bf16 kernel's V layout
    auto expand_v = [&](const char* vcodes, char* vexp, int rows) __attribute__((always_inline)) {
        for (int ci = tid; ci < rows * CH; ci += kThreads) {
            const int r = ci / CH, c = ci % CH;
            const uint4 w = *reinterpret_cast<const uint4*>(
                vcodes + r * ROWB + ((c ^ code_swz<ROWB>(r)) << 4));
            char* dst = vexp + r * VROWB;
            const int sw = kv_swz<D>(r);
            if constexpr (BITS == 8) {
                *reinterpret_cast<bf16x8*>(dst + (((2 * c) ^ sw) << 4)) = codes8_to_bf16(w.x, w.y);
                *reinterpret_cast<bf16x8*>(dst + (((2 * c + 1) ^ sw) << 4)) = codes8_to_bf16(w.z, w.w);
            } else {
                *reinterpret_cast<bf16x8*>(dst + (((4 * c) ^ sw) << 4)) = codes4_to_bf16(w.x);
                *reinterpret_cast<bf16x8*>(dst + (((4 * c + 1) ^ sw) << 4)) = codes4_to_bf16(w.y);
                *reinterpret_cast<bf16x8*>(dst + (((4 * c + 2) ^ sw) << 4)) = codes4_to_bf16(w.z);
                *reinterpret_cast<bf16x8*>(dst + (((4 * c + 3) ^ sw) << 4)) = codes4_to_bf16(w.w);
            }
        }
    };
    auto compute_tile = [&](int t, const char* kt, const char* vt) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < NB; ++st)
            compute_sub(kt, kt + CODEB, vdq, vt + CODEB, kg * (TK / KG) + st * 32, t * TK, L);
    };
    auto compute_tail = [&]() __attribute__((always_inline)) {
        if (tail_b < tail_e && kg == 0)
            compute_sub(kts, kts + TCODEB, vtdq, vts + TCODEB, 0, tail_b, tail_e);
    };
    auto next_tile = [&](int t, int par) __attribute__((always_inline)) {
        if (tid == 0) s_next[par] = dyn ? a.nsplit + (int)claim : t + 1;
        __syncthreads();
        const int tn = s_next[par];
        if (tn >= t_last) return -1;
        if (dyn && tid == 0) claim = claim_tile(ctr);
        return tn;
    };

    // Tile t + 1 is in flight while tile t is expanded and computed. Before each tile: this
    // wave's DMA landed (s_waitcnt), then every wave's, and every wave is done with the
    // other buffers and with the expanded V of the previous tile.
    if (t_first < 0) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        expand_v(vts, vtdq, 32);
        __syncthreads();
        compute_tail();
    }
    for (int t = t_first; t >= 0;) {
        __builtin_amdgcn_s_waitcnt(0);                 // first time: the tail landed too
        const int t1 = next_tile(t, 0);
        if (t1 >= 0) issue_tile(t1, k1s, v1s);
        if (t == t_first) zero_sb(t, k0s, v0s);
        expand_v(v0s, vdq, TK);
        if (t == t_first && tail_b < tail_e) expand_v(vts, vtdq, 32);
        __syncthreads();
        compute_tile(t, k0s, v0s);
        if (t == t_first) compute_tail();
        if (t1 < 0) break;
        __builtin_amdgcn_s_waitcnt(0);
        const int t2 = next_tile(t1, 1);
        if (t2 >= 0) issue_tile(t2, k0s, v0s);
        expand_v(v1s, vdq, TK);
        __syncthreads();
        compute_tile(t1, k1s, v1s);
        t = t2;
    }

    // ---- the bias term (this lane's keys; the other half-wave holds the rest of the
    // column's), then combine the key groups as in the bf16 kernel
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const float bt = bacc[gi] + __shfl_xor(bacc[gi], 32);
#pragma unroll
        for (int db = gi * (DB / NG); db < (gi + 1) * (DB / NG); ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] += bt;
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    __syncthreads();                                    // buffers no longer needed
    LdsQuad ob;
    ob.p0 = reinterpret_cast<float*>(k0s);
    ob.p1 = reinterpret_cast<float*>(v0s);
    ob.p2 = reinterpret_cast<float*>(k1s);
    ob.p3 = reinterpret_cast<float*>(v1s);
    float* mine = ob[wave];
    if (h == 0) {
        stats[kg * a.mcap + n] = m_run;
        stats[kStatCap + kg * a.mcap + n] = l_tot;
    }
    // accumulator entries r = 4 i .. 4 i + 3 are 4 consecutive d: one 16-byte store each
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 32 * db + 8 * i + 4 * h;
            *reinterpret_cast<float4*>(mine + col * OS + d) =
                make_float4(o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]);
        }
    __syncthreads();
    attn_epilogue<D, KG, NB>(a, ob, stats, unit, split, g, s, OS);
}

// -------------------------------------------------------------------------- fp32 / FMA
// Same split and merge as the bf16 kernel; per tile of 32 keys: scores S[n][key] (one dot
// product per thread task), an online-softmax update per column, then O[n][d] += P V. All
// state lives in LDS, laid out so the shared epilogue finds O and (max, sum) in place.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const AttnArgs a) {
    constexpr int TK = 32;
    constexpr int MCOLS = 128;                  // column capacity
    constexpr int KROW = D + 1;                 // padded K row (floats)
    //  O [MCOLS][D] | m, l, 3 epilogue arrays [5][MCOLS] | S [MCOLS][TK] | alpha [MCOLS]
    //  | K [TK][KROW] | V [TK][D]
    constexpr int SMEM = (MCOLS * D + 5 * MCOLS + MCOLS * TK + MCOLS + TK * KROW + TK * D) * 4;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    int unit, split;
    map_block(blockIdx.x, a.nsplit, &unit, &split);
    if (unit >= a.units) return;
    const int b = unit / a.hkv, g = unit % a.hkv;
    const int tid = threadIdx.x;
    const SeqGeom s = seq_geometry(a, b, tid == 0 && split == 0 && g == 0);
    if (!s.ok) {
        if (a.nsplit > 1 && !a.merge_kernel) attn_finish_unit<D>(a, unit, g, s, false);
        return;
    }
    const int M = s.rows * a.group;
    const int L = s.ctx + s.rows;
    const int lo_first = key_lo(a, s, 0);
    const int k0 = lo_first / TK * TK;                   // first streamed key
    const int ntiles = (L - k0 + TK - 1) / TK;
    const int t_begin = (int)((long)split * ntiles / a.nsplit);
    const int t_end = (int)((long)(split + 1) * ntiles / a.nsplit);
    float* os = reinterpret_cast<float*>(smem);          // [MC][D]   (epilogue O)
    float* st = os + MCOLS * D;                          // epilogue statistics
    float* ms = st;                                      // [MC]      (epilogue gm)
    float* ls = st + kStatCap;                           // [MC]      (epilogue gl)
    float* ss = os + MCOLS * D + 5 * MCOLS;              // [MCOLS][TK]
    if (t_begin >= t_end) {
        attn_empty_split<D>(a, unit, split, g, s);
        return;
    }

    float* al = ss + MCOLS * TK;                         // [MCOLS]
    float* ks = al + MCOLS;                              // [TK][KROW]
    float* vs = ks + TK * KROW;                          // [TK][D]

    for (int e = tid; e < M * D; e += kThreads) os[e] = 0.f;
    for (int n = tid; n < M; n += kThreads) { ms[n] = kNegInf; ls[n] = 0.f; }

    const float* qg = reinterpret_cast<const float*>(a.q);
    const size_t kv_off = ((size_t)b * a.hkv + g) * (size_t)a.s_max * D;
    const float* kb = reinterpret_cast<const float*>(a.k) + kv_off;
    const float* vb = reinterpret_cast<const float*>(a.v) + kv_off;

    for (int t = t_begin; t < t_end; ++t) {
        __syncthreads();
        for (int e = tid; e < TK * D; e += kThreads) {
            const int kr = e / D, d = e % D;
            const int key = k0 + t * TK + kr;
            const bool in = key < L && key >= lo_first;
            ks[kr * KROW + d] = in ? kb[(size_t)key * D + d] : 0.f;
            vs[e] = in ? vb[(size_t)key * D + d] : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < M * TK; e += kThreads) {
            const int n = e / TK, kr = e % TK;
            const int key = k0 + t * TK + kr;
            const float* qrow = qg + ((size_t)(s.r0 + n / a.group) * a.hq + g * a.group +
                                      n % a.group) * D;
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(qrow[d], ks[kr * KROW + d], dot);
            const int ri = n / a.group;
            const bool vis = key < L && key <= key_hi(a, s, ri) && key >= key_lo(a, s, ri);
            ss[n * TK + kr] = vis ? dot * a.scale_log2 : kNegInf;
        }
        __syncthreads();
        for (int n = tid; n < M; n += kThreads) {
            float mt = kNegInf;
            for (int kr = 0; kr < TK; ++kr) mt = fmaxf(mt, ss[n * TK + kr]);
            const float m_new = fmaxf(ms[n], mt);
            const float alpha = (m_new == kNegInf) ? 1.f : exp2f(ms[n] - m_new);
            float lsum = 0.f;
            for (int kr = 0; kr < TK; ++kr) {
                const float sc = ss[n * TK + kr];
                const float p = (sc == kNegInf) ? 0.f : exp2f(sc - m_new);
                ss[n * TK + kr] = p;
                lsum += p;
            }
            ls[n] = ls[n] * alpha + lsum;
            ms[n] = m_new;
            al[n] = alpha;
        }
        __syncthreads();
        for (int e = tid; e < M * D; e += kThreads) {
            const int n = e / D, d = e % D;
            float o = os[e] * al[n];
            for (int kr = 0; kr < TK; ++kr) o = fmaf(ss[n * TK + kr], vs[kr * D + d], o);
            os[e] = o;
        }
    }
    __syncthreads();
    LdsQuad ob;
    ob.p0 = os;
    ob.p1 = os + 32 * D;
    ob.p2 = os + 64 * D;
    ob.p3 = os + 96 * D;
    attn_epilogue<D, 1, 4>(a, ob, st, unit, split, g, s, D);
}


// -------------------------------------------------------------------------- split merge
// For units whose partials are too many for one workgroup to merge quickly (many splits of
// many columns, see plan_attention), this kernel runs after the attention kernel (stream
// order makes every partial visible):
//   out = sum_s w_s O_s,   w_s = 2^(m_s - m) / sum_s' 2^(m_s' - m) l_s',   m = max_s m_s
// over the key splits s of one (sequence, KV head) unit. Thread e of the unit's slice owns
// column n = e / (D/4) and 4 consecutive d; the geometry, (max, sum) and O loads of up to
// kMergeGroup splits are issued together, so one memory round trip covers <= 8 splits.
// Columns past the sequence's M read workspace slots nobody wrote this call; their
// results are computed and dropped.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnArgs a) {
    constexpr int D4 = D / 4;
    constexpr int SG = kMergeGroup;
    const int chunks = (a.mcap * D4 + kThreads - 1) / kThreads;
    const int unit = blockIdx.x / chunks;
    const int e = (blockIdx.x % chunks) * kThreads + threadIdx.x;
    if (unit >= a.units) return;
    // the attention kernel has finished: its tile counter returns to zero for the next call
    if (a.dyn && e == 0) __hip_atomic_store(counter_at(a.tile_ctr, a.tile_ctr_x, unit), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e >= a.mcap * D4) return;
    const int b = unit / a.hkv, g = unit % a.hkv;
    const int n = e / D4, d4 = e % D4;
    const int ns = a.nsplit;
    const size_t base = (size_t)unit * ns;
    const float2* pml = a.part_ml + base * a.mcap + n;
    const float4* po = reinterpret_cast<const float4*>(a.part_o) + (base * a.mcap + n) * D4 + d4;
    const size_t sstride = (size_t)a.mcap * D4;              // float4s between splits

    float m_run = kNegInf, l_run = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    SeqGeom s{};
    for (int s0 = 0; s0 < ns; s0 += SG) {
        float2 ml[SG];
        float4 v[SG];
#pragma unroll
        for (int u = 0; u < SG; ++u) {
            const int sp = s0 + u < ns ? s0 + u : ns - 1;    // in bounds; dropped below
            ml[u] = pml[(size_t)sp * a.mcap];
            v[u] = po[sp * sstride];
        }
        if (s0 == 0) s = seq_geometry(a, b, false);
        float m = m_run;
#pragma unroll
        for (int u = 0; u < SG; ++u)
            if (s0 + u < ns) m = fmaxf(m, ml[u].x);
        if (m == kNegInf) continue;
        const float c = exp2f(m_run - m);                    // m_run = -inf gives 0
        l_run *= c;
        acc = make_float4(acc.x * c, acc.y * c, acc.z * c, acc.w * c);
#pragma unroll
        for (int u = 0; u < SG; ++u) {
            const float f = (s0 + u < ns && ml[u].x != kNegInf) ? exp2f(ml[u].x - m) : 0.f;
            l_run += f * ml[u].y;
            acc.x += f * v[u].x;
            acc.y += f * v[u].y;
            acc.z += f * v[u].z;
            acc.w += f * v[u].w;
        }
        m_run = m;
    }
    if (!s.ok || n >= s.rows * a.group) return;
    const float il = 1.f / l_run;
    const int row = s.r0 + n / a.group, head = g * a.group + n % a.group;
    *reinterpret_cast<float4*>(a.out + ((size_t)row * a.hq + head) * D + 4 * d4) =
        make_float4(acc.x * il, acc.y * il, acc.z * il, acc.w * il);
}

}  // namespace

AttnPlan plan_attention(int B, int Hq, int Hkv, int D, int max_rows, int max_kv_len) {
    AttnPlan p{};
    const int G = Hq / Hkv;
    const int cols = G * max_rows;
    p.nb = cols <= 32 ? 1 : cols <= 64 ? 2 : 4;
    p.mcap = 32 * p.nb;
    p.units = B * Hkv;
    p.tile = 128;
    // Aim for about VSA_ATTN_TARGET_WGS workgroups over the 256 CUs, at least one tile each.
    const int tiles = (int)(((long)max_kv_len + p.tile - 1) / p.tile);
    int nsplit = (VSA_ATTN_TARGET_WGS + p.units - 1) / p.units;
    if (nsplit > tiles) nsplit = tiles;
    if (nsplit > kMaxSplits) nsplit = kMaxSplits;
    if (nsplit < 1) nsplit = 1;
    p.nsplit = nsplit;
    // The last split of a unit to finish merges the unit's partials itself while they are
    // few (it reads nsplit * mcap * D floats, from the device-coherent level: up to 128 KB
    // takes one workgroup about a microsecond); beyond that a separate kernel merges, spread
    // over the units' columns.
    p.merge_kernel = nsplit > 1 && (size_t)nsplit * p.mcap * D * 4 > ((size_t)128 << 10);
    size_t off = kWsHeader;                                      // error word, counters
    // tile claims, arrivals, then the merge slots of every (unit, split)
    p.n_ctr_x = extra_counters(2L * p.units + (long)p.units * nsplit);
    p.off_ctr_x = off;
    off += (p.n_ctr_x * 4 + 255) / 256 * 256;
    p.off_ml = off;
    off += ((size_t)p.units * nsplit * p.mcap * 8 + 255) / 256 * 256;
    p.off_o = off;
    off += (size_t)p.units * nsplit * p.mcap * D * 4;
    p.bytes = off;
    return p;
}

// Compute units of the current device (cached per device).
static int device_cus() {
    static std::mutex mu;
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
            cus[dev] = n;
    }
    return cus[dev];
}

hipError_t launch_attention(const AttnArgs& args, const AttnPlan& p, vsa_dtype dtype,
                            hipStream_t stream) {
    const dim3 grid(p.units * p.nsplit), block(kThreads);
    // The merge is split over the unit's splits when the whole grid fits on the device at
    // once (one workgroup per CU at most), so a split waiting for its slice never holds a CU
    // that another split of its unit still needs; the wait is bounded in any case.
    AttnArgs a = args;
    a.slice_merge = p.nsplit > 1 && !p.merge_kernel && (int)grid.x <= device_cus();
    a.merge_wait = kMergeWaitTicks;
    if (a.bits == 8 || a.bits == 4) {
#define VSA_KVQ(DD, NBB, BB) hipLaunchKernelGGL((attn_kvq_kernel<DD, NBB, BB>), grid, block, 0, stream, a)
        if (a.bits == 8) {
            if (a.d == 128) {
                if (p.nb == 1) VSA_KVQ(128, 1, 8); else if (p.nb == 2) VSA_KVQ(128, 2, 8); else VSA_KVQ(128, 4, 8);
            } else {
                if (p.nb == 1) VSA_KVQ(64, 1, 8); else if (p.nb == 2) VSA_KVQ(64, 2, 8); else VSA_KVQ(64, 4, 8);
            }
        } else {
            if (a.d == 128) {
                if (p.nb == 1) VSA_KVQ(128, 1, 4); else if (p.nb == 2) VSA_KVQ(128, 2, 4); else VSA_KVQ(128, 4, 4);
            } else {
                if (p.nb == 1) VSA_KVQ(64, 1, 4); else if (p.nb == 2) VSA_KVQ(64, 2, 4); else VSA_KVQ(64, 4, 4);
            }
        }
#undef VSA_KVQ
    } else if (dtype == VSA_BF16) {
#define VSA_BF16K(DD, NBB, WW) hipLaunchKernelGGL((attn_bf16_kernel<DD, NBB, WW>), grid, block, 0, stream, a)
#define VSA_BF16D(DD, WW)                                                      \
    do {                                                                       \
        if (p.nb == 1) VSA_BF16K(DD, 1, WW);                                   \
        else if (p.nb == 2) VSA_BF16K(DD, 2, WW);                              \
        else VSA_BF16K(DD, 4, WW);                                             \
    } while (0)
        const bool win = a.window > 0 || a.mask != 0;
        if (a.d == 128) {
            if (win) VSA_BF16D(128, true); else VSA_BF16D(128, false);
        } else {
            if (win) VSA_BF16D(64, true); else VSA_BF16D(64, false);
        }
#undef VSA_BF16D
#undef VSA_BF16K
    } else {
        if (a.d == 128) hipLaunchKernelGGL((attn_f32_kernel<128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_f32_kernel<64>), grid, block, 0, stream, a);
    }
    if (p.merge_kernel) {
        const dim3 mgrid(p.units * ((p.mcap * (a.d / 4) + kThreads - 1) / kThreads));
        if (a.d == 128) hipLaunchKernelGGL((attn_merge_kernel<128>), mgrid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_merge_kernel<64>), mgrid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace vsa
