// Fused vocabulary stage for sequences without truncation (gfx950): penalties, greedy or
// sampled acceptance, the residual / bonus draw and chosen logprobs in ONE kernel.
//
// Pages (mlx-dspark): penalties per verify position from the base counts plus the
// position's own draft prefix, raw logprobs (Changelog [0.2.0] "Added"); accept with
// probability min(1, p/q), resample max(0, p - q) on rejection, an exact target sample
// (release v0.0.2 "Highlights"); greedy acceptance as the product of positionwise matches
// (Changelog [0.2.0] "Decode-path performance"); one-hot proposals for prompt-lookup drafts
// (Changelog [0.2.0] "Added", --mode lookup).
//
// Grid B x NC workgroups, workgroup (b, c) owns ids [2048 c, 2048 c + 2048) of every row of
// sequence b. All of them are resident at once (the host launches this kernel only when the
// occupancy allows it).
//   phase 1  the chunk of the count histogram and of every row (target, draft, raw) in one
//            round of loads; per (row, chunk) the max and sum of 2^((v - max) log2(e) / T),
//            or the (value, id) argmax of a greedy row, stored write-through; then the
//            sequence's arrival counter A.
//   greedy   the last arriver merges the chunks, accepts the longest matching prefix and
//            writes every output.
//   sampled  the last arriver merges the chunks, takes the acceptance decisions, writes
//            the accepted length and drafts, and publishes the decision (a record of the
//            draw's rows and their merged statistics, written through, then a go flag);
//            every other workgroup waits for the flag and reads the record. The draw over
//            the vocabulary (residual of the first rejected row, or the bonus row) is an
//            exponential race; each workgroup races its own chunk from the values still in
//            its registers and folds the winner into the sequence's 64-bit word with an
//            atomic max (key bits over the complemented id: larger key, then lower id,
//            wins). The workgroup that counts the last chunk into the done counter D writes
//            the token and returns the sequence's words and counters to zero.
// Waiting can time out (a budget per workgroup; other work may hold CUs). A chunk is then
// never lost: its owner marks it abandoned and counts in; every workgroup counts into the
// sequence's done counter D exactly once (after racing its chunk, or abandoning it), and the
// one that completes D (so every other has finished with the sequence's state) races the
// abandoned chunks itself, writes the token and returns the state to zero. The token is
// thus always the race's.
#include "sample_common.h"

namespace vsa {

using namespace samp;

namespace {

constexpr int kRowBatch = 12;        // rows whose chunk loads are in flight together
constexpr int kFusedRows = 3 * kMaxSeqRows;
constexpr int kPrePos = 8;           // draw positions whose race variates a waiting workgroup
                                     // may compute ahead (sequences with K < kPrePos)

// The decision of a sampled sequence, published by its last arriver for the others (the
// workspace's race-request slot of the sequence, 56 bytes: seven 8-byte stores).
struct DrawRec {
    int kind, acc, pos, onehot_d;    // draw kind (1 residual, 2 bonus), accepted drafts
    float m_p, m_q, m_x, pad;        // row maxima: target row acc, draft row acc + 1, raw row
    double z_p, z_q, z_x;            // their normalizers
};
static_assert(sizeof(DrawRec) == 56 && sizeof(DrawRec) <= sizeof(RaceReq), "record slot");

struct FusedShared {
    float4 part[2 * kRowBatch][4];   // per (row of the batch or its raw row, wave) partials
    int drafts[kMaxSeqRows];
    float rm[kFusedRows];            // merged per row: max (softmax) / best value (greedy)
    double rz[kFusedRows];           // normalizer (softmax rows)
    int rarg[kFusedRows];            // argmax (greedy rows)
    unsigned long long win[8];       // per-wave race winners (residual, fallback)
    DrawRec rec;                     // the decision, as the last arriver published it
    int acc, kind;                   // decision: accepted drafts, draw kind (1 resid, 2 bonus)
    int flag;
    int go_seen;                     // the go flag, as thread 0 last read it
    uint32_t state[kMaxChunks];      // abandon flags seen by the workgroup completing D
    // 1 / (-log2 U) of this chunk's ids for the draw at position positions[b] + p, computed
    // while the workgroup waits for the decision
    float einv[kPrePos][kEpt][kThreads];
};

__device__ __forceinline__ float2 coh_load2(const float2* p) { return handoff_load(p); }

// Sequence b's arrival counter A and done counter D sit alone on lines 4b and 4b + 1
// (counters sharing a line serialize each other's atomics), the go flag on line 4b + 2 (so
// waiting workgroups poll a line the arrivals do not need), the count of abandoned chunks
// on line 4b + 3, the winner words in the 64-bit slots of lines 4b + 2 and 4b + 3, and the
// abandon flags of its chunks on the lines past the first 4B.
struct SeqState {
    uint32_t* A;
    uint32_t* D;
    uint32_t* go;      // set by the last arriver once the decision record is in place
    uint32_t* Ab;      // chunks abandoned by their owners
    unsigned long long* Wr;
    unsigned long long* Wp;
    int first;         // abandon flag of chunk c: flag_at(first + c)
};
__device__ __forceinline__ SeqState seq_state(const SampArgs& a, int b) {
    SeqState s;
    s.A = counter_at(a.ctr, a.ctr_x, 4 * b);
    s.D = counter_at(a.ctr, a.ctr_x, 4 * b + 1);
    s.go = counter_at(a.ctr, a.ctr_x, 4 * b + 2);
    s.Ab = counter_at(a.ctr, a.ctr_x, 4 * b + 3);
    s.Wr = word64_at(a.ctr, 4 * b + 2);
    s.Wp = word64_at(a.ctr, 4 * b + 3);
    s.first = b * a.nchunk;
    return s;
}
__device__ __forceinline__ uint32_t* flag_at(const SampArgs& a, const SeqState& s, int c) {
    const int span = kCtrLines - 4 * a.batch;
    const int i = s.first + c;
    return a.ctr + ctr_slot((1 + i / span) * kCtrLines + 4 * a.batch + i % span);
}

__device__ __forceinline__ uint32_t coh_load_u32(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long coh_load_u64(unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide max of two packed race winners at once (both chains interleave), on the DPP
// steps of the float reductions with each 64-bit value moved as two halves; the results
// are wave-uniform.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ void max_step_u64(uint32_t& hi, uint32_t& lo) {
    const uint32_t oh = (uint32_t)dpp_i<CTRL, ROWS>((int)hi, (int)hi);
    const uint32_t ol = (uint32_t)dpp_i<CTRL, ROWS>((int)lo, (int)lo);
    const bool take = (oh > hi) | ((oh == hi) & (ol > lo));
    hi = take ? oh : hi;
    lo = take ? ol : lo;
}
__device__ __forceinline__ void wave_max2_u64(unsigned long long& x, unsigned long long& y) {
    uint32_t xh = (uint32_t)(x >> 32), xl = (uint32_t)x, yh = (uint32_t)(y >> 32), yl = (uint32_t)y;
    max_step_u64<kDppSwap1>(xh, xl);
    max_step_u64<kDppSwap1>(yh, yl);
    max_step_u64<kDppSwap2>(xh, xl);
    max_step_u64<kDppSwap2>(yh, yl);
    max_step_u64<kDppHalfMirror>(xh, xl);
    max_step_u64<kDppHalfMirror>(yh, yl);
    max_step_u64<kDppMirror>(xh, xl);
    max_step_u64<kDppMirror>(yh, yl);
    max_step_u64<kDppBcast15, 0xA>(xh, xl);
    max_step_u64<kDppBcast15, 0xA>(yh, yl);
    max_step_u64<kDppBcast31, 0xC>(xh, xl);
    max_step_u64<kDppBcast31, 0xC>(yh, yl);
    x = ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)xh, 63) << 32) |
        (uint32_t)__builtin_amdgcn_readlane((int)xl, 63);
    y = ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)yh, 63) << 32) |
        (uint32_t)__builtin_amdgcn_readlane((int)yl, 63);
}

// Race of one chunk: keys w_j / (-log2 U_j) (the keys w_j / E_j times ln 2, the same
// argmax) over this thread's ids, the wave's best packed winner of the weights w and of
// the fallback weights p (the race on p decides only where no residual weight is
// positive anywhere). zp: the penalized target row of the draw; xq: the draft row of a
// residual draw (kind 1), unused for a bonus draw (kind 2); onehot_d: the draft id of a
// one-hot proposal (q = 1 there, 0 elsewhere), or -1.
struct DrawSpec {
    int kind, pos;
    float m_p, m_q, cs;
    float inv_zp, inv_zq;
    int onehot_d;
};
// 1 / (-log2 U) of the thread's ids of the chunk at `base` for the draw at absolute position
// pos. The key words sit in vector registers (the kernel's scalar registers are taken, and
// scalar round keys would be spilled and reloaded).
__device__ __forceinline__ void race_variates(const SampArgs& a, int b, int base, int pos,
                                              float (&inv_e)[kEpt]) {
    const int tid = threadIdx.x;
    uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    asm volatile("" : "+v"(k0), "+v"(k1));
#pragma unroll
    for (int qd = 0; qd < kQuads; ++qd) {
        const RaceWords w = race_words4_k(k0, k1, base + 1024 * qd + 4 * tid, pos, b);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            inv_e[4 * qd + r] = __builtin_amdgcn_rcpf(race_e2(w.hi(r), w.lo(r)));
    }
}

// einv: this chunk's variates for the draw's position ([kEpt][kThreads] in LDS), or null
// to compute them here.
__device__ __forceinline__ void race_chunk_regs(const SampArgs& a, const DrawSpec& ds, int b,
                                                int base, const float (&zp)[kEpt],
                                                const float (&xq)[kEpt], const float* einv,
                                                unsigned long long* best_r,
                                                unsigned long long* best_p) {
    const int tid = threadIdx.x;
    // the weights p and w; the draw kind is uniform, so its tests sit outside the id loops
    float pw[kEpt], rw[kEpt];
#pragma unroll
    for (int e = 0; e < kEpt; ++e) pw[e] = __builtin_amdgcn_exp2f((zp[e] - ds.m_p) * ds.cs) * ds.inv_zp;
    if (ds.kind == 1 && ds.onehot_d >= 0) {
#pragma unroll
        for (int e = 0; e < kEpt; ++e)
            rw[e] = fmaxf(0.f, pw[e] - (elem_id(base, e) == ds.onehot_d ? 1.f : 0.f));
    } else if (ds.kind == 1) {
#pragma unroll
        for (int e = 0; e < kEpt; ++e)
            rw[e] = fmaxf(0.f, pw[e] - __builtin_amdgcn_exp2f((xq[e] - ds.m_q) * ds.cs) * ds.inv_zq);
    } else {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) rw[e] = pw[e];
    }
    // the variates of the thread's ids: from the table computed while waiting, or here
    float inv_e[kEpt];
    if (einv) {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) inv_e[e] = einv[e * kThreads + tid];
    } else {
        race_variates(a, b, base, ds.pos, inv_e);
    }
    float kr_best = 0.f, kp_best = 0.f;
    int jr = 0, jp = 0;
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        const int j = elem_id(base, e);
        const float kr = rw[e] * inv_e[e], kp = pw[e] * inv_e[e];
        // a thread visits its ids in increasing order, so a strict > keeps the lower id of a
        // tie; ids past the vocabulary hold -inf logits: weight 0, never a winner
        const bool ur = kr > kr_best, up = kp > kp_best;
        kr_best = ur ? kr : kr_best;
        jr = ur ? j : jr;
        kp_best = up ? kp : kp_best;
        jp = up ? j : jp;
    }
    unsigned long long r = kr_best > 0.f ? pack_key(kr_best, jr) : 0ull;
    unsigned long long p = kp_best > 0.f ? pack_key(kp_best, jp) : 0ull;
    wave_max2_u64(r, p);
    *best_r = r;
    *best_p = p;
}

__device__ __forceinline__ float uniform_f(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Folds the workgroup's race winners into the sequence's words (thread 0; the atomics are
// acknowledged before it returns).
__device__ __forceinline__ void publish_race(FusedShared& sh, const SeqState& st,
                                             unsigned long long br, unsigned long long bp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sh.win[wave] = br;
        sh.win[4 + wave] = bp;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long r = 0ull, p = 0ull;
        for (int w = 0; w < 4; ++w) {
            r = sh.win[w] > r ? sh.win[w] : r;
            p = sh.win[4 + w] > p ? sh.win[4 + w] : p;
        }
        // the fallback race on p only matters when no residual weight is positive anywhere
        if (r) atomicMax(st.Wr, r);
        else if (p) atomicMax(st.Wp, p);
        __builtin_amdgcn_s_waitcnt(0);
    }
}

// Thread 0 counts the workgroup into D; true in every thread of the one that completes it.
__device__ __forceinline__ bool count_done(FusedShared& sh, const SeqState& st, uint32_t total) {
    __syncthreads();
    if (threadIdx.x == 0) sh.flag = (int)(atomicAdd(st.D, 1u) == total - 1u);
    __syncthreads();
    return sh.flag != 0;
}

// Loads the chunk values the race of chunk c needs (an abandoned chunk's path): the penalized
// target row `a_rows` and draft row a_rows + 1.
template <bool VEC, bool MAP>
__device__ __forceinline__ void load_race_chunk(const SampArgs& a, const SeqMode& m, int b,
                                                int c, int arow,
                                const int* drafts, float (&zp)[kEpt], float (&xq)[kEpt],
                                bool want_q) {
    const int base = c * kChunk;
    int cnt[kEpt];
    load_counts<VEC>(a.counts ? a.counts + (size_t)b * a.vocab : nullptr, base, a.vocab, cnt);
    load_chunk<VEC>(a.tl + (size_t)(m.r0 + arow) * a.vocab, base, a.vocab, zp);
    if (want_q) load_draft_chunk<VEC, MAP>(a, m.d0 + arow, base, xq);
    else
#pragma unroll
        for (int e = 0; e < kEpt; ++e) xq[e] = 0.f;
    uint32_t dm[kEpt];
    draft_masks(drafts, arow, base, dm);
#pragma unroll
    for (int e = 0; e < kEpt; ++e) zp[e] = penalize(zp[e], cnt[e] + __popc(dm[e]), m.pp, m.fp);
}

// Phase 1 of the fused kernel for the data rows q0 .. q0 + kRowBatch - 1 (target rows
// 0 .. R - 1, then draft rows 1 .. K), whose chunk values are in xv: penalties (target rows),
// the statistics, the wave reduction, a partial per wave in LDS. A target row also yields its
// raw statistics (logprobs) from the values before its penalties, so raw rows are never
// loaded. Then the waves' partials are combined and each row's chunk entry is stored
// write-through. The statistics run G rows at a time in one straight-line block, so the
// rows' reduction chains (each a few dozen dependent steps) overlap; every row's own
// arithmetic is the same whatever the grouping.

// (max, sum 2^((x - max) c)) of rows u0 .. u0 + G - 1 into LDS slots slot0 + u
template <int G>
__device__ __forceinline__ void group_maxsum(FusedShared& sh, const float (&xv)[kRowBatch][kEpt],
                                             int u0, int slot0, float cs) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float mx[G], sm[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mx[g] = xv[u0 + g][0];
#pragma unroll
        for (int e = 1; e < kEpt; ++e) mx[g] = fmaxf(mx[g], xv[u0 + g][e]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) mx[g] = wave_max(mx[g]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        // a row with no ordered value (max -inf) sums to 0; the select keeps this block
        // free of branches
        const float mcs = mx[g] * cs;
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < kEpt; ++e) t += __builtin_amdgcn_exp2f(__builtin_fmaf(xv[u0 + g][e], cs, -mcs));
        sm[g] = mx[g] != kNegInf ? t : 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) sm[g] = wave_sum(sm[g]);
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) sh.part[slot0 + u0 + g][wave] = make_float4(mx[g], sm[g], 0.f, 0.f);
    }
}

// (max, id of the max) of rows u0 .. u0 + G - 1 into LDS slots u; ties go to the lower id
template <int G>
__device__ __forceinline__ void group_argmax(FusedShared& sh, const float (&xv)[kRowBatch][kEpt],
                                             int u0, int base) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float bv[G];
    int bi[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        // a thread visits its ids in increasing order, so a strict > keeps the lowest id of a
        // tie; ids past the vocabulary hold -inf and never replace the start
        bv[g] = kNegInf;
        bi[g] = kBigIdx;
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const bool up = xv[u0 + g][e] > bv[g];
            bv[g] = up ? xv[u0 + g][e] : bv[g];
            bi[g] = up ? elem_id(base, e) : bi[g];
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) wave_argmax(bv[g], bi[g]);
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
            sh.part[u0 + g][wave] = make_float4(bv[g], __int_as_float(bi[g]), 0.f, 0.f);
    }
}

// The statistics of rows 0 .. n - 1 of the batch (n uniform), four rows to a group.
__device__ __forceinline__ void batch_stats(FusedShared& sh, const float (&xv)[kRowBatch][kEpt],
                                            int n, bool argmax, int slot0, float cs, int base) {
#pragma unroll
    for (int u0 = 0; u0 < kRowBatch; u0 += 4) {
        if (u0 >= n) break;
        const int left = n - u0;
        if (argmax) {
            if (left >= 4) group_argmax<4>(sh, xv, u0, base);
            else if (left == 3) group_argmax<3>(sh, xv, u0, base);
            else if (left == 2) group_argmax<2>(sh, xv, u0, base);
            else group_argmax<1>(sh, xv, u0, base);
        } else {
            if (left >= 4) group_maxsum<4>(sh, xv, u0, slot0, cs);
            else if (left == 3) group_maxsum<3>(sh, xv, u0, slot0, cs);
            else if (left == 2) group_maxsum<2>(sh, xv, u0, slot0, cs);
            else group_maxsum<1>(sh, xv, u0, slot0, cs);
        }
    }
}

template <bool VEC, bool MAP>
__device__ __forceinline__ void process_batch(
    const SampArgs& a, const SeqMode& m, FusedShared& sh, float (&xv)[kRowBatch][kEpt],
    int q0, int ndata, int nd, float cs_t, bool has_pen, const int (&cnt)[kEpt],
    const uint32_t (&dm)[kEpt], uint32_t dmo, const float (&fpc)[kEpt],
    const float (&ppc)[kEpt], int base, int c) {
    const int tid = threadIdx.x;
    // rows of this batch, and how many of them are target rows (the first ones)
    const int nhere = min(kRowBatch, ndata - q0);
    const int ntg = max(0, min(nhere, m.rows - q0));
    // LDS partial slots: u for row q0 + u, kRowBatch + u for the raw row of target row q0 + u
    if (m.raw) batch_stats(sh, xv, ntg, false, kRowBatch, kLog2e, base);
    if (has_pen) {
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
            if (u >= ntg) continue;
            const uint32_t lm = low_bits(q0 + u);
            if (__ballot((dmo & lm) != 0u)) {
                // a draft of an earlier position is among this wave's ids
#pragma unroll
                for (int e = 0; e < kEpt; ++e)
                    xv[u][e] = penalize(xv[u][e], cnt[e] + __popc(dm[e] & lm), m.pp, m.fp);
            } else {
#pragma unroll
                for (int e = 0; e < kEpt; ++e)
                    xv[u][e] = __fsub_rn(__fsub_rn(xv[u][e], fpc[e]), ppc[e]);
            }
        }
    }
    // target rows of a greedy sequence: the argmax; every other row: (max, sum) (a greedy
    // sequence loads no draft rows)
    batch_stats(sh, xv, nhere, !m.sampled, 0, cs_t, base);
    __syncthreads();
    // combine the waves and store this chunk's entry of each row (and raw row), write-through
    for (int v = tid; v < 2 * kRowBatch; v += kThreads) {
        const int u = v < kRowBatch ? v : v - kRowBatch;
        const int q = q0 + u;
        const bool raw = v >= kRowBatch;
        if (q >= ndata || (raw && !(q < m.rows && m.raw))) continue;
        const RowRef r = row_ref(a, m, raw ? m.rows + nd + q : q);
        float2 out;
        if (!raw && r.kind == 0 && !m.sampled) {
            float bv = sh.part[v][0].x;
            int bi = __float_as_int(sh.part[v][0].y);
            for (int w = 1; w < 4; ++w)
                if (better(sh.part[v][w].x, __float_as_int(sh.part[v][w].y), bv, bi)) {
                    bv = sh.part[v][w].x;
                    bi = __float_as_int(sh.part[v][w].y);
                }
            out = make_float2(bv, __int_as_float(bi));
        } else {
            const float cs = raw ? kLog2e : cs_t;
            float mx = sh.part[v][0].x;
            for (int w = 1; w < 4; ++w) mx = fmaxf(mx, sh.part[v][w].x);
            float sm = 0.f;
            if (mx != kNegInf)
                for (int w = 0; w < 4; ++w)
                    if (sh.part[v][w].x != kNegInf)
                        sm += sh.part[v][w].y * exp2f((sh.part[v][w].x - mx) * cs);
            out = make_float2(mx, sm);
        }
        handoff_store(reinterpret_cast<float2*>(a.stats) + (size_t)r.slot * a.nchunk + c, out);
    }
}

// out = row u of the batch (u uniform), zeros when u is out of range: one branch, not a
// select per row
__device__ __forceinline__ void pick_row(const float (&xv)[kRowBatch][kEpt], int u,
                                         float (&out)[kEpt]) {
#pragma unroll
    for (int e = 0; e < kEpt; ++e) out[e] = 0.f;
    switch (u) {
#define VSA_PICK(n) \
    case n:         \
        _Pragma("unroll") for (int e = 0; e < kEpt; ++e) out[e] = xv[n][e]; \
        break;
        VSA_PICK(0) VSA_PICK(1) VSA_PICK(2) VSA_PICK(3) VSA_PICK(4) VSA_PICK(5)
        VSA_PICK(6) VSA_PICK(7) VSA_PICK(8) VSA_PICK(9) VSA_PICK(10) VSA_PICK(11)
#undef VSA_PICK
        default:
            break;
    }
}
static_assert(kRowBatch == 12, "pick_row covers the batch");

template <bool VEC, bool MAP>
__global__ __launch_bounds__(kThreads) void fused_kernel(const SampArgs a) {
    __shared__ FusedShared sh;
    preload_args(a);
    const int b = __builtin_amdgcn_readfirstlane(blockIdx.x / a.nchunk);
    const int c = __builtin_amdgcn_readfirstlane(blockIdx.x - b * a.nchunk);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int base = c * kChunk;
    // Load order matters (vector loads return in order): the sequence's geometry and
    // parameters, then the counts and the first batch of rows, then the draft ids, whose
    // wait thus never holds up the rows' requests.
    uint32_t ebits = 0;
    const SeqMode m = seq_mode(a, b, &ebits);
    int cnt[kEpt];
    load_counts<VEC>(a.counts ? a.counts + (size_t)b * a.vocab : nullptr, base, a.vocab, cnt);
    if (c == 0 && tid == 0 && ebits) atomicOr(a.err, ebits);
    if (!m.valid) return;
    const SeqState st = seq_state(a, b);
    const bool onehot = a.onehot != 0;
    const int nd = seq_ndraft(a, m);
    const int nrows = seq_nrows(a, m);         // the row list: target, draft, raw rows
    const int ndata = m.rows + nd;             // rows whose chunks are loaded
    const float cs_t = kLog2e / m.temp;        // target / draft rows of a sampled sequence
    int dreg = 0;
    bool valid_l = false;
    float pre_x = 0.f, pre_w = 0.f;
    int pre_c = 0;
    uint32_t dm[kEpt];
    uint32_t dmo = 0;
    const bool has_pen = m.pp != 0.f || m.fp != 0.f;
    float fpc[kEpt], ppc[kEpt];

    // ---- phase 1: per-row statistics of this chunk, kRowBatch rows at a time. The draft
    // ids come by scalar loads, which wait apart from the rows' vector loads: the draft
    // masks are ready while the rows still stream in.
    float xv[kRowBatch][kEpt];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u)
        if (u < ndata) load_row_chunk<VEC, MAP>(a, m, row_ref(a, m, u), base, xv[u]);
    scalar_drafts(a, m, m.k, base, sh.drafts, dm, dreg);
#pragma unroll
    for (int e = 0; e < kEpt; ++e) {
        dmo |= dm[e];
        fpc[e] = __fmul_rn(m.fp, (float)cnt[e]);
        ppc[e] = cnt[e] > 0 ? m.pp : 0.f;
    }
    // Per draft (wave 0, lane t - 1 for draft t): its target logit in row t - 1, its draft
    // logit in row t and its base count, for the acceptance test; requested now, used after
    // the arrival
    valid_l = wave == 0 && lane < m.k && dreg >= 0 && dreg < a.vocab;
    if (valid_l && (m.sampled || m.logprobs)) {
        pre_x = a.tl[(size_t)(m.r0 + lane) * a.vocab + dreg];
        if (m.sampled) {
            pre_c = a.counts ? a.counts[(size_t)b * a.vocab + dreg] : 0;
            if (!onehot) pre_w = draft_logit<MAP>(a, m.d0 + lane, dreg);
        }
    }
    process_batch<VEC, MAP>(a, m, sh, xv, 0, ndata, nd, cs_t, has_pen, cnt, dm, dmo, fpc, ppc,
                            base, c);
    for (int q0 = kRowBatch; q0 < ndata; q0 += kRowBatch) {
        __syncthreads();                                  // sh.part is reused
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u)
            if (q0 + u < ndata) load_row_chunk<VEC, MAP>(a, m, row_ref(a, m, q0 + u), base, xv[u]);
        process_batch<VEC, MAP>(a, m, sh, xv, q0, ndata, nd, cs_t, has_pen, cnt, dm, dmo, fpc,
                                ppc, base, c);
    }

    // ---- arrival
    int* const s_flag = &sh.flag;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) *s_flag = (int)(atomicAdd(st.A, 1u) == (uint32_t)a.nchunk - 1u);
    __syncthreads();
    const bool last = *s_flag != 0;
    if (!m.sampled && !last) return;
    DrawRec* const rec = reinterpret_cast<DrawRec*>(a.race + b);
    const int xq0 = m.rows + nd;                 // first raw row in the row list
    bool abandoned_final = false;                // this workgroup abandoned its chunk and
                                                 // then completed D
    int npre = 0;                                // positions whose variates are in sh.einv
    if (!last && m.k < kPrePos) {
        // While the last arriver decides: the race variates of every position the draw can
        // take (positions[b] + a, a the accepted drafts, 0 <= a <= K), one position at a
        // time, each followed by a look at the go flag (thread 0); the first look that finds
        // it set ends this.
        const int pos0 = a.positions[b];
        for (int pp = 0; pp <= m.k; ++pp) {
            float inv_e[kEpt];
            race_variates(a, b, base, pos0 + pp, inv_e);
#pragma unroll
            for (int e = 0; e < kEpt; ++e) sh.einv[pp][e][tid] = inv_e[e];
            if (tid == 0) sh.go_seen = (int)coh_load_u32(st.go);
            __syncthreads();
            npre = pp + 1;
            const int seen = sh.go_seen;
            __syncthreads();                             // sh.go_seen is rewritten next
            if (seen) break;
        }
    }
    if (!last) {
        // a sampled sequence's other workgroups: wait (bounded) for the decision, then load
        // the record; on a timeout the chunk is abandoned to whoever completes D
        if (tid == 0) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            int seen = 0;
            for (;;) {
                if (coh_load_u32(st.go) != 0u) { seen = 1; break; }
                if (__builtin_amdgcn_s_memrealtime() - t0 >= (uint64_t)a.wait_ticks) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (!seen) {
                atomicOr(a.err, VSA_DEVERR_WAIT_TIMEOUT);
                __hip_atomic_store(flag_at(a, st, c), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                atomicAdd(st.Ab, 1u);
                __builtin_amdgcn_s_waitcnt(0);
            }
            *s_flag = seen;
        }
        __syncthreads();
        if (*s_flag == 0) {
            // abandoned: count in; the workgroup completing D races the chunk
            if (!count_done(sh, st, (uint32_t)a.nchunk)) return;
            abandoned_final = true;
            if (tid < 7) {
                const float2 v = coh_load2(reinterpret_cast<const float2*>(rec) + tid);
                reinterpret_cast<float2*>(&sh.rec)[tid] = v;
            }
            __syncthreads();
        } else {
            if (tid < 7) {
                const float2 v = coh_load2(reinterpret_cast<const float2*>(rec) + tid);
                reinterpret_cast<float2*>(&sh.rec)[tid] = v;
            }
            __syncthreads();
        }
    } else {
        // ---- the last arriver: merge the chunk statistics of every row (one wave per row,
        //      up to 3 rows per wave in one round of coherent loads), decide, write the
        //      outputs and, for a sampled sequence, publish the decision
        for (int q0 = wave; q0 < nrows; q0 += 12) {
            float2 stv[3][kChunkLoads];
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                const int q = q0 + 4 * x;
                const RowRef r = row_ref(a, m, q < nrows ? q : 0);
#pragma unroll
                for (int u = 0; u < kChunkLoads; ++u) {
                    const int cc = lane + 64 * u;
                    stv[x][u] = (q < nrows && cc < a.nchunk)
                                    ? coh_load2(reinterpret_cast<const float2*>(a.stats) +
                                                (size_t)r.slot * a.nchunk + cc)
                                    : make_float2(kNegInf, __int_as_float(kBigIdx));
                }
            }
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                const int q = q0 + 4 * x;
                if (q >= nrows) break;
                const RowRef r = row_ref(a, m, q);
                if (r.kind == 0 && !m.sampled) {
                    float bv = kNegInf;
                    int bi = kBigIdx;
#pragma unroll
                    for (int u = 0; u < kChunkLoads; ++u) {
                        const int ci = __float_as_int(stv[x][u].y);
                        if (better(stv[x][u].x, ci, bv, bi)) { bv = stv[x][u].x; bi = ci; }
                    }
                    wave_argmax(bv, bi);
                    if (lane == 0) {
                        sh.rm[q] = bv;
                        sh.rarg[q] = bi;
                    }
                } else {
                    float mx;
                    double z;
                    merge_row_wave(stv[x], r.kind == 2 ? kLog2e : cs_t, &mx, &z);
                    if (lane == 0) {
                        sh.rm[q] = mx;
                        sh.rz[q] = z;
                    }
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            int acc;
            if (!m.sampled) {
                acc = 0;
                while (acc < m.k) {
                    const int d = sh.drafts[acc];
                    if (d != sh.rarg[acc]) break;
                    ++acc;
                }
            } else {
                // every draft's test at once: lane t - 1 holds draft t, p_{t-1}(d_t) and
                // q_t(d_t) (the race's exp2 over the merged normalizers, fp64 ratio) and u_t
                // from its stream
                bool ok = false;
                if (valid_l) {
                    int cd = pre_c;
                    for (int s2 = 0; s2 < lane; ++s2) cd += sh.drafts[s2] == dreg ? 1 : 0;
                    const float zt = penalize(pre_x, cd, m.pp, m.fp);
                    const double pd =
                        (double)__builtin_amdgcn_exp2f((zt - sh.rm[lane]) * cs_t) / sh.rz[lane];
                    const double qd =
                        onehot ? 1.0
                               : (double)__builtin_amdgcn_exp2f((pre_w - sh.rm[m.rows + lane]) * cs_t) /
                                     sh.rz[m.rows + lane];
                    ok = accept_uniform(a.seed, b, a.positions[b] + lane) * qd < pd;
                }
                const unsigned long long rej = __ballot(lane < m.k && !ok);
                acc = rej ? __ffsll(rej) - 1 : m.k;
            }
            if (__ballot(lane < m.k && lane <= acc && !(dreg >= 0 && dreg < a.vocab)) && lane == 0)
                atomicOr(a.err, VSA_DEVERR_DRAFT_ID);
            if (m.sampled && lane == 0) {
                DrawRec& d = sh.rec;
                d.kind = acc < m.k ? 1 : 2;
                d.acc = acc;
                d.pos = a.positions[b] + acc;
                d.onehot_d = (d.kind == 1 && onehot) ? sh.drafts[acc] : -1;
                d.m_p = sh.rm[acc];
                d.z_p = sh.rz[acc];
                d.m_q = (d.kind == 1 && !onehot) ? sh.rm[m.rows + acc] : 0.f;
                d.z_q = (d.kind == 1 && !onehot) ? sh.rz[m.rows + acc] : 1.0;
                d.m_x = m.raw ? sh.rm[xq0 + acc] : 0.f;
                d.z_x = m.raw ? sh.rz[xq0 + acc] : 1.0;
                d.pad = 0.f;
            }
            wave_sync();
            if (m.sampled && lane < 7) {
                // the record, write-through, then the go flag
                handoff_store(reinterpret_cast<float2*>(rec) + lane,
                              reinterpret_cast<const float2*>(&sh.rec)[lane]);
                __builtin_amdgcn_s_waitcnt(0);
            }
            wave_sync();
            if (m.sampled && lane == 0)
                __hip_atomic_store(st.go, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // outputs (every row but a sampled sequence's draw)
            if (lane == 0) a.accepted[b] = acc;
            for (int s = lane; s < m.rows; s += 64) {
                const int grow = m.r0 + s;
                int out = -1;
                if (s < acc) out = sh.drafts[s];
                else if (s == acc && !m.sampled) {
                    out = sh.rarg[acc];
                    if (out < 0 || out >= a.vocab) out = 0;   // a row with no ordered value
                }
                if (!(m.sampled && s == acc)) a.out_tokens[grow] = out;
                if (a.chosen_lp && !(m.sampled && s == acc)) {
                    float lpv = __builtin_nanf("");
                    if (m.logprobs && out >= 0) {
                        const float x = s < acc ? pre_x : a.tl[(size_t)grow * a.vocab + out];   // s == lane
                        lpv = (float)((double)x - (double)sh.rm[xq0 + s] - log(sh.rz[xq0 + s]));
                    }
                    a.chosen_lp[grow] = lpv;
                }
                if (a.diag_thr) a.diag_thr[grow] = m.sampled ? kNegInf : __builtin_nanf("");
                if (a.diag_kept) {
                    a.diag_kept[2 * grow] = m.sampled ? a.vocab : 0;
                    a.diag_kept[2 * grow + 1] = m.sampled ? a.vocab : 0;
                }
            }
        }
        if (!m.sampled) {
            if (tid == 0) __hip_atomic_store(st.A, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __syncthreads();
    }
    const DrawRec d = sh.rec;
    const int acc = __builtin_amdgcn_readfirstlane(d.acc);
    const int kind = __builtin_amdgcn_readfirstlane(d.kind);

    // ---- the draw: this chunk's race from the registers (or reloaded past one row batch)
    DrawSpec ds;
    ds.kind = kind;
    ds.pos = __builtin_amdgcn_readfirstlane(d.pos);
    ds.cs = cs_t;
    ds.m_p = uniform_f(d.m_p);
    ds.inv_zp = uniform_f((float)(1.0 / d.z_p));
    ds.onehot_d = __builtin_amdgcn_readfirstlane(d.onehot_d);
    ds.m_q = uniform_f(d.m_q);
    ds.inv_zq = uniform_f((float)(1.0 / d.z_q));
    float zp[kEpt], xq[kEpt];
    if (ndata <= kRowBatch) {
        pick_row(xv, acc, zp);
        pick_row(xv, (kind == 1 && nd > 0) ? m.rows + acc : -1, xq);
    } else {
        load_race_chunk<VEC, MAP>(a, m, b, c, acc, sh.drafts, zp, xq, kind == 1 && !onehot);
    }
    const uint32_t total = (uint32_t)a.nchunk;
    unsigned long long br, bp;
    bool final_wg = abandoned_final;
    if (!abandoned_final) {
        race_chunk_regs(a, ds, b, base, zp, xq, acc < npre ? &sh.einv[acc][0][0] : nullptr, &br,
                        &bp);
        publish_race(sh, st, br, bp);
        final_wg = count_done(sh, st, total);
    }
    if (!final_wg) return;

    // ---- D is complete: every other workgroup of the sequence is done with its state.
    //      The abandoned chunks (if any), then the token, its logprob, and the state back
    //      to zero.
    if (coh_load_u32(st.Ab) != 0u) {
        for (int cc = tid; cc < a.nchunk; cc += kThreads) {
            uint32_t* f = flag_at(a, st, cc);
            sh.state[cc] = coh_load_u32(f);
            if (sh.state[cc]) __hip_atomic_store(f, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        for (int cc = 0; cc < a.nchunk; ++cc) {
            if (sh.state[cc] == 0u) continue;
            float zr[kEpt], qr[kEpt];
            load_race_chunk<VEC, MAP>(a, m, b, cc, acc, sh.drafts, zr, qr, kind == 1 && !onehot);
            race_chunk_regs(a, ds, b, cc * kChunk, zr, qr, nullptr, &br, &bp);
            publish_race(sh, st, br, bp);
        }
    }
    if (tid != 0) return;
    const unsigned long long wr = coh_load_u64(st.Wr), wp = coh_load_u64(st.Wp);
    int tok = wr ? packed_id(wr) : (wp ? packed_id(wp) : 0);
    if (tok < 0 || tok >= a.vocab) tok = 0;
    const int grow = m.r0 + acc;
    a.out_tokens[grow] = tok;
    if (a.chosen_lp) {
        float lpv = __builtin_nanf("");
        if (m.logprobs)
            lpv = (float)((double)a.tl[(size_t)grow * a.vocab + tok] - (double)d.m_x - log(d.z_x));
        a.chosen_lp[grow] = lpv;
    }
    __hip_atomic_store(st.Wr, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(st.Wp, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(st.go, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(st.Ab, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(st.D, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(st.A, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// Workgroups of the fused kernel the device holds at once (cached per device).
static int fused_capacity(bool vec, bool map) {
    static int cache[2][2][64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int& c = cache[vec ? 1 : 0][map ? 1 : 0][dev];
    if (c == 0) {
        int per_cu = 0, cus = 0;
        const void* k =
            map ? (vec ? reinterpret_cast<const void*>(&fused_kernel<true, true>)
                       : reinterpret_cast<const void*>(&fused_kernel<false, true>))
                : (vec ? reinterpret_cast<const void*>(&fused_kernel<true, false>)
                       : reinterpret_cast<const void*>(&fused_kernel<false, false>));
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            per_cu = cus = 0;
        c = per_cu * cus > 0 ? per_cu * cus : -1;
    }
    return c;
}

bool fused_fits(const SampArgs& a) {
    const bool vec = (a.vocab % 4) == 0;
    const bool map = a.t2d != nullptr;
    // abandon flags: (batch x nchunk) over the kCtrLines - 4B lines past the hot ones, at
    // most 60 to a line (words 1..60; word 0 of those lines stays free)
    return a.max_top_k == 0 && a.max_top_lp == 0 && a.batch <= kFusedMaxBatch &&
           (long)a.batch * a.nchunk <= 60L * (kCtrLines - 4L * a.batch) &&
           (long)a.batch * a.nchunk <= (long)fused_capacity(vec, map);
}

hipError_t launch_fused(const SampArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.batch * a.nchunk), block(kThreads);
    const bool vec = (a.vocab % 4) == 0;
    if (a.t2d) {
        if (vec) hipLaunchKernelGGL((fused_kernel<true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((fused_kernel<false, true>), grid, block, 0, stream, a);
    } else {
        if (vec) hipLaunchKernelGGL((fused_kernel<true, false>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((fused_kernel<false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace vsa
