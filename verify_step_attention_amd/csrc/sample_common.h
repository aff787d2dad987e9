// Device pieces shared by the vocabulary-stage kernels (sample_fused.hip, sample_accept.hip).
//
// Pages (mlx-dspark): penalties per verify position from base counts plus the position's
// own draft prefix (Changelog [0.2.0] "Added"); truncation of draft and target and exact
// target samples (release v0.1.0 and v0.0.2, "Highlights").
// Random numbers: Philox4x32-10 (Salmon et al., SC'11), key = seed, counter
// (block, position, sequence, tag). Acceptance uniform: block 0, tag 0, words (x, y).
// Race variates of token id j: block j >> 1, tag 1, words (2 (j & 1), 2 (j & 1) + 1).
// Both are 64-bit uniforms on the open interval, U = (hi 2^32 + lo + 1/2) 2^-64.
#pragma once

#include <math.h>

#include "vsa_internal.h"

namespace vsa {
namespace samp {

constexpr int kThreads = 256;
constexpr int kEpt = kChunk / kThreads;        // ids per thread per chunk (8)
constexpr int kQuads = kChunk / 1024;          // float4 groups per thread per chunk
constexpr float kNegInf = -__builtin_inff();
constexpr int kBigIdx = 0x7FFFFFFF;
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kTwoM32 = 2.3283064365386963e-10;   // 2^-32

// ------------------------------------------------------------------ Philox4x32-10
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // each 32 x 32 -> 64-bit product in one instruction (v_mad_u64_u32)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1,
                       (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
    }
    return c;
}

__device__ __forceinline__ uint4 philox_block(uint64_t seed, uint32_t block, uint32_t pos,
                                              uint32_t seq, uint32_t tag) {
    return philox4x32_10(make_uint4(block, pos, seq, tag), (uint32_t)seed,
                         (uint32_t)(seed >> 32));
}

// U = (hi 2^32 + lo + 1/2) 2^-64 in fp64: the sum rounds once, the scalings are exact.
__device__ __forceinline__ double uniform64(uint32_t hi, uint32_t lo) {
    return ((double)hi + ((double)lo + 0.5) * kTwoM32) * kTwoM32;
}

// The acceptance uniform of the draft at absolute position `pos` of sequence b.
__device__ __forceinline__ double accept_uniform(uint64_t seed, int b, int pos) {
    const uint4 w = philox_block(seed, 0u, (uint32_t)pos, (uint32_t)b, 0u);
    return uniform64(w.x, w.y);
}

// E = -ln U of a race variate in fp64 (kept-list races): -ln U while U < 1/2, else
// -log1p(-c) with c = 1 - U from the complemented words (exact in real arithmetic).
__device__ __forceinline__ double race_e64(uint32_t hi, uint32_t lo) {
    if (hi < 0x80000000u) return -log(uniform64(hi, lo));
    return -log1p(-uniform64(~hi, ~lo));
}

// -log2 U of a race variate in fp32 (full-vocabulary races; the keys w / (-log2 U) are the
// keys w / E times ln 2, the same argmax). Relative error a few fp32 ulps: U (or its
// complement c) rounds once to fp32 and v_log_f32 is about one ulp; near U = 1 the
// complement goes through -log2(1 - c) = -log2(w) c / (1 - w) with w = fl(1 - c), whose
// 1 - w is exact (the quotient by the hardware reciprocal, one more ulp). Branch-free: one
// logarithm per id.
__device__ __forceinline__ float race_e2(uint32_t hi, uint32_t lo) {
    constexpr float k2m32 = 2.3283064365386963e-10f;
    const bool low = hi < 0x80000000u;
    const uint32_t h = low ? hi : ~hi, l = low ? lo : ~lo;
    const float v = ((float)h + ((float)l + 0.5f) * k2m32) * k2m32;   // U, or c = 1 - U
    const float w = low ? v : 1.0f - v;
    float lg = -__builtin_amdgcn_logf(w);
    float hi_c = lg * (v * __builtin_amdgcn_rcpf(1.0f - w));
    float one_c = v * kLog2e;
    // every candidate on every lane, so the selects below stay selects (no divergent branch)
    asm volatile("" : "+v"(lg), "+v"(hi_c), "+v"(one_c));
    return low ? lg : (w == 1.0f ? one_c : hi_c);
}

// Race words of ids 4 i .. 4 i + 3 (blocks 2 i and 2 i + 1): (hi, lo) of id 4 i + r.
struct RaceWords {
    uint4 a, b;
    __device__ __forceinline__ uint32_t hi(int r) const {
        return r == 0 ? a.x : r == 1 ? a.z : r == 2 ? b.x : b.z;
    }
    __device__ __forceinline__ uint32_t lo(int r) const {
        return r == 0 ? a.y : r == 1 ? a.w : r == 2 ? b.y : b.w;
    }
};
__device__ __forceinline__ RaceWords race_words4(uint64_t seed, int j0, int pos, int b) {
    RaceWords w;
    w.a = philox_block(seed, (uint32_t)j0 >> 1, (uint32_t)pos, (uint32_t)b, 1u);
    w.b = philox_block(seed, ((uint32_t)j0 >> 1) + 1u, (uint32_t)pos, (uint32_t)b, 1u);
    return w;
}
// The same words with the key halves (k0, k1) = (low, high word of the seed) passed in, e.g.
// held in vector registers so that the round keys need no scalar registers.
__device__ __forceinline__ RaceWords race_words4_k(uint32_t k0, uint32_t k1, int j0, int pos,
                                                   int b) {
    RaceWords w;
    w.a = philox4x32_10(make_uint4((uint32_t)j0 >> 1, (uint32_t)pos, (uint32_t)b, 1u), k0, k1);
    w.b = philox4x32_10(make_uint4(((uint32_t)j0 >> 1) + 1u, (uint32_t)pos, (uint32_t)b, 1u), k0, k1);
    return w;
}

// ------------------------------------------------------------------ values and keys
// order-preserving map float -> uint32 (larger float, larger key); -0 is folded into +0
__device__ __forceinline__ uint32_t ord_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// z = (x - fp * c) - pp * [c > 0], each operation rounded once (no contraction)
__device__ __forceinline__ float penalize(float x, int c, float pp, float fp) {
    const float z = __fsub_rn(x, __fmul_rn(fp, (float)c));
    return __fsub_rn(z, c > 0 ? pp : 0.f);
}

// exp((v - vmax) / T) in fp64, the probability weight of the definition (unnormalized)
__device__ __forceinline__ double weight64(float v, float vmax, float temp) {
    if (v == kNegInf) return 0.0;
    return exp(((double)v - (double)vmax) / (double)temp);
}

// Nucleus rows without top-k: mass e^((v - vmax) / T) with the exponent in fp64 and split
// into integer and fraction, only 2^f (0 <= f < 1) from the fp32 hardware power, so the
// relative error (~1e-7) does not grow with the distance to the maximum.
__device__ __forceinline__ double nuc_mass(float v, float vmax, float temp) {
    if (v == kNegInf) return 0.0;
    double t = ((double)v - (double)vmax) * (1.4426950408889634 / (double)temp);
    if (!(t > -1100.0)) return 0.0;                  // NaN or below every double
    if (!(t <= 0.0)) t = 0.0;                        // v <= vmax
    const double n = floor(t);
    return ldexp((double)__builtin_amdgcn_exp2f((float)(t - n)), (int)n);
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return (v > bv) | ((v == bv) & (i < bi));
}

// A race winner packed for a 64-bit atomic max: the key's bits (positive floats order as
// their bits) above the complement of the id, so equal keys go to the lower id.
__device__ __forceinline__ unsigned long long pack_key(float key, int id) {
    return ((unsigned long long)__float_as_uint(key) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int packed_id(unsigned long long w) {
    return (int)(0xFFFFFFFFu - (uint32_t)(w & 0xFFFFFFFFull));
}

// ------------------------------------------------------------------ per-sequence mode
struct SeqMode {
    int r0, rows, k, d0;
    bool valid, sampled, topk, raw;
    bool nucleus;    // sampled, top_p < 1 without top-k: full-vocabulary nucleus rows
    int ntop, topk_k, logprobs;
    float temp, top_p, pp, fp;
};

__device__ __forceinline__ SeqMode seq_mode(const SampArgs& a, int b, uint32_t* errbits) {
    SeqMode m{};
    // the row range and the parameters are requested together (b < B: both in bounds)
    const int c0 = a.cu_rows[b], c1 = a.cu_rows[b + 1];
    const vsa_row_params p = a.params[b];
    m.r0 = c0;
    m.rows = c1 - c0;
    m.k = m.rows - 1;
    m.d0 = m.r0 - b;
    m.valid = m.rows >= 1 && m.rows <= a.max_rows && m.r0 >= 0 &&
              m.r0 + m.rows <= a.total_rows && m.d0 >= 0 &&
              m.d0 + m.k <= a.total_rows - a.batch;
    if (!m.valid) {
        *errbits |= VSA_DEVERR_SEQ_SHAPE;
        return m;
    }
    const bool bad = !(p.temperature >= 0.f) || !isfinite(p.temperature) || p.top_k < 0 ||
                     p.top_k > a.max_top_k || !(p.top_p > 0.f && p.top_p <= 1.f) ||
                     p.top_logprobs < 0 || p.top_logprobs > a.max_top_lp ||
                     (p.top_p < 1.f && p.temperature > 0.f &&
                      !(p.top_k > 0 && p.top_k < a.vocab) && a.max_top_k == 0);
    if (bad) *errbits |= VSA_DEVERR_PARAMS;
    m.temp = p.temperature;
    m.sampled = !bad && p.temperature > 0.f;
    if (m.sampled && m.k > 0 && a.dl == nullptr && !a.onehot) {
        *errbits |= VSA_DEVERR_NO_DRAFT_LOGITS;
        m.sampled = false;
    }
    m.topk = m.sampled && p.top_k > 0 && p.top_k < a.vocab;
    m.nucleus = m.sampled && !m.topk && p.top_p < 1.f;
    m.topk_k = p.top_k;
    m.top_p = p.top_p;
    m.pp = p.presence_penalty;
    m.fp = p.frequency_penalty;
    m.logprobs = bad ? 0 : p.logprobs;
    m.ntop = bad ? 0 : p.top_logprobs;
    m.raw = (m.logprobs != 0) || m.ntop > 0;
    return m;
}

// Row q of a sequence's row list: target rows, then draft rows (sampled, unless the
// proposals are one-hot: those have no rows), then raw rows.
struct RowRef {
    int kind;   // 0 target, 1 draft, 2 raw
    int i;      // target / raw: row 0..R-1; draft: t = 1..K
    int slot;   // workspace slot
};

__device__ __forceinline__ int seq_ndraft(const SampArgs& a, const SeqMode& m) {
    return (m.sampled && !a.onehot) ? m.k : 0;
}
__device__ __forceinline__ int seq_nrows(const SampArgs& a, const SeqMode& m) {
    return m.rows + seq_ndraft(a, m) + (m.raw ? m.rows : 0);
}

__device__ __forceinline__ RowRef row_ref(const SampArgs& a, const SeqMode& m, int q) {
    RowRef r;
    const int nd = seq_ndraft(a, m);
    if (q < m.rows) {
        r.kind = 0;
        r.i = q;
        r.slot = m.r0 + q;
    } else if (q < m.rows + nd) {
        r.kind = 1;
        r.i = q - m.rows + 1;
        r.slot = a.total_rows + m.d0 + r.i - 1;
    } else {
        r.kind = 2;
        r.i = q - m.rows - nd;
        r.slot = 2 * a.total_rows - a.batch + m.r0 + r.i;
    }
    return r;
}

// ------------------------------------------------------------------ chunk loads
// 16-byte loads that bypass the caches' retention (each logit and count is read once).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt4(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ int4 load_nt4(const int32_t* p) {
    const i32x4 v = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
    return make_int4(v[0], v[1], v[2], v[3]);
}

// NT: streaming loads (the nontemporal policy) for rows read once; plain loads for rows
// read again shortly (they stay in L2).
template <bool VEC, bool NT = true>
__device__ __forceinline__ void load_chunk(const float* row, int base, int vocab,
                                           float (&x)[kEpt]) {
    const int tid = threadIdx.x;
    if (VEC) {
#pragma unroll
        for (int q = 0; q < kQuads; ++q) {
            const int j = base + 1024 * q + 4 * tid;
            float4 v = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
            if (j < vocab) v = NT ? load_nt4(row + j) : *reinterpret_cast<const float4*>(row + j);
            x[4 * q] = v.x;
            x[4 * q + 1] = v.y;
            x[4 * q + 2] = v.z;
            x[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const int j = base + 1024 * (e >> 2) + 4 * tid + (e & 3);
            x[e] = j < vocab ? row[j] : kNegInf;
        }
    }
}

// A draft row's logits at the chunk's target ids. With a reduced draft vocabulary
// (mlx-dspark Changelog [0.8.0] "Added": draft id j stands for target id j + d2t[j], and
// the draft distribution is widened onto the target vocabulary before the accept test)
// a target id takes the logit of its draft id through the inverse table t2d, and -inf
// (probability 0) when no draft id maps to it; an entry outside [-1, dvocab) reads as
// -inf and sets VSA_DEVERR_DRAFT_MAP.
__device__ __forceinline__ float mapped_logit(const SampArgs& a, const float* row, int m,
                                              uint32_t* ebits) {
    if ((uint32_t)m < (uint32_t)a.dvocab) return row[m];
    if (m != -1) *ebits |= VSA_DEVERR_DRAFT_MAP;
    return kNegInf;
}
// MAP: the call has a reduced draft vocabulary (kernels are compiled both ways, so the
// full-vocabulary path carries none of this).
template <bool VEC, bool MAP, bool NT = true>
__device__ __forceinline__ void load_draft_chunk(const SampArgs& a, int drow, int base,
                                                 float (&x)[kEpt]) {
    if constexpr (!MAP) {
        load_chunk<VEC, NT>(a.dl + (size_t)drow * a.vocab, base, a.vocab, x);
        return;
    }
    const float* row = a.dl + (size_t)drow * a.dvocab;
    const int tid = threadIdx.x;
    int map[kEpt];
    if (VEC) {
#pragma unroll
        for (int q = 0; q < kQuads; ++q) {
            const int j = base + 1024 * q + 4 * tid;
            int4 v = make_int4(-1, -1, -1, -1);
            if (j < a.vocab) v = *reinterpret_cast<const int4*>(a.t2d + j);
            map[4 * q] = v.x;
            map[4 * q + 1] = v.y;
            map[4 * q + 2] = v.z;
            map[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const int j = base + 1024 * (e >> 2) + 4 * tid + (e & 3);
            map[e] = j < a.vocab ? a.t2d[j] : -1;
        }
    }
    uint32_t ebits = 0;
#pragma unroll
    for (int e = 0; e < kEpt; ++e) x[e] = mapped_logit(a, row, map[e], &ebits);
    if (ebits) atomicOr(a.err, ebits);
}
// The draft logit of target id `id` in draft row drow (id inside [0, V)).
template <bool MAP>
__device__ __forceinline__ float draft_logit(const SampArgs& a, int drow, int id) {
    if constexpr (!MAP) return a.dl[(size_t)drow * a.vocab + id];
    const float* row = a.dl + (size_t)drow * a.dvocab;
    uint32_t ebits = 0;
    const float v = mapped_logit(a, row, a.t2d[id], &ebits);
    if (ebits) atomicOr(a.err, ebits);
    return v;
}
// Row q of a sequence's row list (target, draft or raw) at the chunk's ids.
template <bool VEC, bool MAP, bool NT = true>
__device__ __forceinline__ void load_row_chunk(const SampArgs& a, const SeqMode& m,
                                               const RowRef& r, int base, float (&x)[kEpt]) {
    if constexpr (!MAP) {
        // one load path for every row kind: only the row's address differs
        const float* row = r.kind == 1 ? a.dl + (size_t)(m.d0 + r.i - 1) * a.vocab
                                       : a.tl + (size_t)(m.r0 + r.i) * a.vocab;
        load_chunk<VEC, NT>(row, base, a.vocab, x);
    } else {
        if (r.kind == 1) load_draft_chunk<VEC, MAP, NT>(a, m.d0 + r.i - 1, base, x);
        else load_chunk<VEC, NT>(a.tl + (size_t)(m.r0 + r.i) * a.vocab, base, a.vocab, x);
    }
}

template <bool VEC>
__device__ __forceinline__ void load_counts(const int32_t* row, int base, int vocab,
                                            int (&c)[kEpt]) {
    const int tid = threadIdx.x;
    if (row == nullptr) {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) c[e] = 0;
        return;
    }
    if (VEC) {
#pragma unroll
        for (int q = 0; q < kQuads; ++q) {
            const int j = base + 1024 * q + 4 * tid;
            int4 v = make_int4(0, 0, 0, 0);
            if (j < vocab) v = load_nt4(row + j);
            c[4 * q] = v.x;
            c[4 * q + 1] = v.y;
            c[4 * q + 2] = v.z;
            c[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            const int j = base + 1024 * (e >> 2) + 4 * tid + (e & 3);
            c[e] = j < vocab ? row[j] : 0;
        }
    }
}

__device__ __forceinline__ int elem_id(int base, int e) {
    return base + 1024 * (e >> 2) + 4 * (int)threadIdx.x + (e & 3);
}

// Per id of this thread: bit t set when draft t + 1 equals the id (the penalty count at
// target row i is then the base count plus popcount(mask & (2^i - 1))).
__device__ __forceinline__ void draft_masks(const int* s_draft, int k, int base,
                                            uint32_t (&dm)[kEpt]) {
#pragma unroll
    for (int e = 0; e < kEpt; ++e) dm[e] = 0u;
    for (int t = 0; t < k; ++t) {
        const int off = s_draft[t] - base;
        if (off >= 0 && off < kChunk && ((off & 1023) >> 2) == (int)threadIdx.x) {
            const int ee = (off >> 10) * 4 + (off & 3);
#pragma unroll
            for (int e = 0; e < kEpt; ++e) dm[e] |= (e == ee) ? (1u << t) : 0u;
        }
    }
}

// The draft ids of sequence m by scalar loads (read-only input, so the constant address
// space): those wait apart from the vector loads of the rows issued before, which return
// in issue order. Computes what draft_masks computes over the first n drafts (dm), stores
// the k ids in lds (thread 0; read after the next barrier) and gives lane t of wave 0 the
// id of draft t + 1 (dreg).
__device__ __forceinline__ void scalar_drafts(const SampArgs& a, const SeqMode& m, int n,
                                              int base, int* lds, uint32_t (&dm)[kEpt],
                                              int& dreg) {
    typedef __attribute__((address_space(4))) const int const_int;
    const const_int* dp = (const const_int*)(a.drafts + m.d0);
#pragma unroll
    for (int e = 0; e < kEpt; ++e) dm[e] = 0u;
    for (int t = 0; t < m.k; ++t) {
        const int d = dp[t];
        if (threadIdx.x == 0) lds[t] = d;
        if ((int)threadIdx.x == t) dreg = d;
        const int off = d - base;
        if (t < n && off >= 0 && off < kChunk && ((off & 1023) >> 2) == (int)threadIdx.x) {
            const int ee = (off >> 10) * 4 + (off & 3);
#pragma unroll
            for (int e = 0; e < kEpt; ++e) dm[e] |= (e == ee) ? (1u << t) : 0u;
        }
    }
}

__device__ __forceinline__ uint32_t low_bits(int i) { return i >= 32 ? ~0u : (1u << i) - 1u; }

// (max, normalizer) of a softmax row from its per-chunk (max, sum) entries, one wave: lane
// holds entries lane, lane + 64, ... Every caller uses this same order of operations, so
// every workgroup that merges a row gets the same bits.
__device__ __forceinline__ void merge_row_wave(const float2 (&st)[kChunkLoads], float cs,
                                               float* m_out, double* z_out) {
    float bm = kNegInf;
#pragma unroll
    for (int u = 0; u < kChunkLoads; ++u) bm = fmaxf(bm, st[u].x);
    bm = wave_max(bm);
    // normalizer sum_j 2^((v_j - m) c) over the row, c = log2(e) / T (raw: T = 1)
    double z = 0.0;
    if (bm != kNegInf) {
#pragma unroll
        for (int u = 0; u < kChunkLoads; ++u)
            if (st[u].x != kNegInf) z += (double)st[u].y * (double)exp2f((st[u].x - bm) * cs);
        z = wave_sum_f64(z);
    }
    *m_out = bm;
    *z_out = z;
}

}  // namespace samp
}  // namespace vsa
