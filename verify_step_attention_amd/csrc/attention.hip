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

namespace vsa {

namespace {

constexpr float kNegInf = -__builtin_inff();

#ifndef VSA_ATTN_TARGET_WGS
#define VSA_ATTN_TARGET_WGS 256      // workgroups the key split aims for (one per CU)
#endif
constexpr int kMaxSplits = 32;       // key splits per (sequence, KV head)
constexpr int kMergeGroup = 8;       // splits whose partials the merge loads in one round

// Block index -> (unit, split). Consecutive block ids go to different XCDs (round-robin
// dispatch), so units are dealt out across XCDs and all splits of one unit land on one XCD,
// where the partial states merged at the end stay in that XCD's L2.
__device__ __forceinline__ void map_block(int bid, int units, int nsplit, int* unit,
                                          int* split) {
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    *unit = (slot / nsplit) * 8 + xcd;
    *split = slot % nsplit;
}

struct SeqGeom {
    int r0, rows, ctx;
    bool ok;
};

__device__ __forceinline__ SeqGeom seq_geometry(const AttnArgs& a, int b, bool report) {
    SeqGeom s;
    s.r0 = a.cu_rows[b];
    s.rows = a.cu_rows[b + 1] - s.r0;
    s.ctx = a.ctx_lens[b];
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

// The last split of a unit to finish merges every split's (max, sum, O):
//   out = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s,   m = max_s m_s.
// Partials arrive through the fence-free hand-off (agent-scope loads, which go to the
// device-coherent level), so each round trip is expensive: a thread issues the (max, sum)
// and O loads of every split for all of its output slices in one round, then computes.
// Empty splits publish m = -inf, l = 0 and O = 0, so no load depends on another.
template <int D>
__device__ void attn_merge(const AttnArgs& a, int unit, int g, const SeqGeom& s) {
    constexpr int D4 = D / 4;
    constexpr int EPT = 2;                                   // output float4s per thread
    constexpr int SG = kMergeGroup;                          // splits per round of loads
    const int M = s.rows * a.group;
    const int ns = a.nsplit;
    const size_t base = (size_t)unit * ns;
    const size_t stride = (size_t)a.mcap * D4;               // float4s between splits
    for (int e0 = threadIdx.x; e0 < M * D4; e0 += EPT * blockDim.x) {
        float rm[EPT], rl[EPT];
        float4 racc[EPT];
#pragma unroll
        for (int x = 0; x < EPT; ++x) {
            rm[x] = kNegInf;
            rl[x] = 0.f;
            racc[x] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int s0 = 0; s0 < ns; s0 += SG) {
            float2 ml[EPT][SG];
            float4 v[EPT][SG];
#pragma unroll
            for (int x = 0; x < EPT; ++x) {
                const int e = e0 + x * blockDim.x;
                const int n = e / D4, d4 = e % D4;
                const bool live = e < M * D4;
                const float4* src =
                    reinterpret_cast<const float4*>(a.part_o) + (base * a.mcap + n) * D4 + d4;
#pragma unroll
                for (int u = 0; u < SG; ++u) {
                    const int sp = s0 + u;
                    const bool use = live && sp < ns;
                    ml[x][u] = use ? handoff_load(a.part_ml + (base + sp) * a.mcap + n)
                                   : make_float2(kNegInf, 0.f);
                    v[x][u] = use ? handoff_load4(src + (size_t)sp * stride)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
#pragma unroll
            for (int x = 0; x < EPT; ++x) {
                float m = rm[x];
#pragma unroll
                for (int u = 0; u < SG; ++u) m = fmaxf(m, ml[x][u].x);
                if (m == kNegInf) continue;
                const float c = exp2f(rm[x] - m);            // rescale the running state
                float l = rl[x] * c;
                float4 acc = make_float4(racc[x].x * c, racc[x].y * c, racc[x].z * c,
                                         racc[x].w * c);
#pragma unroll
                for (int u = 0; u < SG; ++u) {
                    const float f = (ml[x][u].x == kNegInf) ? 0.f : exp2f(ml[x][u].x - m);
                    l += f * ml[x][u].y;
                    acc.x += f * v[x][u].x;
                    acc.y += f * v[x][u].y;
                    acc.z += f * v[x][u].z;
                    acc.w += f * v[x][u].w;
                }
                rm[x] = m;
                rl[x] = l;
                racc[x] = acc;
            }
        }
#pragma unroll
        for (int x = 0; x < EPT; ++x) {
            const int e = e0 + x * blockDim.x;
            if (e >= M * D4) break;
            const int n = e / D4, d4 = e % D4;
            const float inv = 1.f / rl[x];
            const int row = s.r0 + n / a.group, head = g * a.group + n % a.group;
            *reinterpret_cast<float4*>(a.out + ((size_t)row * a.hq + head) * D + 4 * d4) =
                make_float4(racc[x].x * inv, racc[x].y * inv, racc[x].z * inv,
                            racc[x].w * inv);
        }
    }
}

// Combines the key groups of one workgroup and writes either the final output (single
// split) or this split's partial state.
//   obuf[(kg * MC + n) * D + d]  unnormalized O of key group kg (relative to its own max)
//   gm[kg * MC + n], gl[...]     that group's running max (log2 units) and sum
// with gm = obuf + KGX * MC * D and gl = gm + KGX * MC.
template <int D, int KGX>
__device__ void attn_epilogue(const AttnArgs& a, char* smem, int unit, int split, int g,
                              const SeqGeom& s, int MC) {
    const int tid = threadIdx.x;
    const int M = s.rows * a.group;
    float* obuf = reinterpret_cast<float*>(smem);
    float* gm = obuf + KGX * MC * D;
    float* gl = gm + KGX * MC;
    float* fac = gl + KGX * MC;          // [KGX][MC] factor 2^(m_kg - m_wg)
    float* wm = fac + KGX * MC;          // [MC] workgroup max
    float* wl = wm + MC;                 // [MC] workgroup sum

    for (int n = tid; n < M; n += blockDim.x) {
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

    if (a.nsplit == 1) {
        for (int e = tid; e < M * D; e += blockDim.x) {
            const int n = e / D, d = e % D;
            float o = 0.f;
            for (int k = 0; k < KGX; ++k) o += fac[k * MC + n] * obuf[(k * MC + n) * D + d];
            const int row = s.r0 + n / a.group, head = g * a.group + n % a.group;
            a.out[((size_t)row * a.hq + head) * D + d] = o / wl[n];
        }
        return;
    }
    const size_t pslot = (size_t)unit * a.nsplit + split;
    for (int e = tid; e < M * (D / 4); e += blockDim.x) {
        const int n = e / (D / 4), d = 4 * (e % (D / 4));
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k = 0; k < KGX; ++k) {
            const float f = fac[k * MC + n];
            const float4 v = *reinterpret_cast<const float4*>(obuf + (k * MC + n) * D + d);
            o.x += f * v.x;
            o.y += f * v.y;
            o.z += f * v.z;
            o.w += f * v.w;
        }
        handoff_store4(reinterpret_cast<float4*>(a.part_o + (pslot * a.mcap + n) * D + d), o);
    }
    for (int n = tid; n < M; n += blockDim.x)
        handoff_store(a.part_ml + pslot * a.mcap + n, make_float2(wm[n], wl[n]));
    __shared__ int s_last;
    if (handoff_arrive(a.counters + unit, (uint32_t)a.nsplit, &s_last))
        attn_merge<D>(a, unit, g, s);
}

// A split that owns no tile publishes an empty state (m = -inf, l = 0, O = 0), which
// adds nothing in the merge, and still counts its arrival.
template <int D>
__device__ void attn_empty_split(const AttnArgs& a, int unit, int split, int g,
                                 const SeqGeom& s) {
    const int M = s.rows * a.group;
    const size_t pslot = (size_t)unit * a.nsplit + split;
    for (int e = threadIdx.x; e < M * (D / 4); e += blockDim.x)
        handoff_store4(reinterpret_cast<float4*>(a.part_o + (pslot * a.mcap) * D) + e,
                       make_float4(0.f, 0.f, 0.f, 0.f));
    for (int n = threadIdx.x; n < M; n += blockDim.x)
        handoff_store(a.part_ml + pslot * a.mcap + n, make_float2(kNegInf, 0.f));
    __shared__ int s_last;
    if (handoff_arrive(a.counters + unit, (uint32_t)a.nsplit, &s_last))
        attn_merge<D>(a, unit, g, s);
}

// -------------------------------------------------------------------------- bf16 / MFMA
template <int D, int NB>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const AttnArgs a) {
    constexpr int TK = 128;                  // keys per workgroup tile
    constexpr int ROWB = D * 2 + 16;         // LDS row stride in bytes (bank-spread padding)
    constexpr int KSTEPS = D / 16;           // k-steps of QK^T
    constexpr int DB = D / 32;               // 32-wide d blocks of PV
    constexpr int KG = 4 / NB;               // key groups (waves sharing a column block)
    constexpr int CHUNKS = D * 2 / 16;       // 16-byte chunks per K/V row
    constexpr int RPP = 256 / CHUNKS;        // rows staged per pass
    constexpr int PASSES = TK / RPP;
    constexpr int MC = 32 * NB;
    __shared__ __attribute__((aligned(16))) char smem[2 * TK * ROWB];

    int unit, split;
    map_block(blockIdx.x, a.units, a.nsplit, &unit, &split);
    if (unit >= a.units) return;
    const int b = unit / a.hkv, g = unit % a.hkv;
    const int tid = threadIdx.x;
    const SeqGeom s = seq_geometry(a, b, tid == 0 && split == 0 && g == 0);
    if (!s.ok) return;

    const int L = s.ctx + s.rows;                      // keys of this sequence
    const int ntiles = (L + TK - 1) / TK;
    const int t_begin = (int)((long)split * ntiles / a.nsplit);
    const int t_end = (int)((long)(split + 1) * ntiles / a.nsplit);
    if (t_begin >= t_end) {
        attn_empty_split<D>(a, unit, split, g, s);
        return;
    }

    const int wave = tid >> 6, lane = tid & 63;
    const int nb = wave % NB, kg = wave / NB;
    const int h = lane >> 5, col = lane & 31;
    const int n = nb * 32 + col;
    const int M = s.rows * a.group;
    const bool col_valid = n < M;
    const int ri = col_valid ? n / a.group : 0;
    const int hh = col_valid ? n % a.group : 0;
    const int causal_lim = s.ctx + ri;                 // key t visible iff t <= causal_lim

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

    const size_t kv_off = ((size_t)b * a.hkv + g) * (size_t)a.s_max * D;
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + kv_off;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + kv_off;
    const int ld_row = tid / CHUNKS, ld_chunk = tid % CHUNKS;

    uint4 pk[PASSES], pv[PASSES];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int key = t * TK + p * RPP + ld_row;
            if (key < L) {
                pk[p] = *reinterpret_cast<const uint4*>(kbase + (size_t)key * D + ld_chunk * 8);
                pv[p] = *reinterpret_cast<const uint4*>(vbase + (size_t)key * D + ld_chunk * 8);
            } else {
                pk[p] = make_uint4(0, 0, 0, 0);
                pv[p] = make_uint4(0, 0, 0, 0);
            }
        }
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;
    char* const ktile = smem;
    char* const vtile = smem + TK * ROWB;

    load_tile(t_begin);
    for (int t = t_begin; t < t_end; ++t) {
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int row = p * RPP + ld_row;
            *reinterpret_cast<uint4*>(ktile + row * ROWB + ld_chunk * 16) = pk[p];
            *reinterpret_cast<uint4*>(vtile + row * ROWB + ld_chunk * 16) = pv[p];
        }
        __syncthreads();
        if (t + 1 < t_end) load_tile(t + 1);

#pragma unroll
        for (int st = 0; st < NB; ++st) {
            const int kl0 = kg * (TK / KG) + st * 32;       // first key of this sub-tile
            // ---- S^T = K Q^T
            f32x16 sacc;
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
                    ktile + (kl0 + col) * ROWB + (16 * kk + 8 * h) * 2);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], sacc, 0, 0, 0);
            }
            // ---- mask + online softmax (lane owns column n; keys 8(r/4)+4h+r%4)
            float sv[16];
            float mt = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tg = t * TK + kl0 + 8 * (r >> 2) + 4 * h + (r & 3);
                const bool vis = col_valid && tg < L && tg <= causal_lim;
                sv[r] = vis ? sacc[r] * a.scale_log2 : kNegInf;
                mt = fmaxf(mt, sv[r]);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            const float alpha = (m_new == kNegInf) ? 1.f : exp2f(m_run - m_new);
            // P goes into the PV product as a bf16 pair hi + lo (about 16 significant
            // bits): a single bf16 rounding of P would perturb the weights by up to 2^-8.
            bf16x8 pb_hi[2], pb_lo[2];
            float ls = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pf = (sv[r] == kNegInf) ? 0.f : exp2f(sv[r] - m_new);
                const uint32_t hi = f32_to_bf16_bits(pf);
                const uint32_t lo = f32_to_bf16_bits(pf - bf16_bits_to_f32(hi));
                ls += pf;
                pb_hi[r >> 3][r & 7] = (short)hi;
                pb_lo[r >> 3][r & 7] = (short)lo;
            }
            l_run = l_run * alpha + ls;
            m_run = m_new;
            if (alpha != 1.f) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            }
            // ---- O^T += V^T P^T  (two 16-key k-steps)
            const int i16 = lane & 15;
            const int half = (lane >> 4) & 1;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int vrow = kl0 + 16 * s2 + 4 * h + (i16 >> 2);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int vcol = 32 * db + 16 * half + 4 * (i16 & 3);
                    const lds_char* base = (const lds_char*)(vtile + vrow * ROWB + vcol * 2);
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_bf16x4*)(base));
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_bf16x4*)(base + 8 * ROWB));
                    const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_hi[s2], o[db], 0, 0, 0);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_lo[s2], o[db], 0, 0, 0);
                }
            }
        }
    }

    // ---- combine the key groups through LDS
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    __syncthreads();                                    // tiles no longer needed
    float* obuf = reinterpret_cast<float*>(smem);
    float* gm = obuf + KG * MC * D;
    float* gl = gm + KG * MC;
    if (h == 0) {
        gm[kg * MC + n] = m_run;
        gl[kg * MC + n] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = 32 * db + 8 * (r >> 2) + 4 * h + (r & 3);
            obuf[(kg * MC + n) * D + d] = o[db][r];
        }
    __syncthreads();
    attn_epilogue<D, KG>(a, smem, unit, split, g, s, MC);
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
    map_block(blockIdx.x, a.units, a.nsplit, &unit, &split);
    if (unit >= a.units) return;
    const int b = unit / a.hkv, g = unit % a.hkv;
    const int tid = threadIdx.x;
    const SeqGeom s = seq_geometry(a, b, tid == 0 && split == 0 && g == 0);
    if (!s.ok) return;
    const int MC = a.mcap;
    const int M = s.rows * a.group;
    const int L = s.ctx + s.rows;
    const int ntiles = (L + TK - 1) / TK;
    const int t_begin = (int)((long)split * ntiles / a.nsplit);
    const int t_end = (int)((long)(split + 1) * ntiles / a.nsplit);
    if (t_begin >= t_end) {
        attn_empty_split<D>(a, unit, split, g, s);
        return;
    }

    float* os = reinterpret_cast<float*>(smem);          // [MC][D]   (epilogue obuf)
    float* ms = os + MC * D;                             // [MC]      (epilogue gm)
    float* ls = ms + MC;                                 // [MC]      (epilogue gl)
    float* ss = os + MCOLS * D + 5 * MCOLS;              // [MCOLS][TK]
    float* al = ss + MCOLS * TK;                         // [MCOLS]
    float* ks = al + MCOLS;                              // [TK][KROW]
    float* vs = ks + TK * KROW;                          // [TK][D]

    for (int e = tid; e < M * D; e += blockDim.x) os[e] = 0.f;
    for (int n = tid; n < M; n += blockDim.x) { ms[n] = kNegInf; ls[n] = 0.f; }

    const float* qg = reinterpret_cast<const float*>(a.q);
    const size_t kv_off = ((size_t)b * a.hkv + g) * (size_t)a.s_max * D;
    const float* kb = reinterpret_cast<const float*>(a.k) + kv_off;
    const float* vb = reinterpret_cast<const float*>(a.v) + kv_off;

    for (int t = t_begin; t < t_end; ++t) {
        __syncthreads();
        for (int e = tid; e < TK * D; e += blockDim.x) {
            const int kr = e / D, d = e % D;
            const int key = t * TK + kr;
            const bool in = key < L;
            ks[kr * KROW + d] = in ? kb[(size_t)key * D + d] : 0.f;
            vs[e] = in ? vb[(size_t)key * D + d] : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < M * TK; e += blockDim.x) {
            const int n = e / TK, kr = e % TK;
            const int key = t * TK + kr;
            const float* qrow = qg + ((size_t)(s.r0 + n / a.group) * a.hq + g * a.group +
                                      n % a.group) * D;
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(qrow[d], ks[kr * KROW + d], dot);
            const bool vis = key < L && key <= s.ctx + n / a.group;
            ss[n * TK + kr] = vis ? dot * a.scale_log2 : kNegInf;
        }
        __syncthreads();
        for (int n = tid; n < M; n += blockDim.x) {
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
        for (int e = tid; e < M * D; e += blockDim.x) {
            const int n = e / D, d = e % D;
            float o = os[e] * al[n];
            for (int kr = 0; kr < TK; ++kr) o = fmaf(ss[n * TK + kr], vs[kr * D + d], o);
            os[e] = o;
        }
    }
    __syncthreads();
    attn_epilogue<D, 1>(a, smem, unit, split, g, s, MC);
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
    const int tiles = (max_kv_len + p.tile - 1) / p.tile;
    int nsplit = (VSA_ATTN_TARGET_WGS + p.units - 1) / p.units;
    if (nsplit > tiles) nsplit = tiles;
    if (nsplit > kMaxSplits) nsplit = kMaxSplits;
    if (nsplit < 1) nsplit = 1;
    p.nsplit = nsplit;
    size_t off = 256;                                            // error word + pad
    p.off_counters = off;
    off += ((size_t)p.units * 4 + 255) / 256 * 256;
    p.off_ml = off;
    off += ((size_t)p.units * nsplit * p.mcap * 8 + 255) / 256 * 256;
    p.off_o = off;
    off += (size_t)p.units * nsplit * p.mcap * D * 4;
    p.bytes = off;
    return p;
}

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, vsa_dtype dtype,
                            hipStream_t stream) {
    const int groups = (p.units + 7) / 8;
    const dim3 grid(groups * 8 * p.nsplit), block(256);
    if (dtype == VSA_BF16) {
        if (a.d == 128) {
            if (p.nb == 1) hipLaunchKernelGGL((attn_bf16_kernel<128, 1>), grid, block, 0, stream, a);
            else if (p.nb == 2) hipLaunchKernelGGL((attn_bf16_kernel<128, 2>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((attn_bf16_kernel<128, 4>), grid, block, 0, stream, a);
        } else {
            if (p.nb == 1) hipLaunchKernelGGL((attn_bf16_kernel<64, 1>), grid, block, 0, stream, a);
            else if (p.nb == 2) hipLaunchKernelGGL((attn_bf16_kernel<64, 2>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((attn_bf16_kernel<64, 4>), grid, block, 0, stream, a);
        }
    } else {
        if (a.d == 128) hipLaunchKernelGGL((attn_f32_kernel<128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_f32_kernel<64>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace vsa
