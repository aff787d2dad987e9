// Truncation pipeline of the vocabulary stage (gfx950): top-k thresholds, nuclei, raw top
// logprobs, then the acceptance and the draws, for calls whose sequences need them (and
// for calls too large for the fused kernel of sample_fused.hip to be resident at once).
//
// Pages (mlx-dspark): top-k threshold and nucleus cutoff from small grouped selections
// instead of full-vocabulary sorts, with the same truncated distribution (Changelog
// [0.20.2] "Changed"); truncation of draft and target (release v0.1.0); accept with
// probability min(1, p/q) and resample the residual (release v0.0.2); penalties and raw
// logprobs (Changelog [0.2.0] "Added"); one-hot proposals (Changelog [0.2.0] "Added",
// --mode lookup).
//
// Kernels, in stream order (each reads what the previous ones wrote):
//   sweep_kernel     grid (B x chunks of 2048 ids x row splits). Each wave of a workgroup
//                    takes whole rows of one sequence's row list (target rows as penalized z,
//                    draft rows, raw rows) over one chunk: per (row, chunk) max /
//                    sum-of-exp / argmax, and for truncated and top-n rows the chunk's
//                    candidates for the k-th-largest threshold (keys at or above a cheap
//                    bound on the chunk's k-th largest, or, when they overflow their slots,
//                    the exact k-th key from a workgroup radix select).
//   select_kernel    one workgroup per truncated or top-n row: the row's threshold and kept
//                    list (sort of the few candidates above a bound on the row's k-th
//                    largest), its nucleus, or the raw top-n logprobs; a nucleus without
//                    top-k by a weighted selection over the whole row.
//   finalize_kernel  one workgroup per sequence: merged statistics, the acceptance tests,
//                    the draws over kept lists, the outputs, and a race request for draws
//                    over the whole vocabulary.
//   race_kernel      grid (B x chunks): the exponential race over the whole vocabulary for
//                    those requests; the last chunk to finish writes the token.
// Random numbers: Philox4x32-10 (Salmon et al., SC'11), see sample_common.h.
#include "sample_common.h"

namespace vsa {

using namespace samp;

namespace {

// ------------------------------------------------------------------ workgroup radix select
// The k-th largest key (1-based) among the valid keys of the workgroup, 8 bits at a time.
// hist: LDS[256]; sh: LDS[>= 2].
__device__ uint32_t wg_select_kth(const uint32_t (&key)[kEpt], uint32_t valid, int k,
                                  uint32_t* hist, int* sh) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint32_t prefix = 0, mask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kEpt; ++e)
            if (((valid >> e) & 1u) && (key[e] & mask) == prefix)
                atomicAdd(&hist[(key[e] >> shift) & 255u], 1u);
        __syncthreads();
        if (tid < 64) {
            const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
            const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
            const uint32_t sl = h0 + h1 + h2 + h3;
            uint32_t incl = sl;
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t v = __shfl_down(incl, off);
                if (lane + off < 64) incl += v;
            }
            const uint32_t above = incl - sl;
            if (above < (uint32_t)need && (uint32_t)need <= incl) {
                uint32_t cum = above;
                int digit;
                if (cum + h3 >= (uint32_t)need) digit = 4 * lane + 3;
                else if ((cum += h3) + h2 >= (uint32_t)need) digit = 4 * lane + 2;
                else if ((cum += h2) + h1 >= (uint32_t)need) digit = 4 * lane + 1;
                else { cum += h1; digit = 4 * lane; }
                sh[0] = digit;
                sh[1] = need - (int)cum;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sh[0] << shift;
        mask |= 0xFFu << shift;
        need = sh[1];
        __syncthreads();
    }
    return prefix;
}

// ------------------------------------------------------------------ wave-level pieces
// Bitonic sort of n <= kKeep (key, id) pairs: key descending, id ascending.
// A lower bound of the k-th largest (1-based, k <= 256) of the 256 threads' values v, in
// every thread: a radix selection on the top 16 bits, 4 bits a round, whose result with
// the low 16 bits cleared has at least k values at or above it (for ordered float keys,
// within 2^-7 relative of the k-th largest). Per round each wave counts in its own LDS
// table the values that carry the prefix chosen so far, per nibble; lanes 0..15 of every
// wave add the four waves' counts (descending nibble order), scan them with row shifts and
// pick the nibble where the running count reaches the remaining k. One barrier a round
// (the count tables are double-buffered by round).
__device__ uint32_t wg_kth_bound(uint32_t v, int k, int (&cnt)[2][4][16]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t prefix = 0u, pmask = 0u;
    int need = k;
    for (int shift = 28, par = 0; shift >= 16; shift -= 4, par ^= 1) {
        // this wave's counts per nibble: its own table, cleared and filled by the wave
        // alone (its LDS operations complete in order)
        if (lane < 16) cnt[par][wave][lane] = 0;
        if ((v & pmask) == prefix) atomicAdd(&cnt[par][wave][(v >> shift) & 15u], 1);
        __syncthreads();
        int t = 0;
        if (lane < 16) {
            const int c = 15 - lane;
            t = cnt[par][0][c] + cnt[par][1][c] + cnt[par][2][c] + cnt[par][3][c];
        }
        int incl = t;                                  // inclusive scan in lanes 0..15
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);   // row_shr:1
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);   // row_shr:2
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);   // row_shr:4
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);   // row_shr:8
        const unsigned long long hit = __ballot(lane < 16 && incl >= need);
        const int L = __ffsll(hit) - 1;             // the prefix's values number >= need
        need -= __builtin_amdgcn_readlane(incl - t, L);
        prefix |= (uint32_t)(15 - L) << shift;
        pmask |= 15u << shift;
    }
    return prefix;
}

// Sorts n <= kKeep (key, id) pairs in LDS by key descending, id ascending (one wave). Up to
// 64 pairs: each pair's rank is the number of pairs before it in that order (ids are
// distinct, so ranks are a permutation) and the pairs move through `tmp` to their ranks:
// n independent LDS reads per lane instead of a bitonic network's log^2 n dependent
// stages. Larger lists take the bitonic network.
__device__ void wave_sort_bitonic(uint32_t* lkey, int* lidx, int n);
__device__ void wave_sort(uint32_t* lkey, int* lidx, int n, uint2* tmp) {
    if (n > 64) {
        wave_sort_bitonic(lkey, lidx, n);
        return;
    }
    const int lane = threadIdx.x & 63;
    for (int i = lane; i < n; i += 64) {
        const uint32_t k = lkey[i];
        const int id = lidx[i];
        int rank = 0;
        for (int t = 0; t < n; ++t) {
            const uint32_t kt = lkey[t];
            const int it = lidx[t];
            rank += (kt > k || (kt == k && it < id)) ? 1 : 0;
        }
        tmp[rank] = make_uint2(k, (uint32_t)id);
    }
    wave_sync();
    for (int i = lane; i < n; i += 64) {
        const uint2 e = tmp[i];
        lkey[i] = e.x;
        lidx[i] = (int)e.y;
    }
    wave_sync();
}

__device__ void wave_sort_bitonic(uint32_t* lkey, int* lidx, int n) {
    const int lane = threadIdx.x & 63;
    int np = 1;
    while (np < n) np <<= 1;
    for (int i = n + lane; i < np; i += 64) {
        lkey[i] = 0u;
        lidx[i] = kBigIdx;
    }
    wave_sync();
    for (int size = 2; size <= np; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = lane; i < np / 2; i += 64) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint32_t ka = lkey[lo], kb = lkey[hi];
                const int ia = lidx[lo], ib = lidx[hi];
                const bool b_first = kb > ka || (kb == ka && ib < ia);
                const bool a_first = ka > kb || (ka == kb && ia < ib);
                if (desc ? b_first : a_first) {
                    lkey[lo] = kb;
                    lkey[hi] = ka;
                    lidx[lo] = ib;
                    lidx[hi] = ia;
                }
            }
            wave_sync();
        }
    }
}

__device__ __forceinline__ double wave_sum_d(double v) { return wave_sum_f64(v); }
__device__ __forceinline__ int wave_min_i(int v) {
    for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
// ------------------------------------------------------------------ workgroup selection
constexpr int kSelTile = 32;     // candidate slots per thread held in registers at once

__device__ __forceinline__ int wg_sum_i(int v, int* sh /* LDS[4] */) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    const int r = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return r;
}

__device__ __forceinline__ uint32_t wg_max_u(uint32_t v, int* sh /* LDS[4] */) {
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = (int)v;
    __syncthreads();
    const uint32_t r = max(max((uint32_t)sh[0], (uint32_t)sh[1]),
                           max((uint32_t)sh[2], (uint32_t)sh[3]));
    __syncthreads();
    return r;
}

// Keys of the candidate slots s0 + tid + 256 j (j < kSelTile) of one row's padded table
// [chunk][capc]; returns the bit mask of the slots that hold a candidate (slot i of chunk c
// is one when i < ccount[c]). All loads are issued before any is used.
__device__ __forceinline__ uint32_t load_slot_keys(const uint2* cand, const int* ccount,
                                                   int capc, int nslots, int s0,
                                                   uint32_t (&kt)[kSelTile]) {
    const float rc = 1.f / (float)capc;
    uint32_t vm = 0u;
#pragma unroll
    for (int j = 0; j < kSelTile; ++j) {
        const int sl = s0 + (int)threadIdx.x + kThreads * j;
        // chunk = sl / capc, from a float quotient corrected by one step (sl < 2^24)
        int c = (int)((float)sl * rc);
        int i = sl - c * capc;
        if (i < 0) { --c; i += capc; }
        else if (i >= capc) { ++c; i -= capc; }
        c = c < 0 ? 0 : c < kMaxChunks - 1 ? c : kMaxChunks - 1;   // in the table
        const bool v = sl < nslots && i < ccount[c];
        vm |= (v ? 1u : 0u) << j;
    }
    // every load issued (clamped into the row's table), then masked: no load waits behind
    // the branch of another
#pragma unroll
    for (int j = 0; j < kSelTile; ++j)
        kt[j] = cand[min(s0 + (int)threadIdx.x + kThreads * j, nslots - 1)].x;
#pragma unroll
    for (int j = 0; j < kSelTile; ++j) kt[j] = ((vm >> j) & 1u) ? kt[j] : 0u;
    return vm;
}

// After a histogram pass: the digit whose bin holds the `need`-th largest key, and how many
// of the keys in that bin are still needed (sh[0], sh[1]). Wave 0 does the scan.
__device__ __forceinline__ void hist_digit(const uint32_t* hist, int need, int* sh) {
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
        const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const uint32_t sl = h0 + h1 + h2 + h3;
        uint32_t incl = sl;
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t v = __shfl_down(incl, off);
            if (lane + off < 64) incl += v;
        }
        const uint32_t above = incl - sl;
        if (above < (uint32_t)need && (uint32_t)need <= incl) {
            uint32_t cum = above;
            int digit;
            if (cum + h3 >= (uint32_t)need) digit = 4 * lane + 3;
            else if ((cum += h3) + h2 >= (uint32_t)need) digit = 4 * lane + 2;
            else if ((cum += h2) + h1 >= (uint32_t)need) digit = 4 * lane + 1;
            else { cum += h1; digit = 4 * lane; }
            sh[0] = digit;
            sh[1] = need - (int)cum;
        }
    }
}

// The k-th largest candidate key of one row (1-based), 8 bits at a time over every valid
// slot; `kt` / `vm0` hold the first tile, reloaded per pass only when the table is larger.
__device__ uint32_t wg_select_slots(const uint2* cand, const int* ccount, int capc, int nslots,
                                    int k, const uint32_t (&kt0)[kSelTile], uint32_t vm0,
                                    uint32_t* hist, int* sh) {
    const int tid = threadIdx.x;
    const bool one_tile = nslots <= kThreads * kSelTile;
    uint32_t prefix = 0, mask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int s0 = 0; s0 < nslots; s0 += kThreads * kSelTile) {
            uint32_t kt[kSelTile];
            uint32_t vm = vm0;
            if (one_tile) {
#pragma unroll
                for (int j = 0; j < kSelTile; ++j) kt[j] = kt0[j];
            } else {
                vm = load_slot_keys(cand, ccount, capc, nslots, s0, kt);
            }
#pragma unroll
            for (int j = 0; j < kSelTile; ++j)
                if (((vm >> j) & 1u) && (kt[j] & mask) == prefix)
                    atomicAdd(&hist[(kt[j] >> shift) & 255u], 1u);
        }
        __syncthreads();
        hist_digit(hist, need, sh);
        __syncthreads();
        prefix |= (uint32_t)sh[0] << shift;
        mask |= 0xFFu << shift;
        need = sh[1];
        __syncthreads();
    }
    return prefix;
}

// ------------------------------------------------------------------ finalize helpers
// Probability of id d under row `slot`'s truncated distribution (its kept list).
__device__ __forceinline__ double keep_lookup(const SampArgs& a, int kslot, int n, int d) {
    const int lane = threadIdx.x & 63;
    const KeepEntry* k = a.keep + (size_t)kslot * a.keepcap;
    double p = 0.0;
    for (int i = lane; i < n; i += 64)
        if (k[i].idx == d) p = k[i].p;
    return wave_sum_d(p);
}
// A double moved by DPP (its two halves with the same control); lanes without a source read 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_d(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xF, false);
    return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}
// (value, id) with the larger value, ties to the lower id, over the wave (every lane), for
// non-negative values (a lane without a source reads value 0, id 0, which never wins over
// a value > 0 and, at 0, only over a larger id: callers treat 0 as "none")
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ void argmax_step_d(double& v, int& i) {
    const double ov = dpp_d<CTRL, ROWS>(v);
    const int oi = dpp_i<CTRL, ROWS>(kBigIdx, i);
    const bool take = (ov > v) | ((ov == v) & (oi < i));
    v = take ? ov : v;
    i = take ? oi : i;
}
__device__ __forceinline__ void wave_argmax_d(double& v, int& i) {
    argmax_step_d<kDppSwap1>(v, i);
    argmax_step_d<kDppSwap2>(v, i);
    argmax_step_d<kDppHalfMirror>(v, i);
    argmax_step_d<kDppMirror>(v, i);
    argmax_step_d<kDppBcast15, 0xA>(v, i);
    argmax_step_d<kDppBcast31, 0xC>(v, i);
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    v = __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
    i = __builtin_amdgcn_readlane(i, 63);
}

// Exponential race over a kept list: weights max(0, p - q) (q from another kept list, a
// one-hot proposal at `onehot_d`, or none) with a fallback to p if every weight is 0. fp64
// keys w / E with E = -ln U from the two race words of the id; ties to the lowest id.
__device__ __forceinline__ int keep_race(const SampArgs& a, int pslot, int np, int qslot, int nq, int onehot_d,
                         int b, int pos, int* qidx /* LDS, kKeep */, double* qp /* LDS, kKeep */) {
    const int lane = threadIdx.x & 63;
    const KeepEntry* kp = a.keep + (size_t)pslot * a.keepcap;
    const KeepEntry* kq = qslot >= 0 ? a.keep + (size_t)qslot * a.keepcap : nullptr;
    const bool resid = kq != nullptr || onehot_d >= 0;
    // the q list in LDS: every p entry scans it there, one broadcast read per entry
    if (kq) {
        for (int t = lane; t < nq; t += 64) {
            qidx[t] = kq[t].idx;
            qp[t] = kq[t].p;
        }
        wave_sync();
    }
    double best = 0.0, fbest = 0.0;
    int bi = kBigIdx, fbi = kBigIdx;
    for (int i = lane; i < np; i += 64) {
        const int j = kp[i].idx;
        const double p = kp[i].p;
        double q = 0.0;
        if (kq)
            for (int t = 0; t < nq; ++t)
                if (qidx[t] == j) q = qp[t];
        if (j == onehot_d) q = 1.0;
        const double r = resid ? fmax(0.0, p - q) : p;
        const uint4 w = philox_block(a.seed, (uint32_t)j >> 1, (uint32_t)pos, (uint32_t)b, 1u);
        const double inv_e = 1.0 / race_e64((j & 1) ? w.z : w.x, (j & 1) ? w.w : w.y);
        if (r > 0.0) {
            const double key = r * inv_e;
            if (key > best || (key == best && j < bi)) { best = key; bi = j; }
        }
        if (p > 0.0) {
            const double key = p * inv_e;
            if (key > fbest || (key == fbest && j < fbi)) { fbest = key; fbi = j; }
        }
    }
    wave_argmax_d(best, bi);
    wave_argmax_d(fbest, fbi);
    if (kq) wave_sync();                               // the LDS list may be reused next
    return best > 0.0 ? bi : fbi;
}

struct FinalShared {
    int sel[8];                  // selection scratch: counter, sums, digit + remaining k
    uint32_t hist[256];
    uint32_t lkey[kKeep];
    int lidx[kKeep];
    double lp[kKeep];
    int ccount[kMaxChunks];
    int nib[2][4][16];           // radix-bound counts (wg_kth_bound)
    int live[kMaxChunks];        // chunks whose maximum reaches the bound, and their count
    int nlive;
    int drafts[kMaxSeqRows];
    double pq[2][kMaxSeqRows];   // p_{t-1}(d_t), q_t(d_t) of truncated rows (finalize)
};

// ------------------------------------------------------------------ per-row selection
// (max, normalizer) of one row from its chunk statistics, by one wave (every lane returns it).
__device__ __forceinline__ RowInfo row_stats_wave(const SampArgs& a, const SeqMode& m, const RowRef& r) {
    const int lane = threadIdx.x & 63;
    float4 st[kChunkLoads];
#pragma unroll
    for (int u = 0; u < kChunkLoads; ++u) {
        const int c = lane + 64 * u;
        st[u] = c < a.nchunk ? a.stats[(size_t)r.slot * a.nchunk + c]
                             : make_float4(kNegInf, 0.f, 0.f, 0.f);
    }
    float bm = kNegInf;
#pragma unroll
    for (int u = 0; u < kChunkLoads; ++u) bm = fmaxf(bm, st[u].x);
    bm = wave_max(bm);
    double z = 0.0;
    if (bm != kNegInf) {
        const float cs = r.kind == 2 ? kLog2e : kLog2e / m.temp;
#pragma unroll
        for (int u = 0; u < kChunkLoads; ++u)
            if (st[u].x != kNegInf) z += (double)st[u].y * (double)exp2f((st[u].x - bm) * cs);
        z = wave_sum_d(z);
    }
    RowInfo ri{};
    ri.m = bm;
    ri.z = z;
    return ri;
}

// Truncated row (top-k threshold, kept set, nucleus; results to the row's workspace RowInfo
// and kept list) or raw top-n row (top ids and their logprobs to the outputs), by one
// workgroup, after the sweep (stream order makes its tables visible). A row's candidates sit
// in a padded table [chunk][capc] (first ccount[c] valid); each thread loads the keys of its
// slots tid + 256 j (coalesced, one round trip per tile of kSelTile slots per thread).
// Lower bounds of the row's k-th largest key usually leave a few dozen candidates, sorted
// exactly; otherwise a radix select over the registers decides. The kept ids (key >= theta)
// go to an LDS list that wave 0 sorts.
__device__ __forceinline__ void select_row(const SampArgs& a, const SeqMode& m, int q, FinalShared& fs) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int* const ccount = fs.ccount;
    const RowRef r = row_ref(a, m, q);
    const bool trunc = m.topk && r.kind != 2;
    const bool topn = r.kind == 2 && m.ntop > 0;
    if (!trunc && !topn) return;
    const int kk = trunc ? m.topk_k : m.ntop;
    const uint2* cand = a.cand + (size_t)r.slot * a.nchunk * a.capc;
    uint32_t ovf_key = 0u;                         // a chunk's k-th key where ties were cut
    bool ovf = false;
    uint32_t cmax = 0u;
    if (tid < a.nchunk) {
        const uint2 meta = a.cand_meta[(size_t)r.slot * a.nchunk + tid];
        const float4 st = a.stats[(size_t)r.slot * a.nchunk + tid];
        ccount[tid] = min((int)meta.x, a.capc);
        ovf = (int)meta.x > a.capc;
        ovf_key = meta.y;
        cmax = ord_key(st.x);
    }
    if (tid == 0) {
        fs.sel[0] = 0;
        fs.nlive = 0;
    }
    __syncthreads();
    const int nslots = a.nchunk * a.capc;
    int tot = 0;
    for (int c = tid; c < a.nchunk; c += kThreads) tot += ccount[c];
    tot = wg_sum_i(tot, fs.sel + 1);
    const int ksel = min(kk, tot);
    if (ksel < 1) {
        if (tid == 0 && trunc) {
            a.rows[r.slot].kept_k = 0;
            a.rows[r.slot].kept_p = 0;
            a.rows[r.slot].theta = kNegInf;
        }
        return;
    }
    // Lower bounds of the row's ksel-th largest key theta: every chunk holds at least k
    // values >= its own k-th key (meta.y), and the ksel largest chunk maxima are ksel
    // distinct values (a radix bound at or below the ksel-th largest of them serves). Usually only a few dozen candidates reach the larger bound; they
    // are sorted exactly. Otherwise a radix select over every candidate decides.
    uint32_t lb = wg_max_u(tid < a.nchunk ? ovf_key : 0u, fs.sel + 1);
    if (a.nchunk >= ksel) lb = max(lb, wg_kth_bound(cmax, ksel, fs.nib));

    uint32_t kt0[kSelTile];
    uint32_t vm0 = 0u;                             // loaded only if the exact path runs
    // every candidate >= bound goes to the LDS list (ids loaded for those only)
    auto collect = [&](uint32_t bound) {
        for (int s0 = 0; s0 < nslots; s0 += kThreads * kSelTile) {
            uint32_t kt[kSelTile];
            uint32_t vmask = vm0;
            if (s0 == 0) {
#pragma unroll
                for (int j = 0; j < kSelTile; ++j) kt[j] = kt0[j];
            } else {
                vmask = load_slot_keys(cand, ccount, a.capc, nslots, s0, kt);
            }
#pragma unroll
            for (int j = 0; j < kSelTile; ++j) {
                // one list reservation per wave and slot column, not one per candidate
                const bool take = ((vmask >> j) & 1u) && kt[j] >= bound;
                const unsigned long long bal = __ballot(take);
                if (bal == 0ull) continue;
                int pos0 = 0;
                if (lane == 0) pos0 = atomicAdd(&fs.sel[0], __popcll(bal));
                pos0 = __builtin_amdgcn_readfirstlane(pos0);
                if (take) {
                    const int pos = pos0 + __popcll(bal & ((1ull << lane) - 1ull));
                    if (pos < kKeep) {
                        fs.lkey[pos] = kt[j];
                        fs.lidx[pos] = (int)cand[s0 + tid + kThreads * j].y;
                    }
                }
            }
        }
        __syncthreads();
    };
    // First pass: only chunks whose maximum reaches lb can hold a candidate >= lb (usually a
    // few dozen of them); their slots are read as (key, id) pairs in one round.
    {
        const bool live = tid < a.nchunk && cmax >= lb && ccount[tid] > 0;
        const unsigned long long bal = __ballot(live);
        int p0 = 0;
        if (lane == 0 && bal) p0 = atomicAdd(&fs.nlive, __popcll(bal));
        p0 = __builtin_amdgcn_readfirstlane(p0);
        if (live) fs.live[p0 + __popcll(bal & ((1ull << lane) - 1ull))] = tid;
    }
    __syncthreads();
    {
        constexpr int kLiveTile = 16;
        const int nlive = fs.nlive;
        const int nls = nlive * a.capc;
        const float rc = 1.f / (float)a.capc;
        for (int s0 = 0; s0 < nls; s0 += kThreads * kLiveTile) {
            uint2 kv[kLiveTile];
            uint32_t vm = 0u;
#pragma unroll
            for (int j = 0; j < kLiveTile; ++j) {
                const int sl = s0 + tid + kThreads * j;
                int li = (int)((float)sl * rc);          // corrected by one step (sl < 2^24)
                int i = sl - li * a.capc;
                if (i < 0) { --li; i += a.capc; }
                else if (i >= a.capc) { ++li; i -= a.capc; }
                li = li < 0 ? 0 : li < nlive - 1 ? li : nlive - 1;
                const int c = fs.live[li];
                vm |= (sl < nls && i < ccount[c] ? 1u : 0u) << j;
                kv[j] = cand[c * a.capc + i];
            }
#pragma unroll
            for (int j = 0; j < kLiveTile; ++j) {
                const bool take = ((vm >> j) & 1u) && kv[j].x >= lb;
                const unsigned long long bal = __ballot(take);
                if (bal == 0ull) continue;
                int pos0 = 0;
                if (lane == 0) pos0 = atomicAdd(&fs.sel[0], __popcll(bal));
                pos0 = __builtin_amdgcn_readfirstlane(pos0);
                if (take) {
                    const int pos = pos0 + __popcll(bal & ((1ull << lane) - 1ull));
                    if (pos < kKeep) {
                        fs.lkey[pos] = kv[j].x;
                        fs.lidx[pos] = (int)kv[j].y;
                    }
                }
            }
        }
        __syncthreads();
    }
    int n_all = fs.sel[0];
    uint32_t theta;
    bool sorted = false;
    if (n_all >= ksel && n_all <= kKeep) {
        if (wave == 0) wave_sort(fs.lkey, fs.lidx, n_all, reinterpret_cast<uint2*>(fs.lp));
        __syncthreads();
        theta = fs.lkey[ksel - 1];
        int cnt = 0;
        for (int i = tid; i < n_all; i += kThreads) cnt += fs.lkey[i] >= theta ? 1 : 0;
        n_all = wg_sum_i(cnt, fs.sel + 1);          // the sorted list's first n_all
        sorted = true;
    } else {
        vm0 = load_slot_keys(cand, ccount, a.capc, nslots, 0, kt0);
        theta = wg_select_slots(cand, ccount, a.capc, nslots, ksel, kt0, vm0, fs.hist,
                                fs.sel + 5);
        if (tid == 0) fs.sel[0] = 0;
        __syncthreads();
        collect(theta);
        n_all = fs.sel[0];
    }
    if (__syncthreads_or(ovf && ovf_key == theta) && tid == 0)
        atomicOr(a.err, VSA_DEVERR_TIE_OVERFLOW);
    if (n_all > kKeep && tid == 0) atomicOr(a.err, VSA_DEVERR_TIE_OVERFLOW);
    if (wave != 0) return;
    const int n = min(n_all, kKeep);
    if (!sorted) wave_sort(fs.lkey, fs.lidx, n, reinterpret_cast<uint2*>(fs.lp));
    if (topn) {
        // raw top-n ids with their log-softmax values
        const RowInfo ri = row_stats_wave(a, m, r);
        const int grow = m.r0 + r.i;
        const double lz = log(ri.z);
        for (int i = lane; i < a.max_top_lp; i += 64) {
            const bool has = i < m.ntop && i < n;
            if (a.top_ids) a.top_ids[(size_t)grow * a.max_top_lp + i] = has ? fs.lidx[i] : -1;
            if (a.top_vals)
                a.top_vals[(size_t)grow * a.max_top_lp + i] =
                    has ? (float)((double)key_float(fs.lkey[i]) - (double)ri.m - lz)
                        : 0.f;
        }
        return;
    }
    // probabilities over the kept set, fp64, in sorted order: exp((v - vmax) / T)
    const float vmax = key_float(fs.lkey[0]);
    double part = 0.0;
    for (int i = lane; i < n; i += 64) {
        const double w = weight64(key_float(fs.lkey[i]), vmax, m.temp);
        fs.lp[i] = w;
        part += w;
    }
    const double zs = wave_sum_d(part);
    wave_sync();
    for (int i = lane; i < n; i += 64) fs.lp[i] /= zs;
    wave_sync();
    int n_keep = n;
    if (m.top_p < 1.f) {
        // inclusive scan in sorted order: lane owns a contiguous run
        const int per = (n + 63) / 64;
        const int i0 = min(lane * per, n), i1 = min(i0 + per, n);
        double run = 0.0;
        for (int i = i0; i < i1; ++i) run += fs.lp[i];
        double excl = run;
        for (int off = 1; off < 64; off <<= 1) {
            const double v = __shfl_up(excl, off);
            if (lane >= off) excl += v;
        }
        excl -= run;
        int first = kBigIdx;
        double cum = excl;
        for (int i = i0; i < i1; ++i) {
            cum += fs.lp[i];
            if (cum >= (double)m.top_p && first == kBigIdx) first = i;
        }
        int mstar = wave_min_i(first);
        if (mstar == kBigIdx) mstar = n - 1;
        // kept: every id whose value is at least the crossing id's (ties of the value kept)
        const uint32_t kcut = fs.lkey[mstar];
        int cnt = 0;
        for (int i = lane; i < n; i += 64) cnt += fs.lkey[i] >= kcut ? 1 : 0;
        n_keep = wave_sum_i(cnt);
        double ks = 0.0;
        for (int i = lane; i < n_keep; i += 64) ks += fs.lp[i];
        ks = wave_sum_d(ks);
        wave_sync();
        for (int i = lane; i < n_keep; i += 64) fs.lp[i] /= ks;
        wave_sync();
    }
    KeepEntry* keep = a.keep + (size_t)r.slot * a.keepcap;
    for (int i = lane; i < n_keep; i += 64) {
        KeepEntry e;
        e.idx = fs.lidx[i];
        e.pad = 0;
        e.p = fs.lp[i];
        keep[i] = e;
    }
    if (lane == 0) {
        a.rows[r.slot].theta = key_float(theta);
        a.rows[r.slot].kept_k = n_all;
        a.rows[r.slot].kept_p = n_keep;
    }
}
// The acceptance of one sequence after the sweep and select_kernel (stream order makes
// their tables visible): the merged statistics of every row, the truncated rows' thresholds
// and kept lists, the acceptance tests, the draws over kept lists, the outputs, and a race
// request for a draw over the whole vocabulary (race_kernel, next in the stream).
template <bool MAP>
__device__ __forceinline__ void finalize_sequence(const SampArgs& a, const SeqMode& m, int b, FinalShared& fs,
                                  RowInfo* rinfo /* LDS, one per row of the list */) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nrows = seq_nrows(a, m);
    const int nd = seq_ndraft(a, m);
    const bool onehot = a.onehot != 0;
    uint32_t ebits = 0;
    // The draft ids, and for sampled rows without top-k each draft's target logit, draft
    // logit and base count (wave 0, lane t - 1), are requested before the statistics merge
    // so that they arrive with it.
    const int* const drafts = fs.drafts;
    if (tid < m.k) fs.drafts[tid] = a.drafts[m.d0 + tid];
    int pre_d = -1, pre_c = 0;
    float pre_xt = 0.f, pre_xd = 0.f;
    const int base_pos = (wave == 0 && m.sampled) ? a.positions[b] : 0;
    if (wave == 0 && lane < m.k) {
        pre_d = a.drafts[m.d0 + lane];
        if (m.sampled && !m.topk && pre_d >= 0 && pre_d < a.vocab) {
            pre_c = a.counts ? a.counts[(size_t)b * a.vocab + pre_d] : 0;
            pre_xt = a.tl[(size_t)(m.r0 + lane) * a.vocab + pre_d];
            if (!onehot) pre_xd = draft_logit<MAP>(a, m.d0 + lane, pre_d);
        }
    }

    // the truncated rows' selection results (select_kernel, a kernel earlier), requested
    // ahead of the statistics (thread q holds row q's; nrows <= kThreads)
    RowInfo sel_ri{};
    const bool sel_row = tid < nrows && (m.topk || m.nucleus) && row_ref(a, m, tid).kind != 2;
    if (sel_row) sel_ri = a.rows[row_ref(a, m, tid).slot];
    // ---- A: merge the chunk statistics of every row. One wave per row, rows q = wave,
    //      wave + 4, ...; the (<= kMaxChunks) chunk entries of up to 3 rows per wave are
    //      loaded in one round (up to kChunkLoads per lane per row), only the half of each
    //      entry the row uses: (max, sum) of a softmax row, (value, id) of a greedy row.
    for (int q0 = wave; q0 < nrows; q0 += 12) {
        float2 st[3][kChunkLoads];
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int q = q0 + 4 * x;
            const RowRef rr = row_ref(a, m, q < nrows ? q : 0);
            const int half = rr.kind == 0 && !m.sampled ? 1 : 0;
#pragma unroll
            for (int u = 0; u < kChunkLoads; ++u) {
                const int c = lane + 64 * u;
                const float2* src =
                    reinterpret_cast<const float2*>(a.stats + (size_t)rr.slot * a.nchunk + c) +
                    half;
                st[x][u] = (q < nrows && c < a.nchunk) ? *src
                                                       : make_float2(kNegInf, __int_as_float(kBigIdx));
            }
        }
#pragma unroll
        for (int x = 0; x < 3; ++x) {
            const int q = q0 + 4 * x;
            if (q >= nrows) break;
            const RowRef r = row_ref(a, m, q);
            const bool greedy_row = r.kind == 0 && !m.sampled;
            float bm = kNegInf, bv = kNegInf;
            int bi = kBigIdx;
            double z = 0.0;
            if (greedy_row) {
#pragma unroll
                for (int u = 0; u < kChunkLoads; ++u) {
                    const int ci = __float_as_int(st[x][u].y);
                    if (better(st[x][u].x, ci, bv, bi)) { bv = st[x][u].x; bi = ci; }
                }
                wave_argmax(bv, bi);
            } else {
                merge_row_wave(st[x], r.kind == 2 ? kLog2e : kLog2e / m.temp, &bm, &z);
            }
            if (lane == 0) {
                RowInfo ri{};
                ri.m = bm;
                ri.z = z;
                ri.argmax = bi;
                ri.theta = kNegInf;
                ri.kept_k = a.vocab;
                ri.kept_p = a.vocab;
                ri.ythr = kNegInf;
                rinfo[q] = ri;
            }
        }
    }
    __syncthreads();

    // ---- B: selection results of truncated rows
    if (sel_row) {
        rinfo[tid].theta = sel_ri.theta;
        rinfo[tid].kept_k = sel_ri.kept_k;
        rinfo[tid].kept_p = sel_ri.kept_p;
        if (m.nucleus) {
            rinfo[tid].ythr = sel_ri.ythr;
            rinfo[tid].ymax = sel_ri.ymax;
            rinfo[tid].zk = sel_ri.zk;
        }
    }
    __syncthreads();
    // every draft's p_{t-1}(d_t) and q_t(d_t) from the truncated rows' kept lists, draft
    // t by wave (t - 1) mod 4, so the lists are read in parallel rather than one draft
    // after another in the acceptance loop (a one-hot proposal has q_t(d_t) = 1)
    if (m.topk) {
        for (int t = 1 + wave; t <= m.k; t += 4) {
            const int d = drafts[t - 1];
            double pd = 0.0, qd = 0.0;
            if (d >= 0 && d < a.vocab) {
                pd = keep_lookup(a, row_ref(a, m, t - 1).slot, rinfo[t - 1].kept_p, d);
                qd = onehot ? 1.0
                            : keep_lookup(a, row_ref(a, m, m.rows + t - 1).slot,
                                          rinfo[m.rows + t - 1].kept_p, d);
            }
            if (lane == 0) {
                fs.pq[0][t - 1] = pd;
                fs.pq[1][t - 1] = qd;
            }
        }
        __syncthreads();
    }

    // ---- C: acceptance (wave 0)
    int acc = 0;
    int tok = -1;
    bool pending = false;
    RaceReq rq{};
    rq.onehot_d = -1;
    if (wave == 0) {
        if (!m.sampled) {
            while (acc < m.k) {
                const int d = drafts[acc];
                if (d < 0 || d >= a.vocab) ebits |= VSA_DEVERR_DRAFT_ID;
                if (d != rinfo[acc].argmax) break;
                ++acc;
            }
            tok = rinfo[acc].argmax;
            if (tok < 0 || tok >= a.vocab) tok = 0;      // a row with no ordered value
        } else if (!m.topk) {
            // p_{t-1}(d_t) and q_t(d_t) of every draft, one lane per draft (t = lane + 1), fp64
            double pd_l = 0.0, qd_l = 0.0;
            const int d_l = lane < m.k ? pre_d : -1;
            const bool valid_l = d_l >= 0 && d_l < a.vocab;
            if (lane < m.k && valid_l) {
                const int t = lane + 1;
                int c = pre_c;
                for (int s2 = 0; s2 < t - 1; ++s2) c += drafts[s2] == d_l ? 1 : 0;
                const float zt = penalize(pre_xt, c, m.pp, m.fp);
                if (m.nucleus) {
                    // kept iff v >= the row's threshold; renormalized over the kept mass
                    const RowInfo& ip = rinfo[t - 1];
                    pd_l = zt >= ip.ythr ? nuc_mass(zt, ip.ymax, m.temp) / ip.zk : 0.0;
                    if (!onehot) {
                        const RowInfo& iq = rinfo[m.rows + t - 1];
                        qd_l = pre_xd >= iq.ythr ? nuc_mass(pre_xd, iq.ymax, m.temp) / iq.zk : 0.0;
                    }
                } else {
                    pd_l = weight64(zt, rinfo[t - 1].m, m.temp) / rinfo[t - 1].z;
                    if (!onehot)
                        qd_l = weight64(pre_xd, rinfo[m.rows + t - 1].m, m.temp) /
                               rinfo[m.rows + t - 1].z;
                }
                if (onehot) qd_l = 1.0;
            }
            // every draft's test at once (u_t from the stream (b, its position, tag 0));
            // the accepted prefix ends at the first lane that rejects
            bool ok = false;
            if (lane < m.k) ok = valid_l && accept_uniform(a.seed, b, base_pos + lane) * qd_l < pd_l;
            const unsigned long long rej = __ballot(lane < m.k && !ok);
            acc = rej ? __ffsll(rej) - 1 : m.k;
            if (__ballot(lane < m.k && lane <= acc && !valid_l)) ebits |= VSA_DEVERR_DRAFT_ID;
            pending = true;
            rq.a = acc;
            rq.pos = base_pos + acc;
            if (acc < m.k) {                 // residual of target row acc, draft row acc+1
                rq.kind = 1;
                rq.m_p = rinfo[acc].m;
                rq.z_p = rinfo[acc].z;
                if (onehot) {
                    rq.onehot_d = drafts[acc];
                } else {
                    rq.m_q = rinfo[m.rows + acc].m;
                    rq.z_q = rinfo[m.rows + acc].z;
                }
            } else {                         // bonus draw from target row K
                rq.kind = 2;
                rq.m_p = rinfo[m.k].m;
                rq.z_p = rinfo[m.k].z;
            }
            if (m.nucleus) {                 // the rows' nuclei and kept masses
                rq.nucleus = 1;
                rq.z_p = rinfo[acc].zk;
                rq.ythr_p = rinfo[acc].ythr;
                rq.ymax_p = rinfo[acc].ymax;
                if (acc < m.k && !onehot) {
                    rq.z_q = rinfo[m.rows + acc].zk;
                    rq.ythr_q = rinfo[m.rows + acc].ythr;
                    rq.ymax_q = rinfo[m.rows + acc].ymax;
                }
            }
        } else {
            // truncated rows: every draft's test at once (lane t - 1: p and q from the kept
            // lists, 0 for an invalid draft, so that it is rejected); the accepted prefix
            // ends at the first lane that rejects
            bool ok = false;
            const int d_l = lane < m.k ? drafts[lane] : -1;
            const bool valid_l = d_l >= 0 && d_l < a.vocab;
            if (lane < m.k) ok = accept_uniform(a.seed, b, base_pos + lane) * fs.pq[1][lane] <
                                 fs.pq[0][lane];
            const unsigned long long rej = __ballot(lane < m.k && !ok);
            acc = rej ? __ffsll(rej) - 1 : m.k;
            if (__ballot(lane < m.k && lane <= acc && !valid_l)) ebits |= VSA_DEVERR_DRAFT_ID;
            const bool all = acc == m.k;
            if (!all) {
                const int t = acc + 1, pos = base_pos + acc;
                const int d = drafts[acc];
                const RowRef rp = row_ref(a, m, t - 1);
                if (onehot) {
                    tok = keep_race(a, rp.slot, rinfo[t - 1].kept_p, -1, 0, d, b, pos, fs.lidx,
                                    fs.lp);
                } else {
                    const RowRef rqr = row_ref(a, m, m.rows + t - 1);
                    tok = keep_race(a, rp.slot, rinfo[t - 1].kept_p, rqr.slot,
                                    rinfo[m.rows + t - 1].kept_p, -1, b, pos, fs.lidx, fs.lp);
                }
                if (tok < 0 || tok >= a.vocab) tok = 0;
            }
            if (all) {
                const RowRef rp = row_ref(a, m, m.k);
                tok = keep_race(a, rp.slot, rinfo[m.k].kept_p, -1, 0, -1, b, base_pos + m.k,
                                fs.lidx, fs.lp);
                if (tok < 0 || tok >= a.vocab) tok = 0;
            }
        }
        // raw statistics of the row whose token the race kernel will pick
        if (pending) {
            rq.logprobs = m.logprobs;
            if (m.raw) {
                const int xq = m.rows + nd + acc;
                rq.m_x = rinfo[xq].m;
                rq.z_x = rinfo[xq].z;
            }
        }
    }
    if (wave == 0 && lane == 0) {
        a.race[b] = rq;
        a.accepted[b] = acc;
    }
    if (wave == 0) {
        // emitted tokens, logprobs, diagnostics. The token and logprob of a pending draw
        // are the race kernel's to write.
        for (int s = lane; s < m.rows; s += 64) {
            const int grow = m.r0 + s;
            int out = -1;
            if (s < acc) out = drafts[s];
            else if (s == acc) out = tok;
            if (!(pending && s == acc)) a.out_tokens[grow] = out;
            if (a.chosen_lp && !(pending && s == acc)) {
                float lpv = __builtin_nanf("");
                if (m.logprobs && out >= 0) {
                    const int xq = m.rows + nd + s;
                    lpv = (float)((double)a.tl[(size_t)grow * a.vocab + out] -
                                  (double)rinfo[xq].m - log(rinfo[xq].z));
                }
                a.chosen_lp[grow] = lpv;
            }
            if (a.diag_thr) a.diag_thr[grow] = m.sampled ? rinfo[s].theta : __builtin_nanf("");
            if (a.diag_kept) {
                a.diag_kept[2 * grow] = m.sampled ? rinfo[s].kept_k : 0;
                a.diag_kept[2 * grow + 1] = m.sampled ? rinfo[s].kept_p : 0;
            }
            if (m.ntop == 0 && a.max_top_lp > 0) {
                for (int i = 0; i < a.max_top_lp; ++i) {
                    if (a.top_ids) a.top_ids[(size_t)grow * a.max_top_lp + i] = -1;
                    if (a.top_vals) a.top_vals[(size_t)grow * a.max_top_lp + i] = 0.f;
                }
            }
        }
        if (ebits && lane == 0) atomicOr(a.err, ebits);
    }
}

// ------------------------------------------------------------------ full-vocabulary race
// A categorical draw over the whole vocabulary as an exponential race: id j wins when its
// key w_j / E_j is the largest, E_j = -ln U_j standard exponential from the draw's Philox
// stream (tag 1), w = max(0, p - q) for a residual draw (kind 1) or p (kind 2); when every
// residual weight is 0 the draw falls back to the race on p itself. Each chunk of kChunk
// ids finds its two winners; the last chunk to arrive merges them.

// The winners of this wave's ids of chunk c for request rq: (key, id, fallback key,
// fallback id), valid in every lane. xp / xq hold the chunk of the target row (m.r0 + rq.a)
// and, for kind 1 with a draft row, of the draft row (m.d0 + rq.a); dm[e] marks the drafts
// before row rq.a that equal id e. Ids past the vocabulary hold -inf logits (weight 0).
template <bool NUC>
__device__ float4 race_chunk(const SampArgs& a, const SeqMode& m, const RaceReq& rq, int b,
                             int c, const int (&cnt)[kEpt], const uint32_t (&dm)[kEpt],
                             const float (&xp)[kEpt], const float (&xq)[kEpt]) {
    const int tid = threadIdx.x;
    const int base = c * kChunk;
    const bool draft_q = rq.kind == 1 && rq.onehot_d < 0;
    const float inv_zp = (float)(1.0 / rq.z_p);
    const float inv_zq = draft_q ? (float)(1.0 / rq.z_q) : 0.f;
    const float cs = kLog2e / m.temp;
    // Keys are w / (-log2 U) (the race's w / E times ln 2, the same argmax), with the
    // hardware exp2 / log2 / reciprocal (a few ulps each). A thread visits its ids in
    // increasing order, so a strict > keeps the lower id of a tie; w = 0 gives a key of 0,
    // which never wins.
    float best = 0.f, fbest = 0.f;
    int bi = kBigIdx, fbi = kBigIdx;
#pragma unroll
    for (int qd = 0; qd < kQuads; ++qd) {
        const int j0 = base + 1024 * qd + 4 * tid;
        const RaceWords w = race_words4(a.seed, j0, rq.pos, b);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = 4 * qd + r;
            const int j = j0 + r;
            const float zp = penalize(xp[e], cnt[e] + __popc(dm[e]), m.pp, m.fp);
            float p, q = 0.f;
            if constexpr (NUC) {
                // nucleus rows: ids below the row's threshold have probability 0
                p = zp >= rq.ythr_p ? (float)(nuc_mass(zp, rq.ymax_p, m.temp) / rq.z_p) : 0.f;
                if (draft_q)
                    q = xq[e] >= rq.ythr_q ? (float)(nuc_mass(xq[e], rq.ymax_q, m.temp) / rq.z_q)
                                           : 0.f;
            } else {
                p = __builtin_amdgcn_exp2f((zp - rq.m_p) * cs) * inv_zp;
                if (draft_q) q = __builtin_amdgcn_exp2f((xq[e] - rq.m_q) * cs) * inv_zq;
            }
            if (rq.kind == 1 && j == rq.onehot_d) q = 1.f;
            const float rr = rq.kind == 1 ? fmaxf(0.f, p - q) : p;
            const float inv_e = __builtin_amdgcn_rcpf(race_e2(w.hi(r), w.lo(r)));
            const float key = rr * inv_e, fkey = p * inv_e;
            const bool up = key > best, fup = fkey > fbest;
            best = up ? key : best;
            bi = up ? j : bi;
            fbest = fup ? fkey : fbest;
            fbi = fup ? j : fbi;
        }
    }
    wave_argmax(best, bi);
    // the race on p itself only decides when no residual weight anywhere is positive, so a
    // wave that found one leaves its fallback out
    if (best > 0.f) {
        fbest = 0.f;
        fbi = kBigIdx;
    } else {
        wave_argmax(fbest, fbi);
    }
    return make_float4(best, __int_as_float(bi), fbest, __int_as_float(fbi));
}

__device__ __forceinline__ float4 race_none() {
    return make_float4(0.f, __int_as_float(kBigIdx), 0.f, __int_as_float(kBigIdx));
}

// The drawn id of sequence b from its chunk winners (one hand-off slot per chunk: atomics
// on a shared winner serialize badly), merged by one wave; valid in lane 0.
__device__ int race_winner(const SampArgs& a, int b, int lane) {
    float bb = 0.f, fb = 0.f;
    int bbi = kBigIdx, fbi2 = kBigIdx;
    constexpr int kLoads = 4 * kChunkLoads;               // 4 waves x <= kMaxChunks chunks
    float4 pt[kLoads];                                    // one round
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int cc = lane + 64 * u;
        pt[u] = cc < 4 * a.nchunk
                    ? handoff_load4(a.race_part + (size_t)b * a.nchunk * 4 + cc)
                    : race_none();
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const float4 o = pt[u];
        const int oi = __float_as_int(o.y), ofi = __float_as_int(o.w);
        if (o.x > bb || (o.x == bb && oi < bbi)) { bb = o.x; bbi = oi; }
        if (o.z > fb || (o.z == fb && ofi < fbi2)) { fb = o.z; fbi2 = ofi; }
    }
    wave_argmax(bb, bbi);
    wave_argmax(fb, fbi2);
    int tok = bb > 0.f ? bbi : fbi2;
    if (tok < 0 || tok >= a.vocab) tok = 0;               // a row with no ordered value
    return tok;
}
// The race kernel: only sequences whose draw is over the whole vocabulary do work.
template <bool VEC, bool MAP>
__global__ __launch_bounds__(kThreads) void race_kernel(const SampArgs a) {
    __shared__ int s_draft[kMaxSeqRows];
    __shared__ int s_last;
    preload_args(a);
    const int b = blockIdx.x / a.nchunk, c = blockIdx.x % a.nchunk;
    const int tid = threadIdx.x;
    const RaceReq rq = a.race[b];                  // requested with the sequence's shape
    uint32_t ebits = 0;
    const SeqMode m = seq_mode(a, b, &ebits);
    if (!m.valid || !m.sampled || m.topk || rq.kind == 0) return;
    const int base = c * kChunk;
    int cnt[kEpt];
    load_counts<VEC>(a.counts ? a.counts + (size_t)b * a.vocab : nullptr, base, a.vocab, cnt);
    float xp[kEpt], xq[kEpt];
    load_chunk<VEC>(a.tl + (size_t)(m.r0 + rq.a) * a.vocab, base, a.vocab, xp);
    if (rq.kind == 1 && rq.onehot_d < 0) load_draft_chunk<VEC, MAP>(a, m.d0 + rq.a, base, xq);
    else
#pragma unroll
        for (int e = 0; e < kEpt; ++e) xq[e] = 0.f;
    uint32_t dm[kEpt];
    int dreg = 0;
    scalar_drafts(a, m, rq.a, base, s_draft, dm, dreg);
    const float4 part = rq.nucleus ? race_chunk<true>(a, m, rq, b, c, cnt, dm, xp, xq)
                                   : race_chunk<false>(a, m, rq, b, c, cnt, dm, xp, xq);
    if ((tid & 63) == 0) handoff_store4(a.race_part + ((size_t)b * a.nchunk + c) * 4 + (tid >> 6), part);
    if (!handoff_arrive(counter_at(a.ctr, a.ctr_x, 4 * b + 1), (uint32_t)a.nchunk, &s_last) || tid >= 64) return;
    const int tok = race_winner(a, b, tid);
    if (tid != 0) return;
    const int grow = m.r0 + rq.a;
    a.out_tokens[grow] = tok;
    if (a.chosen_lp)
        a.chosen_lp[grow] = rq.logprobs ? (float)((double)a.tl[(size_t)grow * a.vocab + tok] -
                                                  (double)rq.m_x - log(rq.z_x))
                                        : __builtin_nanf("");
}

// ------------------------------------------------------------------ wave-layout chunk
// A whole chunk of one row in one wave: lane l holds the float4s l + 64 j (j < 8), that is
// ids base + 4 (l + 64 j) + i (i < 4) as element e = 4 j + i. The sweep gives each data row
// (a target row together with its raw twin, which reads the same logits, or a draft row)
// to one wave: penalties, statistics and candidates of the row with wave reductions only,
// no workgroup barrier, while the wave's next row loads. Every global access in that loop
// goes through a buffer resource whose byte count bounds it (a load past it returns 0, a
// store past it is dropped), so no memory instruction there is conditional: the compiler
// then counts the loads in flight exactly and the next row's loads overlap the current
// row's work (a conditional load or store before a use makes it wait for all of them).
constexpr int kWj = kChunk / 256;                 // float4s per lane
constexpr int kWe = 4 * kWj;                      // ids per lane
// candidate slots of a (row, chunk): capc <= max(top-k bound kKeep, top-logprobs bound 32)
// + 32, so kCandStores stores per lane write any of them
constexpr int kCandCap = kKeep + 32;
constexpr int kCandStores = (kCandCap + 63) / 64;
__device__ __forceinline__ int welem_id(int base, int lane, int e) {
    return base + 4 * (lane + 64 * (e >> 2)) + (e & 3);
}
// Inclusive prefix sum over the wave's lanes (lane i: x_0 + ... + x_i): shifts by 1, 2, 4, 8
// within rows of 16 lanes, then the row totals carried by broadcasts.
__device__ __forceinline__ int wave_incl_scan_i(int x) {
    x += dpp_i<0x111>(0, x);                      // row_shr:1 (lanes without a source add 0)
    x += dpp_i<0x112>(0, x);
    x += dpp_i<0x114>(0, x);
    x += dpp_i<0x118>(0, x);
    x += dpp_i<kDppBcast15, 0xA>(0, x);
    x += dpp_i<kDppBcast31, 0xC>(0, x);
    return x;
}
// The 32-bit words at the chunk's ids of the array that `rs` covers (0 past its end).
template <bool VEC>
__device__ __forceinline__ void wbuf_load(__amdgpu_buffer_rsrc_t rs, int base, int lane,
                                          uint32_t (&x)[kWe]) {
    if (VEC) {
#pragma unroll
        for (int j = 0; j < kWj; ++j) {
            const vsa_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                rs, (uint32_t)(base + 4 * (lane + 64 * j)) * 4u, 0, 0);
            x[4 * j] = v.x;
            x[4 * j + 1] = v.y;
            x[4 * j + 2] = v.z;
            x[4 * j + 3] = v.w;
        }
    } else {
        uint32_t o0 = (uint32_t)(base + 4 * lane) * 4u;
        asm volatile("" : "+v"(o0));                   // offsets from here: not 32 hoisted registers
#pragma unroll
        for (int e = 0; e < kWe; ++e)
            x[e] = __builtin_amdgcn_raw_buffer_load_b32(
                rs, o0 + (uint32_t)(256 * (e >> 2) + (e & 3)) * 4u, 0, 0);
    }
}
// Row q of the sequence's row list at the chunk's ids (a raw row reads its target row's
// logits; draft rows through t2d when MAP), -inf past the vocabulary. `present` false: no
// row (the loads cover 0 bytes).
template <bool VEC, bool MAP>
__device__ __forceinline__ void wload_row(const SampArgs& a, const SeqMode& m, int q, bool present,
                                          int base, int lane, uint32_t valid, float (&x)[kWe]) {
    uint32_t u[kWe];
    const RowRef r = row_ref(a, m, q);
    if (MAP && r.kind == 1) {
        const float* row = a.dl + (size_t)(m.d0 + r.i - 1) * a.dvocab;
        wbuf_load<VEC>(handoff_rsrc(a.t2d, present ? (uint32_t)a.vocab * 4u : 0u), base, lane, u);
        const __amdgpu_buffer_rsrc_t rr = handoff_rsrc(row, present ? (uint32_t)a.dvocab * 4u : 0u);
        uint32_t ebits = 0;
#pragma unroll
        for (int e = 0; e < kWe; ++e) {
            const int mp = ((valid >> e) & 1u) ? (int)u[e] : -1;
            // an entry outside [0, dvocab) reads past the resource: 0, replaced by -inf
            const float v = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)mp * 4u, 0, 0));
            x[e] = (uint32_t)mp < (uint32_t)a.dvocab ? v : kNegInf;
            ebits |= (mp < -1 || mp >= a.dvocab) ? VSA_DEVERR_DRAFT_MAP : 0u;
        }
        if (__ballot(ebits != 0u) && lane == 0) atomicOr(a.err, VSA_DEVERR_DRAFT_MAP);
        return;
    }
    const float* row = r.kind == 1 ? a.dl + (size_t)(m.d0 + r.i - 1) * a.vocab
                                   : a.tl + (size_t)(m.r0 + r.i) * a.vocab;
    wbuf_load<VEC>(handoff_rsrc(row, present ? (uint32_t)a.vocab * 4u : 0u), base, lane, u);
#pragma unroll
    for (int e = 0; e < kWe; ++e) x[e] = ((valid >> e) & 1u) ? __uint_as_float(u[e]) : kNegInf;
}

// Chunk statistics of one row, by one wave (valid in every lane): (max v, sum of
// 2^((v - max) cs)) for a softmax row, (0, 0, value, id) of the argmax (lowest id on ties)
// for a greedy target row. Invalid ids hold -inf.
__device__ __forceinline__ float4 wave_row_stats(int base, int lane, uint32_t valid, bool greedy,
                                                 float cs, const float (&v)[kWe]) {
    if (greedy) {
        float bv = kNegInf;
        int bi = kBigIdx;
        int b0 = base + 4 * lane;
        asm volatile("" : "+v"(b0));                   // ids from here: not 32 hoisted registers
#pragma unroll
        for (int e = 0; e < kWe; ++e) {
            const int id = b0 + 256 * (e >> 2) + (e & 3);
            const bool t = ((valid >> e) & 1u) && better(v[e], id, bv, bi);
            bv = t ? v[e] : bv;
            bi = t ? id : bi;
        }
        wave_argmax(bv, bi);
        return make_float4(0.f, 0.f, bv, __int_as_float(bi));
    }
    float mx = v[0];
#pragma unroll
    for (int e = 1; e < kWe; ++e) mx = fmaxf(mx, v[e]);
    mx = wave_max(mx);
    float sm = 0.f;
    if (mx != kNegInf) {
#pragma unroll
        for (int e = 0; e < kWe; ++e) sm += __builtin_amdgcn_exp2f((v[e] - mx) * cs);
    }
    return make_float4(mx, wave_sum(sm), 0.f, 0.f);
}

// Candidates of one truncated or top-n row in this chunk, by one wave: every key >= vk for
// a vk at or below the chunk's kk-th largest key. vk is the largest 16-bit-prefixed value T
// such that at least kk of the lanes' group maxima (the maxima of 1, 2 or 4 disjoint groups
// of each lane's ids as kk needs: distinct ids) are >= T, found by a binary search with
// ballot counts; it lies within 2^-7 of the kk-th largest of those maxima, so the
// candidates are usually the kk largest and a few more. They go to the wave's LDS list
// (the first capc of them); *total counts them all (more than capc: the workgroup path
// takes the row).
__device__ __forceinline__ void wave_candidates(const SampArgs& a, int base, int lane, int kk, int n_valid,
                                uint32_t valid, const uint32_t (&key)[kWe], uint2* list,
                                int* total_out, uint32_t* vk_out) {
    uint32_t vk = 0u;
    if (n_valid > kk) {
        const int ng = kk <= 16 ? 1 : kk <= 32 ? 2 : 4;
        uint32_t g8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) g8[i] = max(max(key[i], key[i + 8]), max(key[i + 16], key[i + 24]));
        uint32_t gm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gm[i] = max(g8[i], g8[i + 4]);      // groups e mod 4
        if (ng <= 2) {
            gm[0] = max(gm[0], gm[2]);
            gm[1] = max(gm[1], gm[3]);
            gm[2] = gm[3] = 0u;
        }
        if (ng == 1) {
            gm[0] = max(gm[0], gm[1]);
            gm[1] = 0u;
        }
        uint32_t t = 0u;
        for (int bit = 31; bit >= 16; --bit) {
            const uint32_t cand = t | (1u << bit);
            int n = __popcll(__ballot(gm[0] >= cand));
            if (ng > 1) n += __popcll(__ballot(gm[1] >= cand));
            if (ng > 2) n += __popcll(__ballot(gm[2] >= cand)) + __popcll(__ballot(gm[3] >= cand));
            if (n >= kk) t = cand;
        }
        vk = t;
    }
    // this lane's candidates as a mask of its elements, their count, and the candidates of
    // the lanes before it: each lane fills consecutive slots, no ballot per element
    uint32_t tm = 0u;
#pragma unroll
    for (int e = 0; e < kWe; ++e) tm |= (((valid >> e) & 1u) && key[e] >= vk) ? (1u << e) : 0u;
    const int n = __popc(tm);
    const int incl = wave_incl_scan_i(n);
    const int off = incl - n;
    // every element is written, a candidate to its slot and any other to the lane's spare
    // slot past the list, so the writes take no branch
    const int spare = kCandCap + lane;
    int b0 = base + 4 * lane;
    asm volatile("" : "+v"(b0));                       // ids from here: not 32 hoisted registers
#pragma unroll
    for (int e = 0; e < kWe; ++e) {
        const int pos = off + __popc(tm & ((1u << e) - 1u));
        const bool w = ((tm >> e) & 1u) && pos < a.capc;
        list[w ? pos : spare] = make_uint2(key[e], (uint32_t)(b0 + 256 * (e >> 2) + (e & 3)));
    }
    *total_out = __builtin_amdgcn_readlane(incl, 63);
    *vk_out = vk;
}

typedef unsigned int vsa_u32x2 __attribute__((ext_vector_type(2)));
// A (row, chunk)'s candidate slots and count from the wave's LDS list: kCandStores + 1
// stores per lane whatever the row (`on` false or an overflow: every one past its
// resource, dropped), so every row issues the same memory instructions.
__device__ __forceinline__ void wave_cand_store(const SampArgs& a, size_t sc, int lane, bool on,
                                                const uint2* list, int total, uint32_t vk) {
    const bool fits = on && total <= a.capc;
    const int nout = fits ? total : 0;
    const __amdgpu_buffer_rsrc_t rs = handoff_rsrc(a.cand + sc * a.capc, on ? (uint32_t)a.capc * 8u : 0u);
#pragma unroll
    for (int s = 0; s < kCandStores; ++s) {
        const int i = lane + 64 * s;
        const uint2 v = list[i < a.capc ? i : 0];
        vsa_u32x2 w;
        w.x = v.x;
        w.y = v.y;
        __builtin_amdgcn_raw_buffer_store_b64(w, rs, i < nout ? (uint32_t)i * 8u : (uint32_t)a.capc * 8u,
                                              0, 0);
    }
    vsa_u32x2 meta;
    meta.x = (uint32_t)total;
    meta.y = vk;
    const __amdgpu_buffer_rsrc_t rm = handoff_rsrc(a.cand_meta + sc, on ? 8u : 0u);
    __builtin_amdgcn_raw_buffer_store_b64(meta, rm, (lane == 0 && fits) ? 0u : 8u, 0, 0);
}

template <bool VEC, bool MAP>
__global__ __launch_bounds__(kThreads, 3) void sweep_kernel(const SampArgs a) {
    __shared__ uint2 s_list[4][kCandCap + 64];      // + a spare slot per lane
    __shared__ int s_draft[kMaxSeqRows];
    __shared__ uint32_t s_hist[256];
    __shared__ int s_ovf[3 * kMaxSeqRows];
    __shared__ int s_novf;
    __shared__ int s_sh[4];

    preload_args(a);
    // workgroup (b, c, s): chunk c of the rows q = s, s + S, ... of sequence b's row list
    // (S = rsplit; targets, drafts, then raw rows); the workgroup's n-th row goes to wave
    // n mod 4
    const int s_row = blockIdx.x % a.rsplit, bc = blockIdx.x / a.rsplit;
    const int b = bc / a.nchunk, c = bc % a.nchunk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: row pointers in SGPRs
    const int base = c * kChunk;
    uint32_t ebits = 0;
    const SeqMode m = seq_mode(a, b, &ebits);
    if (c == 0 && tid == 0 && s_row == 0 && ebits) atomicOr(a.err, ebits);
    if (!m.valid) return;
    const int nrows = seq_nrows(a, m);
    const int nloc = s_row < nrows ? (nrows - s_row + a.rsplit - 1) / a.rsplit : 0;
    if (nloc == 0) return;
    if (tid < m.k) s_draft[tid] = a.drafts[m.d0 + tid];
    if (tid == 0) s_novf = 0;
    const bool has_pen = m.pp != 0.f || m.fp != 0.f;
    const int n_valid = min(kChunk, a.vocab - base);
    uint32_t valid = 0;
#pragma unroll
    for (int e = 0; e < kWe; ++e) valid |= (welem_id(base, lane, e) < a.vocab ? 1u : 0u) << e;

    // this wave's rows: u = wave, wave + 4, ... (row s_row + rsplit u); the base counts (when
    // penalties apply) and the first row are requested together
    uint32_t cnt[kWe];
    {
        const bool pc = has_pen && a.counts != nullptr;
        wbuf_load<VEC>(handoff_rsrc(pc ? (const void*)(a.counts + (size_t)b * a.vocab)
                                       : (const void*)a.tl,
                                    pc ? (uint32_t)a.vocab * 4u : 0u),
                       base, lane, cnt);
    }
    float xa[kWe];
    int u = wave;
    wload_row<VEC, MAP>(a, m, s_row + a.rsplit * u, u < nloc, base, lane, valid, xa);
    __syncthreads();                                   // s_draft, s_novf
    // the wave's target rows come in increasing order, so cnt accumulates the drafts d_1 ..
    // d_i of each in place (`applied` of them so far)
    int applied = 0;
    for (; u < nloc; u += 4) {
        float xb[kWe];
        wload_row<VEC, MAP>(a, m, s_row + a.rsplit * (u + 4), u + 4 < nloc, base, lane, valid, xb);
        const int q = s_row + a.rsplit * u;
        const RowRef r = row_ref(a, m, q);
        if (r.kind == 0 && has_pen) {
            // z = (x - fp c) - pp [c > 0], c the base count plus the drafts d_1 .. d_i
            for (; applied < r.i; ++applied) {
                const int off = __builtin_amdgcn_readfirstlane(s_draft[applied]) - base;
                if (off < 0 || off >= kChunk) continue;             // not in this chunk
                const int ee = 4 * (off >> 8) + (off & 3);
                const bool mine = ((off >> 2) & 63) == lane;
#pragma unroll
                for (int e = 0; e < kWe; ++e) cnt[e] += (mine && e == ee) ? 1u : 0u;
            }
#pragma unroll
            for (int e = 0; e < kWe; ++e) xa[e] = penalize(xa[e], (int)cnt[e], m.pp, m.fp);
        }
        // this row's outputs: its statistics and, for a truncated or top-n row, candidates;
        // log2(e) / T recomputed per row (hoisted, it would hold a vector register across
        // the loop)
        // the sequence's T is uniform over the wave: held in a scalar register, opaque
        float temp = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(m.temp)));
        asm volatile("" : "+s"(temp));
        const float cs = r.kind == 2 ? kLog2e : kLog2e / temp;
        const float4 st = wave_row_stats(base, lane, valid, r.kind == 0 && !m.sampled, cs, xa);
        const bool cand = r.kind == 2 ? m.ntop > 0 : m.topk;
        int tot = 0;
        uint32_t vk = 0u;
        if (cand) {
            uint32_t key[kWe];
#pragma unroll
            for (int e = 0; e < kWe; ++e) key[e] = ((valid >> e) & 1u) ? ord_key(xa[e]) : 0u;
            wave_candidates(a, base, lane, r.kind == 2 ? m.ntop : m.topk_k, n_valid, valid, key,
                            s_list[wave], &tot, &vk);
        }
        wave_sync();
        // the stores: the same instructions for every row (those not wanted fall past
        // zero-byte resources)
        const size_t sc = (size_t)r.slot * a.nchunk + c;
        handoff_store16(handoff_rsrc(a.stats + sc, 16u), lane == 0 ? 0u : 16u, st);
        wave_cand_store(a, sc, lane, cand, s_list[wave], tot, vk);
        wave_sync();                                   // the list is reused by the next row
        if (lane == 0 && cand && tot > a.capc) s_ovf[atomicAdd(&s_novf, 1)] = q;
#pragma unroll
        for (int e = 0; e < kWe; ++e) xa[e] = xb[e];
    }

    // ---- rows whose candidates overflowed the slots: the whole workgroup, with the exact
    // kk-th key (radix select); every key above it and the ties at it up to capc slots are
    // written (the count says how many there were)
    __syncthreads();
    const int novf = s_novf;
    if (novf == 0) return;
    int cnt_t[kEpt];
    load_counts<VEC>(a.counts ? a.counts + (size_t)b * a.vocab : nullptr, base, a.vocab, cnt_t);
    uint32_t dm[kEpt];
    draft_masks(s_draft, m.k, base, dm);
    uint32_t valid_t = 0;
#pragma unroll
    for (int e = 0; e < kEpt; ++e) valid_t |= (elem_id(base, e) < a.vocab ? 1u : 0u) << e;
    for (int o = 0; o < novf; ++o) {
        const int q = s_ovf[o];
        const RowRef r = row_ref(a, m, q);
        const int kk = r.kind != 2 ? m.topk_k : m.ntop;
        float x[kEpt];
        load_row_chunk<VEC, MAP>(a, m, r, base, x);
        uint32_t key[kEpt];
#pragma unroll
        for (int e = 0; e < kEpt; ++e) {
            float val = x[e];
            if (r.kind == 0)
                val = penalize(val, cnt_t[e] + __popc(dm[e] & low_bits(r.i)), m.pp, m.fp);
            key[e] = ord_key(val);
        }
        uint2* out = a.cand + ((size_t)r.slot * a.nchunk + c) * a.capc;
        const uint32_t vk = wg_select_kth(key, valid_t, kk, s_hist, s_sh);
        if (tid == 0) s_sh[2] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kEpt; ++e)
            if (((valid_t >> e) & 1u) && key[e] > vk) {
                const int pos = atomicAdd(&s_sh[2], 1);
                out[pos] = make_uint2(key[e], (uint32_t)elem_id(base, e));
            }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kEpt; ++e)
            if (((valid_t >> e) & 1u) && key[e] == vk) {
                const int pos = atomicAdd(&s_sh[2], 1);
                if (pos < a.capc)
                    out[pos] = make_uint2(key[e], (uint32_t)elem_id(base, e));
            }
        __syncthreads();
        const int ncand = s_sh[2];
        if (tid == 0)
            a.cand_meta[(size_t)r.slot * a.nchunk + c] = make_uint2((uint32_t)ncand, vk);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ nucleus without top-k
// A sampled row with top_p < 1 and no top-k keeps {j : v_j >= v*} (v the penalized target
// logit z, or the draft logit), where v* is the value at which the mass e^((v - vmax) / T)
// of the ids sorted by v (descending) first reaches top_p of the row's mass; ties at v* are
// kept (mlx-dspark release v0.1.0 "Lossless top-p / top-k sampling": the nucleus truncates
// draft and target). No sort: a weighted selection over many workgroups per row.
//  (1) Histogram pass (select kernel): nsel workgroups per row each bin a share of the
//      row's chunks by (vmax - v) / T in steps of 1/16 (kNucBins bins, the last holding
//      every lower value) with the mass in fp64, and add their bins into the row's
//      histogram in the workspace; the last to finish finds the crossing bin b*, where the
//      mass from the top reaches top_p of the row's mass.
//  (2) Listing pass (finalize kernel): one workgroup per (sequence, chunk) appends, for
//      each nucleus row of the sequence, the chunk's ids in b* (their ordered keys) to the
//      row's list (one reservation per row and chunk); the last to finish runs, one wave
//      per row, a radix selection on the listed keys weighted by mass (8 bits at a time,
//      from the top), which gives v*. A row whose crossing bin is the last one, or whose
//      list does not fit, takes the same radix selection over rescans of the whole row.
__device__ __forceinline__ int nuc_bin(float v, float vmax, float s16) {
    const float u = (vmax - v) * s16;         // monotone in v: ties share a bin (s16 = 16/T)
    return u < (float)(kNucBins - 1) ? (int)u : kNucBins - 1;
}
struct NucBins {                              // LDS: a histogram of bins or radix digits
    double hm[kNucBins];                      // mass per bin / digit
    int hn[kNucBins];                         // ids per bin / digit
    int drafts[kMaxSeqRows];
    int pos, cnt_before;
    double mass_before;
};


// Inclusive prefix sum of a double over the wave's lanes (dpp_d moves its two halves).
__device__ __forceinline__ double wave_incl_scan_d(double x) {
    x += dpp_d<0x111>(x);
    x += dpp_d<0x112>(x);
    x += dpp_d<0x114>(x);
    x += dpp_d<0x118>(x);
    x += dpp_d<kDppBcast15, 0xA>(x);
    x += dpp_d<kDppBcast31, 0xC>(x);
    return x;
}
__device__ __forceinline__ double readlane_d(double v, int l) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// One wave walks positions 0..nb-1 of hm / hn (nb a multiple of 64; position p is bin
// nb - 1 - p when rev) from `base`: the first position whose running mass reaches `target`
// (when none does, rounding at the very end, the last non-empty one), the running mass
// before it (base included) and the ids of this histogram before it, in every lane.
__device__ __forceinline__ void wave_crossing(const double* hm, const int* hn, int nb, bool rev,
                                              double base, double target, int* pos_out,
                                              double* mass_out, int* cnt_out) {
    const int lane = threadIdx.x & 63;
    const int per = nb / 64;
    double ms = 0.0;
    int cs = 0;
    for (int i = 0; i < per; ++i) {
        const int p = lane * per + i, idx = rev ? nb - 1 - p : p;
        ms += hm[idx];
        cs += hn[idx];
    }
    const double incl = wave_incl_scan_d(ms);
    const int incl_n = wave_incl_scan_i(cs);
    const unsigned long long hit = __ballot(base + incl >= target);
    const unsigned long long nz = __ballot(cs > 0);
    const int L = hit ? __ffsll(hit) - 1 : (nz ? 63 - __clzll(nz) : 0);   // uniform
    // lane L walks its positions from the running totals of the lanes before it
    double acc = base + (L > 0 ? readlane_d(incl, L - 1) : 0.0);
    int an = L > 0 ? __builtin_amdgcn_readlane(incl_n, L - 1) : 0;
    int pos = -1;
    if (lane == L) {
        int last = -1, last_n = 0;
        double last_m = 0.0;
        for (int i = 0; i < per; ++i) {
            const int p = lane * per + i, idx = rev ? nb - 1 - p : p;
            if (hit && acc + hm[idx] >= target) {
                pos = p;
                break;
            }
            if (hn[idx] > 0) {
                last = p;
                last_m = acc;
                last_n = an;
            }
            acc += hm[idx];
            an += hn[idx];
        }
        if (pos < 0) {                                  // no crossing here: last non-empty
            pos = last < 0 ? lane * per : last;
            acc = last_m;
            an = last_n;
        }
    }
    *pos_out = __builtin_amdgcn_readlane(pos, L);
    *mass_out = readlane_d(acc, L);
    *cnt_out = __builtin_amdgcn_readlane(an, L);
}

// One pass over row r's values v in chunks [cb, ce), f(v) per id (ids past the vocabulary
// skipped). Target rows carry their penalties (base counts plus the drafts before the row).
template <bool VEC, bool MAP, class F>
__device__ __forceinline__ void nuc_pass(const SampArgs& a, const SeqMode& m, const RowRef& r, int b,
                                         const int* drafts, int cb, int ce, F&& f) {
    constexpr int kB = 4;                           // chunks whose loads are in flight together
    const bool pen = r.kind == 0 && (m.pp != 0.f || m.fp != 0.f);
    const int32_t* crow = a.counts ? a.counts + (size_t)b * a.vocab : nullptr;
    for (int c0 = cb; c0 < ce; c0 += kB) {
        float x[kB][kEpt];
        int cnt[kB][kEpt];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            if (c0 + u >= ce) continue;
            load_row_chunk<VEC, MAP>(a, m, r, (c0 + u) * kChunk, x[u]);
            if (pen) load_counts<VEC>(crow, (c0 + u) * kChunk, a.vocab, cnt[u]);
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            if (c0 + u >= ce) continue;
            const int base = (c0 + u) * kChunk;
            if (pen) {
                uint32_t dm[kEpt];
                draft_masks(drafts, r.i, base, dm);   // drafts d_1 .. d_i
#pragma unroll
                for (int e = 0; e < kEpt; ++e)
                    x[u][e] = penalize(x[u][e], cnt[u][e] + __popc(dm[e]), m.pp, m.fp);
            }
#pragma unroll
            for (int e = 0; e < kEpt; ++e)
                if (elem_id(base, e) < a.vocab) f(x[u][e]);
        }
    }
}

// Per-thread run-length aggregation of (bin, mass) before the LDS atomics: ids of one
// thread that fall in the same bin in a row cost one atomic.
struct NucRun {
    int cur = -1;
    double acc = 0.0;
    int n = 0;
    __device__ __forceinline__ void add(NucBins& ns, int k, double w) {
        if (k != cur) {
            flush(ns);
            cur = k;
        }
        acc += w;
        ++n;
    }
    __device__ __forceinline__ void flush(NucBins& ns) {
        if (cur >= 0) {
            atomicAdd(&ns.hm[cur], acc);
            atomicAdd(&ns.hn[cur], n);
        }
        cur = -1;
        acc = 0.0;
        n = 0;
    }
};

// The result of a nucleus row (no top-k) to its RowInfo.
__device__ __forceinline__ void nuc_result(const SampArgs& a, const RowRef& r, float vmax,
                                           uint32_t prefix, int kept, double zk) {
    RowInfo* out = a.rows + r.slot;
    out->theta = kNegInf;
    out->kept_k = a.vocab;
    out->kept_p = kept;
    out->ythr = key_float(prefix);
    out->ymax = vmax;
    out->zk = zk;
}

// (1) Histogram pass of nucleus row q of sequence b, share s of a.nsel.
template <bool VEC, bool MAP>
__device__ __forceinline__ void nucleus_hist(const SampArgs& a, const SeqMode& m, int b, int q,
                                             int s, NucBins& ns, int* s_last) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const RowRef r = row_ref(a, m, q);
    if (tid < m.k) ns.drafts[tid] = a.drafts[m.d0 + tid];
    for (int i = tid; i < kNucBins; i += kThreads) {
        ns.hm[i] = 0.0;
        ns.hn[i] = 0;
    }
    const RowInfo st = row_stats_wave(a, m, r);      // the row's max of v (every wave)
    const float vmax = st.m;
    const float s16 = 16.f / m.temp;
    __syncthreads();
    NucInfo* const ni = a.nuc_info + r.slot;
    if (vmax == kNegInf) {                             // no orderable value: nothing kept
        if (s == 0 && tid == 0) {
            RowInfo* out = a.rows + r.slot;
            out->theta = kNegInf;
            out->kept_k = a.vocab;
            out->kept_p = 0;
            out->ythr = __builtin_inff();
            out->ymax = vmax;
            out->zk = 0.0;
            ni->bstar = -1;
            ni->listed = 0;
        }
        return;
    }
    const int cb = (int)((long)s * a.nchunk / a.nsel), ce = (int)((long)(s + 1) * a.nchunk / a.nsel);
    {
        NucRun run;
        nuc_pass<VEC, MAP>(a, m, r, b, ns.drafts, cb, ce, [&](float v) {
            run.add(ns, nuc_bin(v, vmax, s16), nuc_mass(v, vmax, m.temp));
        });
        run.flush(ns);
    }
    __syncthreads();
    // this share's bins into the row's histogram (device-scope atomics; the bins are zero
    // between calls)
    double* const ghm = a.nuc_hm + (size_t)r.slot * kNucBins;
    uint32_t* const ghn = a.nuc_hn + (size_t)r.slot * kNucBins;
    for (int i = tid; i < kNucBins; i += kThreads)
        if (ns.hn[i] != 0) {
            atomicAdd(ghm + i, ns.hm[i]);
            atomicAdd(ghn + i, (uint32_t)ns.hn[i]);
        }
    if (!handoff_arrive(counter_at(a.ctr, a.ctr_x, 4 * a.batch + r.slot), (uint32_t)a.nsel, s_last))
        return;
    // the last share: the whole histogram (read where the atomics were performed), back to
    // zero for the next call; the row's mass, the target and the crossing bin
    for (int i = tid; i < kNucBins; i += kThreads) {
        unsigned long long* const hb = reinterpret_cast<unsigned long long*>(ghm + i);
        ns.hm[i] = __longlong_as_double(
            (long long)__hip_atomic_load(hb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        ns.hn[i] = (int)__hip_atomic_load(ghn + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(hb, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ghn + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (wave == 0) {
        double t = 0.0;
        for (int i = lane; i < kNucBins; i += 64) t += ns.hm[i];
        t = wave_sum_d(t);
        const double target = (double)m.top_p * t;
        int pos, cbf;
        double mb;
        wave_crossing(ns.hm, ns.hn, kNucBins, false, 0.0, target, &pos, &mb, &cbf);
        if (lane == 0) {
            NucInfo info;
            info.mass_before = mb;
            info.target = target;
            info.vmax = vmax;
            info.bstar = pos;
            info.cnt_before = cbf;
            info.nb = ns.hn[pos];
            info.listed = 0;
            *ni = info;
        }
    }
}

// (2) Listing pass: chunk c of every nucleus row of sequence b, one wave per row; the
// ordered keys of the ids in the row's crossing bin go to its list (the row's candidate
// area, kept as a compact array of keys, capacity nchunk * capc * 2) at offsets reserved
// with one atomic per row and chunk.
template <bool VEC, bool MAP>
__device__ __forceinline__ void nucleus_list(const SampArgs& a, const SeqMode& m, int b, int c) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int base = c * kChunk;
    const int ndata = m.rows + seq_ndraft(a, m);       // targets and drafts: the nucleus rows
    const bool has_pen = m.pp != 0.f || m.fp != 0.f;
    const float s16 = 16.f / m.temp;
    const uint32_t cap = (uint32_t)a.nchunk * (uint32_t)a.capc * 2u;
    uint32_t valid = 0;
#pragma unroll
    for (int e = 0; e < kWe; ++e) valid |= (welem_id(base, lane, e) < a.vocab ? 1u : 0u) << e;
    uint32_t cnt[kWe];
    {
        const bool pc = has_pen && a.counts != nullptr;
        wbuf_load<VEC>(handoff_rsrc(pc ? (const void*)(a.counts + (size_t)b * a.vocab)
                                       : (const void*)a.tl,
                                    pc ? (uint32_t)a.vocab * 4u : 0u),
                       base, lane, cnt);
    }
    int applied = 0;                                   // drafts already in cnt (see the sweep)
    for (int q = wave; q < ndata; q += 4) {
        const RowRef r = row_ref(a, m, q);
        // the row's crossing bin and its chunk, requested together
        const int bstar_v = a.nuc_info[r.slot].bstar;
        const float vmax_v = a.nuc_info[r.slot].vmax;
        float x[kWe];
        wload_row<VEC, MAP>(a, m, q, true, base, lane, valid, x);
        const int bstar = __builtin_amdgcn_readfirstlane(bstar_v);
        if (bstar < 0 || bstar == kNucBins - 1) continue;   // resolved, or rescanned
        const float vmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vmax_v)));
        if (r.kind == 0 && has_pen) {
            for (; applied < r.i; ++applied) {
                const int off = __builtin_amdgcn_readfirstlane(a.drafts[m.d0 + applied]) - base;
                if (off < 0 || off >= kChunk) continue;
                const int ee = 4 * (off >> 8) + (off & 3);
                const bool mine = ((off >> 2) & 63) == lane;
#pragma unroll
                for (int e = 0; e < kWe; ++e) cnt[e] += (mine && e == ee) ? 1u : 0u;
            }
#pragma unroll
            for (int e = 0; e < kWe; ++e) x[e] = penalize(x[e], (int)cnt[e], m.pp, m.fp);
        }
        uint32_t tm = 0u;
#pragma unroll
        for (int e = 0; e < kWe; ++e)
            tm |= (((valid >> e) & 1u) && nuc_bin(x[e], vmax, s16) == bstar) ? (1u << e) : 0u;
        const int n = __popc(tm);
        const int incl = wave_incl_scan_i(n);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (total == 0) continue;
        int r0 = 0;
        if (lane == 0) r0 = atomicAdd(&a.nuc_info[r.slot].listed, total);
        r0 = __builtin_amdgcn_readfirstlane(r0);
        uint32_t* const list = reinterpret_cast<uint32_t*>(a.cand + (size_t)r.slot * a.nchunk * a.capc);
        const __amdgpu_buffer_rsrc_t rl = handoff_rsrc(list, cap * 4u);
        const int o = r0 + incl - n;
#pragma unroll
        for (int e = 0; e < kWe; ++e) {
            const uint32_t pos = (uint32_t)(o + __popc(tm & ((1u << e) - 1u)));
            __builtin_amdgcn_raw_buffer_store_b32(ord_key(x[e]), rl,
                                                  ((tm >> e) & 1u) ? pos * 4u : cap * 4u, 0,
                                                  kCpolSc1);
        }
    }
}

// v* of nucleus row q from its listed keys, by one wave: radix selection on the ordered
// keys, 8 bits at a time from the top, weighted by mass. false: the row takes the rescan.
__device__ __forceinline__ bool nucleus_finish_wave(const SampArgs& a, const SeqMode& m, int q,
                                                    uint32_t* lkey /* LDS, kWaveList */,
                                                    double* hm /* LDS, 256 */, int* hn /* 256 */) {
    constexpr int kWaveList = 1024;
    constexpr int kPer = kWaveList / 64;
    const int lane = threadIdx.x & 63;
    const RowRef r = row_ref(a, m, q);
    // the row's record, its list count and the first kWaveList slots of its list, requested
    // together (slots past the count are masked below)
    const uint32_t cap = (uint32_t)a.nchunk * (uint32_t)a.capc * 2u;
    const uint32_t* list = reinterpret_cast<const uint32_t*>(a.cand + (size_t)r.slot * a.nchunk * a.capc);
    const __amdgpu_buffer_rsrc_t rl = handoff_rsrc(list, cap * 4u);
    uint32_t kv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        kv[j] = __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)(lane + 64 * j) * 4u, 0, kCpolSc1);
    const NucInfo ni = a.nuc_info[r.slot];
    const int listed = (int)__hip_atomic_load(&a.nuc_info[r.slot].listed, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (ni.bstar < 0) return true;                     // resolved by the histogram pass
    if (ni.bstar == kNucBins - 1 || ni.nb > kWaveList || listed != ni.nb || (uint32_t)listed > cap)
        return false;
    // the keys' common leading bits: digits above the first differing bit are fixed (every
    // key has them, so the crossing is there with nothing above it)
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        lkey[lane + 64 * j] = kv[j];
        if (lane + 64 * j < listed) {
            kmin = min(kmin, kv[j]);
            kmax = max(kmax, kv[j]);
        }
    }
    kmin = (uint32_t)wave_min_i((int)(kmin ^ 0x80000000u)) ^ 0x80000000u;
    kmax = ~((uint32_t)wave_min_i((int)(~kmax ^ 0x80000000u)) ^ 0x80000000u);
    const int same = kmin == kmax ? 32 : __clz((int)(kmin ^ kmax));
    const int pass0 = same / 8;                        // passes before it: one digit each
    wave_sync();
    double base = ni.mass_before;
    int cbase = ni.cnt_before;
    double last_m = 0.0;
    int last_n = listed;
    uint32_t prefix = pass0 > 0 ? kmin >> (32 - 8 * pass0) : 0u;
    for (int pass = pass0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hm[lane + 64 * i] = 0.0;
            hn[lane + 64 * i] = 0;
        }
        wave_sync();
        // each lane's keys of one digit in a row cost one atomic
        int cur = -1, n = 0;
        double acc = 0.0;
        for (int i = lane; i < listed; i += 64) {
            const uint32_t key = lkey[i];
            if (pass > 0 && (key >> (shift + 8)) != prefix) continue;
            const int d = (int)((key >> shift) & 255u);
            if (d != cur) {
                if (cur >= 0) {
                    atomicAdd(&hm[cur], acc);
                    atomicAdd(&hn[cur], n);
                }
                cur = d;
                acc = 0.0;
                n = 0;
            }
            acc += nuc_mass(key_float(key), ni.vmax, m.temp);
            ++n;
        }
        if (cur >= 0) {
            atomicAdd(&hm[cur], acc);
            atomicAdd(&hn[cur], n);
        }
        wave_sync();
        int pos, cb;
        double mb;
        wave_crossing(hm, hn, 256, true, base, ni.target, &pos, &mb, &cb);
        const int digit = 255 - pos;
        base = mb;
        cbase += cb;
        last_m = hm[digit];
        last_n = hn[digit];
        prefix = (prefix << 8) | (uint32_t)digit;
        wave_sync();
    }
    if (pass0 == 4) {                                  // every key equal: all of them kept
        double t = 0.0;
        for (int i = lane; i < listed; i += 64) t += nuc_mass(key_float(lkey[i]), ni.vmax, m.temp);
        last_m = wave_sum_d(t);
    }
    if (lane == 0) nuc_result(a, r, ni.vmax, prefix, cbase + last_n, base + last_m);
    return true;
}

// The same selection by the whole workgroup over rescans of row q (the ids of the crossing
// bin found again in each radix pass): any list size, any crossing bin.
template <bool VEC, bool MAP>
__device__ __forceinline__ void nucleus_rescan(const SampArgs& a, const SeqMode& m, int b, int q,
                                               NucBins& ns) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const RowRef r = row_ref(a, m, q);
    const NucInfo ni = a.nuc_info[r.slot];
    const float s16 = 16.f / m.temp;
    if (tid < m.k) ns.drafts[tid] = a.drafts[m.d0 + tid];
    double base = ni.mass_before;
    int cbase = ni.cnt_before;
    double last_m = 0.0;
    int last_n = 0;
    uint32_t prefix = 0u;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += kThreads) {
            ns.hm[i] = 0.0;
            ns.hn[i] = 0;
        }
        __syncthreads();
        {
            NucRun run;
            nuc_pass<VEC, MAP>(a, m, r, b, ns.drafts, 0, a.nchunk, [&](float v) {
                if (nuc_bin(v, ni.vmax, s16) != ni.bstar) return;
                const uint32_t key = ord_key(v);
                if (pass > 0 && (key >> (shift + 8)) != prefix) return;
                run.add(ns, (int)((key >> shift) & 255u), nuc_mass(v, ni.vmax, m.temp));
            });
            run.flush(ns);
        }
        __syncthreads();
        if (wave == 0) {
            int pos, cb;
            double mb;
            wave_crossing(ns.hm, ns.hn, 256, true, base, ni.target, &pos, &mb, &cb);
            if (lane == 0) {
                ns.pos = pos;
                ns.mass_before = mb;
                ns.cnt_before = cb;
            }
        }
        __syncthreads();
        const int digit = 255 - ns.pos;
        base = ns.mass_before;
        cbase += ns.cnt_before;
        last_m = ns.hm[digit];
        last_n = ns.hn[digit];
        prefix = (prefix << 8) | (uint32_t)digit;
        __syncthreads();
    }
    if (tid == 0) nuc_result(a, r, ni.vmax, prefix, cbase + last_n, base + last_m);
}

// ------------------------------------------------------------------ top-k pipeline kernels
// grid (B x rows_cap x nsel): workgroup (b, q, s) selects row q of sequence b when it is a
// truncated or top-n row (s = 0), or runs share s of the histogram pass of a nucleus row;
// every other workgroup returns at once.
template <bool VEC, bool MAP>
__global__ __launch_bounds__(kThreads) void select_kernel(const SampArgs a, int rows_cap) {
    __shared__ FinalShared s_final;
    __shared__ NucBins s_bins;
    __shared__ int s_last;
    preload_args(a);
    // the shares s > 0 come last in the grid: the workgroups with work are dispatched first
    const int nbq = a.batch * rows_cap;
    const int s = blockIdx.x / nbq, bq = blockIdx.x - s * nbq;
    const int b = bq / rows_cap, q = bq % rows_cap;
    uint32_t ebits = 0;
    const SeqMode m = seq_mode(a, b, &ebits);
    if (!m.valid || q >= seq_nrows(a, m)) return;
    if (m.nucleus && row_ref(a, m, q).kind != 2) nucleus_hist<VEC, MAP>(a, m, b, q, s, s_bins, &s_last);
    else if (s == 0) select_row(a, m, q, s_final);
}


// grid (B x nfin): merges the chunk statistics and runs the acceptance of one sequence
// (workgroup (b, 0)); for a sequence with nucleus rows, workgroup (b, c) first lists chunk
// c of them and the last to finish completes the rows, then finalizes the sequence.
template <bool VEC, bool MAP>
__global__ __launch_bounds__(kThreads) void finalize_kernel(const SampArgs a) {
    __shared__ FinalShared s_final;
    __shared__ RowInfo s_rinfo[3 * kMaxSeqRows];
    __shared__ uint32_t s_lkey[4][1024];
    __shared__ double s_whm[4][256];
    __shared__ int s_whn[4][256];
    __shared__ NucBins s_bins;
    __shared__ int s_fb[kMaxSeqRows * 2];
    __shared__ int s_nfb;
    __shared__ int s_last;
    preload_args(a);
    // chunk-major: the workgroups (b, 0), which finalize the sequences without nucleus rows,
    // are dispatched first
    const int c = blockIdx.x / a.batch, b = blockIdx.x - c * a.batch;
    const int tid = threadIdx.x, wave = tid >> 6;
    uint32_t ebits = 0;
    const SeqMode m = seq_mode(a, b, &ebits);
    if (!m.valid) return;
    if (m.nucleus) {
        if (tid == 0) s_nfb = 0;
        // the listed keys go out and come back with the hand-off cache policy (coherent
        // across the XCDs), so the count-in needs no cache write-back
        nucleus_list<VEC, MAP>(a, m, b, c);
        if (!handoff_arrive(counter_at(a.ctr, a.ctr_x, 4 * b + 2), (uint32_t)a.nfin, &s_last)) return;
        const int ndata = m.rows + seq_ndraft(a, m);
        for (int q = wave; q < ndata; q += 4)
            if (!nucleus_finish_wave(a, m, q, s_lkey[wave], s_whm[wave], s_whn[wave]) &&
                (tid & 63) == 0)
                s_fb[atomicAdd(&s_nfb, 1)] = q;
        __syncthreads();
        const int nfb = s_nfb;
        for (int i = 0; i < nfb; ++i) {
            const int q = s_fb[i];
            __syncthreads();
            nucleus_rescan<VEC, MAP>(a, m, b, q, s_bins);
        }
        // this workgroup's row results in place before the acceptance reads them back
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    } else if (c != 0) {
        return;
    }
    finalize_sequence<MAP>(a, m, b, s_final, s_rinfo);
}

}  // namespace

SampPlan plan_sample(int B, int total_rows, int V, int max_top_k, int max_top_lp) {
    SampPlan p{};
    p.nchunk = (V + kChunk - 1) / kChunk;
    const int kmax = max_top_k > max_top_lp ? max_top_k : max_top_lp;
    int capc = kmax > 0 ? kmax + 32 : 0;
    if (capc > kChunk) capc = kChunk;
    if (capc > V) capc = V;
    p.capc = capc;
    p.keepcap = V < kKeep ? V : kKeep;
    p.slots = 3 * total_rows - B;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t off = kWsHeader;                         // error word, counters
    // counters: four per sequence, then one per row slot (the nucleus histogram pass)
    p.n_ctr_x = extra_counters(4L * B + (max_top_k > 0 ? (long)p.slots : 0L));
    p.off_ctr_x = off;
    off += up(p.n_ctr_x * 4);
    p.off_stats = off;
    off += up((size_t)p.slots * p.nchunk * 16);
    p.off_cand = off;
    off += up((size_t)p.slots * p.nchunk * capc * 8);
    p.off_meta = off;
    off += up((size_t)p.slots * p.nchunk * 8);
    p.off_rows = off;
    off += up((size_t)p.slots * sizeof(RowInfo));
    p.off_keep = off;
    off += up(max_top_k > 0 ? (size_t)(2 * total_rows - B) * p.keepcap * sizeof(KeepEntry) : 0);
    p.off_race = off;
    off += up((size_t)B * sizeof(RaceReq));
    p.off_race_part = off;
    off += up((size_t)B * p.nchunk * 4 * 16);
    // nucleus rows without top-k need max_top_k >= 1
    const size_t nslots = max_top_k > 0 ? (size_t)p.slots : 0;
    p.off_nuc_hm = off;
    off += up(nslots * kNucBins * 8);
    p.off_nuc_hn = off;
    off += up(nslots * kNucBins * 4);
    p.off_nuc_info = off;
    off += up(nslots * sizeof(NucInfo));
    p.bytes = off;
    return p;
}

// Inverse of a reduced draft vocabulary's offset table: t2d[x] = the draft id j with
// j + d2t[j] = x, or -1. Two launches in stream order: fill, then scatter (an entry outside
// [0, V) is skipped; if two draft ids share a target id the higher one is kept).
__global__ __launch_bounds__(256) void t2d_fill_kernel(int32_t* t2d, int vocab) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < vocab) t2d[i] = -1;
}
__global__ __launch_bounds__(256) void t2d_scatter_kernel(const int32_t* d2t, int dvocab,
                                                          int vocab, int32_t* t2d) {
    const int j = blockIdx.x * kThreads + threadIdx.x;
    if (j >= dvocab) return;
    const long x = (long)j + d2t[j];
    if (x >= 0 && x < vocab) atomicMax(t2d + x, j);
}

hipError_t launch_draft_vocab_inverse(const int32_t* d2t, int dvocab, int vocab, int32_t* t2d,
                                      hipStream_t stream) {
    hipLaunchKernelGGL(t2d_fill_kernel, dim3((unsigned)((vocab + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, t2d, vocab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(t2d_scatter_kernel, dim3((unsigned)((dvocab + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, d2t, dvocab, vocab, t2d);
    return hipGetLastError();
}

hipError_t launch_sample(const SampArgs& args, hipStream_t stream) {
    SampArgs a = args;
    // Without truncation, top-n logprobs or a grid too large to be resident at once, the
    // whole stage is the fused kernel (sample_fused.hip).
    if (fused_fits(a)) return launch_fused(a, stream);
    const dim3 grid((unsigned)a.batch * a.nchunk), block(kThreads);
    // the sweep splits each sequence's rows over up to 4 workgroups per chunk when the
    // sequences alone give fewer than 512 workgroups
    a.rsplit = 1;
    while (a.rsplit < 4 && (long)a.batch * a.nchunk * a.rsplit < 512) a.rsplit *= 2;
    const dim3 sweep_grid((unsigned)a.batch * a.nchunk * a.rsplit);
    const bool vec = (a.vocab % 4) == 0;
    const bool map = a.t2d != nullptr;
#define VSA_SWEEP(V, M) hipLaunchKernelGGL((sweep_kernel<V, M>), sweep_grid, block, 0, stream, a)
    if (map) {
        if (vec) VSA_SWEEP(true, true); else VSA_SWEEP(false, true);
    } else {
        if (vec) VSA_SWEEP(true, false); else VSA_SWEEP(false, false);
    }
#undef VSA_SWEEP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one workgroup per (sequence, row of its row list), several per nucleus row; then one
    // per sequence, or per (sequence, chunk) when nucleus rows may be present
    const int rows_cap = 3 * a.max_rows;
    a.nsel = 1;
    a.nfin = 1;
    if (a.max_top_k > 0 && a.nuc_info != nullptr) {
        while (a.nsel < 16 && (long)a.batch * rows_cap * a.nsel * 2 <= 1024) a.nsel *= 2;
        a.nfin = a.nchunk;
    }
    const dim3 sgrid((unsigned)a.batch * rows_cap * a.nsel);
    if (map) {
        if (vec) hipLaunchKernelGGL((select_kernel<true, true>), sgrid, block, 0, stream, a, rows_cap);
        else hipLaunchKernelGGL((select_kernel<false, true>), sgrid, block, 0, stream, a, rows_cap);
    } else {
        if (vec) hipLaunchKernelGGL((select_kernel<true, false>), sgrid, block, 0, stream, a, rows_cap);
        else hipLaunchKernelGGL((select_kernel<false, false>), sgrid, block, 0, stream, a, rows_cap);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 fgrid((unsigned)a.batch * a.nfin);
    if (map) {
        if (vec) hipLaunchKernelGGL((finalize_kernel<true, true>), fgrid, block, 0, stream, a);
        else hipLaunchKernelGGL((finalize_kernel<false, true>), fgrid, block, 0, stream, a);
    } else {
        if (vec) hipLaunchKernelGGL((finalize_kernel<true, false>), fgrid, block, 0, stream, a);
        else hipLaunchKernelGGL((finalize_kernel<false, false>), fgrid, block, 0, stream, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Only the device knows which sequences end in a full-vocabulary draw; every other
    // workgroup returns at once.
    if (map) {
        if (vec) hipLaunchKernelGGL((race_kernel<true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((race_kernel<false, true>), grid, block, 0, stream, a);
    } else {
        if (vec) hipLaunchKernelGGL((race_kernel<true, false>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((race_kernel<false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace vsa
