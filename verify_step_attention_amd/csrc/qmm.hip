// Few-row quantized matmul of the verify forward (gfx950): y[M, N] = x[M, K] w[N, K]^T for
// M <= 16 rows, with w affine-quantized per group of 64 inputs (8- or 4-bit codes, fp16
// scale and bias). mlx-dspark Changelog [0.20.0] "Changed": the verify widths' matmul is
// computed with the weights as the matrix operand, shared by every row, instead of paying
// the weight read per row.
//
// The weights are the A operand of v_mfma_f32_16x16x32_f16 (16 output features per MFMA
// tile), the rows of x the B operand (16 columns, zero past M). Codes reach the MFMA as
// exact fp16 integers (built from their bits under the exponent of 1024, minus 1024), x as
// fp16 after scaling each row of a staged chunk by a power of two that puts its largest
// magnitude in [2^14, 2^15) (exact for bf16 values), so no product is rounded before the
// fp32 accumulation:
//   y[m][n] = sum_g ( s[n][g] * sum_{k in g} code[n][k] x[m][k] + b[n][g] * sum_{k in g} x[m][k] )
// One accumulator per group of 64 inputs carries s[n][g]; scale and bias enter through
// mixed fp16/fp32 fma.
//
// Grid: (ceil(N / 128) row tiles) x (key splits of K). A workgroup stages x for 512 inputs
// at a time in LDS (fp16, its row sums per group) with the (scale, bias) of its 128 rows,
// and each wave streams the codes of its 32 rows straight from HBM into registers, all of a
// chunk's loads issued before the first MFMA. With several splits each writes a partial
// y, and a second kernel sums them in split order (deterministic).
#include "vsa_internal.h"

namespace vsa {

namespace {

constexpr int kQThreads = 256;
constexpr int kQTiles = 2;                    // 16-row MFMA tiles per wave
constexpr int kQRows = 4 * 16 * kQTiles;      // rows per workgroup
constexpr int kQChunk = 512;                  // inputs per staged x chunk
constexpr int kQGroups = kQChunk / 64;
constexpr int kQStride = kQChunk + 8;         // fp16 per staged x row (16-byte pad)

typedef _Float16 qh8 __attribute__((ext_vector_type(8)));
typedef _Float16 qh2 __attribute__((ext_vector_type(2)));
typedef float qf4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ qh2 q_pair(uint32_t d) {
    return __builtin_bit_cast(qh2, d) - qh2{(_Float16)1024.f, (_Float16)1024.f};
}
// 8 codes -> fp16 integers. 8-bit: bytes of w0, w1 in order. 4-bit: nibbles of w in order,
// returned as (0, 4, 1, 5, 2, 6, 3, 7) (x is staged in the same order).
__device__ __forceinline__ qh8 q_codes8(uint32_t w0, uint32_t w1) {
    constexpr uint32_t kExp = 0x64646464u;    // byte select: 0..3 from w, 4 = 0x64
    const qh2 p0 = q_pair(__builtin_amdgcn_perm(kExp, w0, 0x04010400u));
    const qh2 p1 = q_pair(__builtin_amdgcn_perm(kExp, w0, 0x04030402u));
    const qh2 p2 = q_pair(__builtin_amdgcn_perm(kExp, w1, 0x04010400u));
    const qh2 p3 = q_pair(__builtin_amdgcn_perm(kExp, w1, 0x04030402u));
    return qh8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
__device__ __forceinline__ qh8 q_codes4(uint32_t w) {
    const qh2 p0 = q_pair((w & 0x000F000Fu) | 0x64006400u);
    const qh2 p1 = q_pair(((w >> 4) & 0x000F000Fu) | 0x64006400u);
    const qh2 p2 = q_pair(((w >> 8) & 0x000F000Fu) | 0x64006400u);
    const qh2 p3 = q_pair(((w >> 12) & 0x000F000Fu) | 0x64006400u);
    return qh8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
__device__ __forceinline__ float q_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float q_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

template <int BITS>
__global__ __launch_bounds__(256) void qmm_kernel(const QmmArgs a) {
    constexpr int CW = BITS == 8 ? 4 : 2;     // code dwords per lane per group (16 inputs)
    __shared__ __attribute__((aligned(16))) _Float16 xs[16 * kQStride];
    __shared__ float xsum[kQGroups][16];
    __shared__ __attribute__((aligned(16))) uint32_t sbs[kQGroups][kQRows];
    __shared__ uint32_t xmax[16];

    const int tile = blockIdx.x / a.nsplit, split = blockIdx.x % a.nsplit;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = tile * kQRows;
    const int kb = split * a.ksplit;
    const int ke = min(a.K, kb + a.ksplit);
    const int r = lane & 15, q = lane >> 4;   // A: row r, inputs 16 q .. 16 q + 15 of a group
    const int m = lane & 15;                  // B / D: column m (row of x)

    // rows of this lane's A operand (clamped: rows past N load row N - 1, never stored)
    const uint32_t* crow[kQTiles];
#pragma unroll
    for (int j = 0; j < kQTiles; ++j) {
        const int n = min(row0 + wave * 32 + j * 16 + r, a.N - 1);
        crow[j] = reinterpret_cast<const uint32_t*>(a.codes + (size_t)n * a.rowbytes);
    }
    qf4 acc_total[kQTiles];
#pragma unroll
    for (int j = 0; j < kQTiles; ++j) acc_total[j] = qf4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = kb; k0 < ke; k0 += kQChunk) {
        const int klen = min(kQChunk, ke - k0);   // a multiple of 64
        const int ng = klen / 64;
        // ---- this chunk's codes: every load issued before any compute
        uint32_t cw[kQTiles][kQGroups][CW];
#pragma unroll
        for (int g = 0; g < kQGroups; ++g)
#pragma unroll
            for (int j = 0; j < kQTiles; ++j) {
                if (g < ng) {
                    const int dw = ((k0 + 64 * g + 16 * q) * BITS / 8) / 4;
                    if constexpr (BITS == 8) {
                        const uint4 v = *reinterpret_cast<const uint4*>(crow[j] + dw);
                        cw[j][g][0] = v.x; cw[j][g][1] = v.y; cw[j][g][2] = v.z; cw[j][g][3] = v.w;
                    } else {
                        const uint2 v = *reinterpret_cast<const uint2*>(crow[j] + dw);
                        cw[j][g][0] = v.x; cw[j][g][1] = v.y;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < CW; ++c) cw[j][g][c] = 0u;
                }
            }
        // ---- stage x: 16 rows x klen inputs, 8 per thread-slot
        if (tid < 16) xmax[tid] = 0u;
        __syncthreads();                          // previous chunk's readers are done too
        float xv[4][8];
        int xm[4], xk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = (tid + kQThreads * i) * 8;
            xm[i] = e / kQChunk;
            xk[i] = e % kQChunk;
            uint4 raw = make_uint4(0u, 0u, 0u, 0u);
            if (xm[i] < a.M && xk[i] < klen)
                raw = *reinterpret_cast<const uint4*>(a.x + (size_t)xm[i] * a.K + k0 + xk[i]);
            const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
            uint32_t mx = 0u;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                xv[i][2 * t] = __uint_as_float(wd[t] << 16);
                xv[i][2 * t + 1] = __uint_as_float(wd[t] & 0xFFFF0000u);
                mx = max(mx, (wd[t] << 16) & 0x7FFFFFFFu);
                mx = max(mx, wd[t] & 0x7FFF0000u);
            }
            if (mx) atomicMax(&xmax[xm[i]], mx);  // |x| bit patterns order as the values
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mxf = __uint_as_float(xmax[xm[i]]);
            int qe = 0;
            if (mxf > 0.f && mxf <= 3.0e38f) {
                int ex;
                (void)__builtin_frexpf(mxf, &ex);
                qe = 15 - ex;
            }
            qh8 h;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int pos = BITS == 4 ? (t < 4 ? 2 * t : 2 * (t - 4) + 1) : t;
                h[pos] = (_Float16)__builtin_ldexpf(xv[i][t], qe);
            }
            *reinterpret_cast<qh8*>(&xs[xm[i] * kQStride + xk[i]]) = h;
        }
        // (scale, bias) of the 128 rows for the chunk's groups, [group][row]
        for (int i = tid; i < kQRows * kQGroups; i += kQThreads) {
            const int rr = i / kQGroups, g = i % kQGroups;
            const int n = row0 + rr;
            sbs[g][rr] = (n < a.N && g < ng)
                             ? reinterpret_cast<const uint32_t*>(a.sb)[(size_t)n * a.sbrow +
                                                                        k0 / 64 + g]
                             : 0u;
        }
        __syncthreads();
        // per-group sums of the staged (scaled) x: the bias term
        if (tid < 16 * kQGroups) {
            const int mm = tid & 15, g = tid >> 4;
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const qh8 h = *reinterpret_cast<const qh8*>(&xs[mm * kQStride + 64 * g + 8 * c]);
#pragma unroll
                for (int t = 0; t < 8; ++t) s += (float)h[t];
            }
            xsum[g][mm] = s;
        }
        __syncthreads();

        // ---- per group: two MFMAs per tile into a fresh accumulator, then scale and bias
        const float mxf = __uint_as_float(xmax[m]);
        int qe = 0;
        if (mxf > 0.f && mxf <= 3.0e38f) {
            int ex;
            (void)__builtin_frexpf(mxf, &ex);
            qe = 15 - ex;
        }
        qf4 acc_c[kQTiles];
#pragma unroll
        for (int j = 0; j < kQTiles; ++j) acc_c[j] = qf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < kQGroups; ++g) {
            if (g >= ng) break;
            const qh8 b0 = *reinterpret_cast<const qh8*>(&xs[m * kQStride + 64 * g + 16 * q]);
            const qh8 b1 = *reinterpret_cast<const qh8*>(&xs[m * kQStride + 64 * g + 16 * q + 8]);
            const float xsg = xsum[g][m];
#pragma unroll
            for (int j = 0; j < kQTiles; ++j) {
                qh8 a0, a1;
                if constexpr (BITS == 8) {
                    a0 = q_codes8(cw[j][g][0], cw[j][g][1]);
                    a1 = q_codes8(cw[j][g][2], cw[j][g][3]);
                } else {
                    a0 = q_codes4(cw[j][g][0]);
                    a1 = q_codes4(cw[j][g][1]);
                }
                qf4 t = qf4{0.f, 0.f, 0.f, 0.f};
                t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, t, 0, 0, 0);
                const uint4 s4 = *reinterpret_cast<const uint4*>(&sbs[g][wave * 32 + j * 16 + 4 * q]);
                const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    acc_c[j][rr] = __builtin_fmaf(q_lo(sw[rr]), t[rr],
                                                  __builtin_fmaf(q_hi(sw[rr]), xsg, acc_c[j][rr]));
            }
        }
        const float unscale = __builtin_ldexpf(1.f, -qe);
#pragma unroll
        for (int j = 0; j < kQTiles; ++j)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                acc_total[j][rr] = __builtin_fmaf(acc_c[j][rr], unscale, acc_total[j][rr]);
    }

    // ---- D layout: this lane holds rows 4 q .. 4 q + 3 of each tile, column m
    if (m >= a.M) return;
    float* dst = a.nsplit == 1 ? a.y : a.part + (size_t)split * a.M * a.N;
#pragma unroll
    for (int j = 0; j < kQTiles; ++j) {
        const int n = row0 + wave * 32 + j * 16 + 4 * q;
        float* p = dst + (size_t)m * a.N + n;
        if (n + 3 < a.N && (a.N & 3) == 0) {
            *reinterpret_cast<float4*>(p) =
                make_float4(acc_total[j][0], acc_total[j][1], acc_total[j][2], acc_total[j][3]);
        } else {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                if (n + rr < a.N) p[rr] = acc_total[j][rr];
        }
    }
}

// y = sum over splits of the partials, in split order.
__global__ __launch_bounds__(256) void qmm_reduce_kernel(const QmmArgs a) {
    const size_t total = (size_t)a.M * a.N;
    const size_t i = (size_t)blockIdx.x * kQThreads + threadIdx.x;
    if (i >= total) return;
    float s = 0.f;
    for (int sp = 0; sp < a.nsplit; ++sp) s += a.part[(size_t)sp * total + i];
    a.y[i] = s;
}

}  // namespace

QmmPlan plan_qmm(int M, int N, int K) {
    QmmPlan p{};
    p.tiles = (int)(((long)N + kQRows - 1) / kQRows);
    // about two workgroups per CU over the 256 CUs, splits of at least one chunk
    const int groups = K / 64;
    int nsplit = (512 + p.tiles - 1) / p.tiles;
    const int max_split = (groups + kQGroups - 1) / kQGroups;
    if (nsplit > max_split) nsplit = max_split;
    if (nsplit < 1) nsplit = 1;
    const int gps = (groups + nsplit - 1) / nsplit;          // groups per split
    p.ksplit = gps * 64;
    p.nsplit = (groups + gps - 1) / gps;
    // partial sums after the common workspace header (error word and counters), so the
    // workspace may be shared with the other calls
    p.bytes = p.nsplit > 1 ? kWsHeader + ((size_t)p.nsplit * M * N * 4 + 255) / 256 * 256 : 0;
    return p;
}

hipError_t launch_qmm(const QmmArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.tiles * a.nsplit)), block(kQThreads);
    if (a.bits == 8) hipLaunchKernelGGL(qmm_kernel<8>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(qmm_kernel<4>, grid, block, 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const size_t total = (size_t)a.M * a.N;
    hipLaunchKernelGGL(qmm_reduce_kernel, dim3((unsigned)((total + kQThreads - 1) / kQThreads)),
                       block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace vsa
