// mn_groupnorm.hpp -- GroupNorm forward and backward on gfx950 (Wu and He,
// "Group Normalization"), one of the row-wise norms the [meTile] coverage
// inventory lists ("Normalization": group/channel layouts and affine
// gradients).
//
// X is [N][C][L] (L positions per channel, contiguous); the C channels form
// G groups of Cg = C / G consecutive channels, so the (sample, group) slice
// s = n * G + g is Cg contiguous channel rows of L values, and rows
// s * Cg .. s * Cg + Cg - 1 of X viewed as [N * C][L].
//
// One workgroup owns one slice and holds it in registers: row groups of T
// lanes each own channel rows r = gi, gi + R, ... (R row groups, U rows per
// group), lane l owning CPT chunks of VEC values at column (k * T + l) * VEC.
//   forward:  the slice mean (workgroup sum), then the centred mean square
//             from the registers (two passes, as LayerNorm), then
//             y = (x - mean) * rstd * gamma[c] + beta[c] per channel c;
//   backward: per channel row, P = sum_l dY * xhat and Q = sum_l dY (the row
//             reduction of the row kernels), written per sample as the
//             [N][C] partials of dgamma and dbeta; the slice sums
//             A = sum_c gamma[c] P_c, B = sum_c gamma[c] Q_c in channel-row
//             group order; dX = rstd * (gamma[c] dY - B / M - xhat A / M),
//             M = Cg * L, with dY for this last pass partly from LDS (the
//             first chunks of each lane, staged after the first pass) and
//             partly read again. A second kernel (the column reduce) adds
//             the N partial rows of dgamma and dbeta in fixed order.
// Every load is unconditional (row and column indices past the slice are
// clamped; their values are masked out), every sum has a fixed order.
#pragma once

#include "mn_kernels.hpp"

namespace mn {
namespace kern {

constexpr int kGnMaxBlock = 1024;

// Sum of one value per thread over the `nw` waves of the workgroup: the wave
// tree, then the waves in order; every thread receives the total.
__device__ __forceinline__ float gn_block_sum(float v, float* buf, int nw)
{
    v = group_sum<64>(v);
    __syncthreads();  // earlier readers of buf are done
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = buf[0];
    for (int w = 1; w < nw; ++w) t += buf[w];
    return t;
}

template <int ST, int T, int VEC, int CPT, int U>
struct GnSlice {
    typedef typename Chunk<ST, VEC>::type HV;
    HV x[U][CPT];
    int r[U];            // channel row within the slice (clamped)
    int rv;              // bit u: row u is a row of the slice
    int64_t base;        // first element of the slice
    int l, L;

    // validity and clamped element offset of chunk (u, k)
    __device__ __forceinline__ bool ok(int u, int k) const
    {
        return ((rv >> u) & 1) && (k * T + l) * VEC < L;
    }
    __device__ __forceinline__ int64_t off(int u, int k) const
    {
        return base + (int64_t)r[u] * L + min((k * T + l) * VEC, L - VEC);
    }
};

// This lane's rows of slice s.
template <int ST, int T, int VEC, int CPT, int U>
__device__ __forceinline__ void gn_map(GnSlice<ST, T, VEC, CPT, U>& t, const GnArgs& a, int s,
                                       int gi, int l, int rpb)
{
    // Rows of at least a wave: every lane of a wave is in the same row group,
    // so its rows (and their gamma and beta) are wave-uniform and live in
    // scalar registers.
    if (T >= 64) gi = __builtin_amdgcn_readfirstlane(gi);
    t.base = (int64_t)s * a.Cg * a.L;
    t.l = l;
    t.L = a.L;
    t.rv = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = gi + rpb * u;
        if (r < a.Cg) t.rv |= 1 << u;
        t.r[u] = min(r, a.Cg - 1);
    }
}

template <int ST, int T, int VEC, int CPT, int U>
__global__ void __launch_bounds__(kGnMaxBlock) gn_fwd_kernel(const GnArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    __shared__ float buf[kGnMaxBlock / 64];
    const int tid = threadIdx.x;
    const int gi = tid / T, l = tid % T;
    const int rpb = blockDim.x / T;
    const int nw = blockDim.x >> 6;
    const int s = blockIdx.x;
    const int grp = s % a.G;

    GnSlice<ST, T, VEC, CPT, U> t;
    gn_map(t, a, s, gi, l, rpb);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k) t.x[u][k] = sload<ST, VEC, 2>(a.X, t.off(u, k));
    float gam[U], bet[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        load_scalar_param(a.gamma, a.pdt, grp * a.Cg + t.r[u], gam[u]);
        load_scalar_param(a.beta, a.pdt, grp * a.Cg + t.r[u], bet[u]);
    }

    const float fM = (float)a.Cg * (float)a.L;
    float s1 = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) s1 += t.ok(u, k) ? cget<ST, VEC>(t.x[u][k], e) : 0.0f;
    // the fp32 values of the first pass are not kept across the reduction
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k) launder(t.x[u][k]);
    const float mu = gn_block_sum(s1, buf, nw) / fM;
    float s2 = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float c = t.ok(u, k) ? cget<ST, VEC>(t.x[u][k], e) - mu : 0.0f;
                s2 = __builtin_fmaf(c, c, s2);
            }
    const float rs = 1.0f / sqrtf(gn_block_sum(s2, buf, nw) / fM + a.eps);
    if (tid == 0) {
        a.mean[s] = mu;
        a.rstd[s] = rs;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            launder(t.x[u][k]);
            HV o;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                cset<ST, VEC>(o, e, __builtin_fmaf((cget<ST, VEC>(t.x[u][k], e) - mu) * rs,
                                                   gam[u], bet[u]));
            if (t.ok(u, k)) cstore<ST, VEC, 1>(a.Y, t.off(u, k), o);
        }
}

template <int ST, int OT, int T, int VEC, int CPT, int U>
__global__ void __launch_bounds__(kGnMaxBlock) gn_bwd_kernel(const GnArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    typedef typename Chunk<OT, VEC>::type OV;
    constexpr int RMAX = kGnMaxBlock / T;   // row groups at most
    __shared__ float red[RedBuf<T, RMAX, 2 * U>::size];
    __shared__ float sums[2][RMAX];
    const int tid = threadIdx.x;
    const int gi = tid / T, l = tid % T;
    const int rpb = blockDim.x / T;
    const int s = blockIdx.x;
    const int n = s / a.G;
    const int grp = s % a.G;

    // dY staging: the first a.sk chunks of each lane, lane-private 16-byte
    // slots [chunk][lane] (16-byte chunks only)
    extern __shared__ u4 gn_stage[];
    constexpr bool STAGE = sizeof(HV) == 16;
    GnSlice<ST, T, VEC, CPT, U> t;
    gn_map(t, a, s, gi, l, rpb);
    HV dy[U][CPT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            t.x[u][k] = sload<ST, VEC, 2>(a.X, t.off(u, k));
            dy[u][k] = sload<ST, VEC, 0>(a.dY, t.off(u, k));
        }
    float gam[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load_scalar_param(a.gamma, a.pdt, grp * a.Cg + t.r[u], gam[u]);
    const float mu = a.mean[s];
    const float rs = a.rstd[s];

    // per channel row: P = sum dY * xhat, Q = sum dY
    float v[2 * U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float p = 0.0f, q = 0.0f;
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float xh = (cget<ST, VEC>(t.x[u][k], e) - mu) * rs;
                const float d = t.ok(u, k) ? cget<ST, VEC>(dy[u][k], e) : 0.0f;
                p = __builtin_fmaf(d, xh, p);
                q += d;
            }
        v[2 * u] = p;
        v[2 * u + 1] = q;
    }
    if constexpr (STAGE) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k)
                if (u * CPT + k < a.sk)
                    gn_stage[(u * CPT + k) * blockDim.x + tid] = __builtin_bit_cast(u4, dy[u][k]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k) launder(t.x[u][k]);
    int phase = 0;
    row_sum<T, RMAX, 2 * U>(v, red, phase, gi, l);

    // per-sample partials of dgamma and dbeta; the slice sums by row group
    float ag = 0.0f, bg = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool rv = gi + rpb * u < a.Cg;
        if (rv) {
            ag = __builtin_fmaf(gam[u], v[2 * u], ag);
            bg = __builtin_fmaf(gam[u], v[2 * u + 1], bg);
            if (l == 0) {
                const int64_t c = (int64_t)n * a.Cp + grp * a.Cg + t.r[u];
                a.part_g[c] = v[2 * u];
                a.part_b[c] = v[2 * u + 1];
            }
        }
    }
    if (l == 0) {
        sums[0][gi] = ag;
        sums[1][gi] = bg;
    }
    __syncthreads();
    float A = sums[0][0], B = sums[1][0];
    for (int g2 = 1; g2 < rpb; ++g2) {
        A += sums[0][g2];
        B += sums[1][g2];
    }
    const float fM = (float)a.Cg * (float)a.L;
    const float c1 = A / fM, c2 = B / fM;
    // dY again rather than held in registers across the reductions: the
    // staged chunks from LDS, the rest from memory (this workgroup read them
    // moments ago: mostly Infinity Cache hits)
    HV dy2[U][CPT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            if constexpr (STAGE) {
                if (u * CPT + k < a.sk)
                    dy2[u][k] = __builtin_bit_cast(HV, gn_stage[(u * CPT + k) * blockDim.x + tid]);
                else
                    dy2[u][k] = sload<ST, VEC, 0>(a.dY, t.off(u, k));
            } else {
                dy2[u][k] = sload<ST, VEC, 0>(a.dY, t.off(u, k));
            }
        }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            launder(t.x[u][k]);
            OV o;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float xh = (cget<ST, VEC>(t.x[u][k], e) - mu) * rs;
                const float gg = cget<ST, VEC>(dy2[u][k], e) * gam[u];
                cset<OT, VEC>(o, e, rs * __builtin_fmaf(-xh, c1, gg - c2));
            }
            if (t.ok(u, k)) cstore<OT, VEC, 1>(a.dX, t.off(u, k), o);
        }
}

}  // namespace kern
}  // namespace mn

namespace mn {

// Launch shapes. Vector path (16-byte chunks; L a multiple of the chunk and
// aligned rows), chosen by the smallest max_l >= L:
//   shape  T  CPT  max_l
#define MN_GN_VEC_SHAPES(X) \
    X(0, 8, 1, 64)          \
    X(1, 16, 1, 128)        \
    X(2, 32, 1, 256)        \
    X(3, 64, 1, 512)        \
    X(4, 128, 1, 1024)      \
    X(5, 256, 1, 2048)      \
    X(6, 256, 2, 4096)      \
    X(7, 512, 2, 8192)      \
    X(8, 1024, 2, 16384)
// Element-wise path (any L, any alignment).
#define MN_GN_ELEM_SHAPES(X) \
    X(9, 64, 4, 256)         \
    X(10, 256, 8, 2048)      \
    X(11, 1024, 16, 16384)
// Rows per row group U: 1 to 8, kept within the register budget of a
// 1024-lane workgroup (128 VGPRs): the backward holds U * CPT chunks of X per
// lane across its reductions and as many of dY in its last pass. 16-byte
// chunks: at most 10 for rows of up to 256 lanes, 8 for 512 lanes and 4 for
// 1024 lanes (whose cross-wave row sums take more registers), halved for
// binary32, whose chunks are twice as many; element chunks: at most 16. A
// launch id is shape * 8 + U - 1.
constexpr bool gn_fits(int st, int vec, int t, int cpt, int u)
{
    if (u > 8) return false;
    if (vec == 1) return u * cpt <= 16;
    const int lim = t >= 1024 ? 4 : t >= 512 ? 8 : 10;
    return u * cpt <= (st == ST_F32 ? lim / 2 : lim);
}

// The forward holds only X across its reductions, so its rows per row group
// go up to 16 and, for rows of 64 to 256 lanes, 20 chunks per lane (80 VGPRs
// of fp16 data; a row group is then wave-uniform, so gamma, beta and the row
// indices sit in scalar registers), which lets one row group of 256 lanes
// hold a whole 10 x 4096 slice; rows of fewer than 64 lanes keep per-lane
// row indices and stop at 12 chunks. Forward launch ids are shape * 16 + U - 1.
constexpr int kGnFwdMaxU = 16;
constexpr bool gn_fits_fwd(int st, int vec, int t, int cpt, int u)
{
    if (u > kGnFwdMaxU) return false;
    if (vec == 1) return u * cpt <= 16;
    const int lim = t >= 1024 ? 4 : t >= 512 ? 8 : t >= 64 ? 20 : 12;
    return u * cpt <= (st == ST_F32 ? lim / 2 : lim);
}

template <int ST, int OT>
hipError_t launch_gn_bwd_t(const GnPlan& p, const GnArgs& a, hipStream_t s);
template <int ST>
hipError_t launch_gn_fwd_t(const GnPlan& p, const GnArgs& a, hipStream_t s);

}  // namespace mn
