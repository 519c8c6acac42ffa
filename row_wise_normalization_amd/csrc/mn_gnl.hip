// mn_gnl.hip -- GroupNorm over channels-last activations X [N][L][C] (L
// positions, C channels contiguous per position: the NHWC layout), on gfx950.
// Same definition as the channels-first GroupNorm (Wu and He, "Group
// Normalization"; one of the row-wise norms of the [meTile] coverage
// inventory, "Normalization": group/channel layouts and affine gradients):
// groups of Cg = C / G consecutive channels, LayerNorm statistics over the
// M = Cg * L values of each (sample, group), per-channel gamma and beta.
//
// A group's values are strided in this layout (Cg channels out of every
// position's C), so no workgroup holds a (sample, group) in registers.
// Instead every pass streams whole positions, each lane owning VEC
// consecutive channels, and the group-wide quantities go through memory:
//
//   forward   1. per position chunk j of sample n and channel c:
//                S1 = sum (x - s_c), S2 = sum (x - s_c)^2, with the shift
//                s_c = X[n][0][c] (a value of the channel itself, so the
//                sums carry no cancellation from a large mean);
//             2. per (n, g), in binary64 from those sums: the group sum
//                sum_x = sum_{c,j} (n_j s_c + S1), mean = sum_x / M, and the
//                centred sum of squares as the exact expansion
//                sum_{c,j} (S2 + 2 d_c S1 + n_j d_c^2), d_c = s_c - mean;
//                rstd = 1 / sqrt(M2 / M + eps);
//             3. y = (x - mean) rstd gamma_c + beta_c.
//   backward  1. per chunk j and channel c: sum dY xhat and sum dY;
//             2. per (n, g): the per-sample channel sums P_c, Q_c (the
//                dgamma, dbeta partials, chunks added in order) and the
//                group sums A = sum gamma_c P_c, B = sum gamma_c Q_c;
//             3. dX = rstd (gamma_c dY - B / M - xhat A / M);
//             then the column reduce adds the N per-sample partial rows.
//
// X (and dY) are read twice, so the forward moves 1.5 times and the
// backward 1.67 times the algorithmic bytes. Every sum has a fixed order
// (rows of a lane in order, the row slots of a workgroup in order, chunks in
// order, workgroup trees in wave order): results are bitwise reproducible.
#include "mn_kernels.hpp"

namespace mn {
namespace kern {

constexpr int kGnlBlock = 256;  // lanes per workgroup
constexpr int kGnlUnroll = 8;   // positions whose loads a lane issues together

// Lane geometry of a streaming workgroup: it covers positions [l0, l1) of
// sample n (chunk j) and channel block cb, that is chunks cb * 256 ..
// cb * 256 + ck - 1 of VEC channels each. Lane t owns chunk k = t % ck of
// the block at positions l0 + r, l0 + r + rp, ... (r = t / ck, rp = 256 / ck
// row slots); lanes with r >= rp are idle.
struct GnlLane {
    int64_t n;
    int j, l0, l1, ck, rp, r, c;
    bool act;
    __device__ __forceinline__ GnlLane(const GnlArgs& a, int vec)
    {
        n = blockIdx.x / a.J;
        j = (int)(blockIdx.x % a.J);
        const int cb = blockIdx.y;
        ck = min(kGnlBlock, a.CK - cb * kGnlBlock);
        rp = kGnlBlock / ck;
        const int t = threadIdx.x;
        r = t / ck;
        c = (cb * kGnlBlock + t % ck) * vec;
        act = r < rp;
        l0 = j * a.LC;
        l1 = min(a.L, l0 + a.LC);
    }
    // element offset of this lane's chunk at position l
    __device__ __forceinline__ int64_t off(const GnlArgs& a, int l) const
    {
        return (n * a.L + l) * (int64_t)a.C + c;
    }
};

// Per-group values (mean, rstd, or the backward's A and B) of each of the
// lane's VEC channels: v[(n * G + g) * stride + off] for g = (c + e) / Cg.
// A chunk of VEC consecutive channels spans at most two groups when
// Cg >= VEC, so two loads serve it; narrower groups load per channel.
template <int VEC>
__device__ __forceinline__ void gnl_group_vals(const GnlArgs& a, const GnlLane& w, const float* v,
                                               int stride, int off, float (&dst)[VEC])
{
    const int g0 = w.c / a.Cg;
    if (VEC == 1 || a.Cg >= VEC) {
        const int g1 = min(g0 + 1, a.G - 1);
        const float v0 = v[(w.n * a.G + g0) * stride + off];
        const float v1 = v[(w.n * a.G + g1) * stride + off];
#pragma unroll
        for (int e = 0; e < VEC; ++e) dst[e] = (w.c + e) / a.Cg == g0 ? v0 : v1;
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) dst[e] = v[(w.n * a.G + (w.c + e) / a.Cg) * stride + off];
    }
}

// gamma (or beta) of the lane's VEC channels, one raw load per chunk.
template <int VEC>
__device__ __forceinline__ void gnl_params(const void* p, int pdt, int c, float (&dst)[VEC])
{
    if constexpr (VEC == 1) {
        load_scalar_param(p, pdt, c, dst[0]);
    } else {
        PRaw<VEC> raw;
        load_param_raw<VEC>(p, pdt, c, raw);
        widen_param<VEC>(raw, pdt, true, dst);
    }
}

// Fixed-order sum over the workgroup of one value per thread (binary64 or
// binary32): the wave's lanes by a butterfly, then the waves in order; every
// thread receives the total.
template <typename V>
__device__ __forceinline__ V gnl_block_sum(V v, V* buf)
{
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m);
    __syncthreads();  // earlier readers of buf are done
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
    __syncthreads();
    V t = buf[0];
#pragma unroll
    for (int w = 1; w < kGnlBlock / 64; ++w) t += buf[w];
    return t;
}

// Step 1 of both directions. MODE 0 (forward): S1 = sum (x - s_c) into sa,
// S2 = sum (x - s_c)^2 into sb. MODE 1 (backward): sum dY xhat into sa, sum dY
// into sb. Each lane sums its positions in order; the row slots of the
// workgroup are then added in slot order through LDS.
template <int MODE, int ST, int VEC>
__global__ void __launch_bounds__(kGnlBlock) gnl_sum_kernel(const GnlArgs a)
{
    typedef typename Chunk<ST, VEC>::type CV;
    __shared__ float red[2][kGnlBlock * VEC];
    const GnlLane w(a, VEC);
    float s1[VEC], s2[VEC], p0[VEC], p1[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        s1[e] = 0.0f;
        s2[e] = 0.0f;
        p0[e] = 0.0f;
        p1[e] = 0.0f;
    }
    if (w.act) {
        if constexpr (MODE == 0) {
            // the shift: this sample's value of the channel at position 0
            const CV sh = sload<ST, VEC, 0>(a.X, w.off(a, 0));
#pragma unroll
            for (int e = 0; e < VEC; ++e) p0[e] = cget<ST, VEC>(sh, e);
        } else {
            gnl_group_vals<VEC>(a, w, a.mean, 1, 0, p0);
            gnl_group_vals<VEC>(a, w, a.rstd, 1, 0, p1);
        }
        for (int l = w.l0 + w.r; l < w.l1; l += w.rp * kGnlUnroll) {
            CV xv[kGnlUnroll], dv[kGnlUnroll];
#pragma unroll
            for (int u = 0; u < kGnlUnroll; ++u) {
                // positions past the chunk re-read a valid one, unused; plain
                // (temporal) loads, so that the apply pass finds much of X
                // (and dY) still in the memory-side cache
                const int lu = l + u * w.rp < w.l1 ? l + u * w.rp : l;
                xv[u] = sload<ST, VEC, 0>(a.X, w.off(a, lu));
                if constexpr (MODE == 1) dv[u] = sload<ST, VEC, 0>(a.dY, w.off(a, lu));
            }
#pragma unroll
            for (int u = 0; u < kGnlUnroll; ++u) {
                if (l + u * w.rp >= w.l1) break;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float x = cget<ST, VEC>(xv[u], e);
                    if constexpr (MODE == 0) {
                        const float d = x - p0[e];
                        s1[e] += d;
                        s2[e] = __builtin_fmaf(d, d, s2[e]);
                    } else {
                        const float dy = cget<ST, VEC>(dv[u], e);
                        const float xh = (x - p0[e]) * p1[e];
                        s1[e] = __builtin_fmaf(dy, xh, s1[e]);
                        s2[e] += dy;
                    }
                }
            }
        }
    }
    // row slots in order: slot r of chunk k at red[.][(r * ck + k) * VEC + e]
    const int k = threadIdx.x % w.ck;
    if (w.act) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            red[0][(w.r * w.ck + k) * VEC + e] = s1[e];
            red[1][(w.r * w.ck + k) * VEC + e] = s2[e];
        }
    }
    __syncthreads();
    if (w.act && w.r == 0) {
        for (int q = 1; q < w.rp; ++q) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                s1[e] += red[0][(q * w.ck + k) * VEC + e];
                s2[e] += red[1][(q * w.ck + k) * VEC + e];
            }
        }
        const int64_t o = (w.n * a.J + w.j) * (int64_t)a.C + w.c;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            a.sa[o + e] = s1[e];
            a.sb[o + e] = s2[e];
        }
    }
}

// Forward step 2: the mean and rstd of (sample, group) blockIdx.x from the
// chunk sums, in binary64.
template <int ST>
__global__ void __launch_bounds__(kGnlBlock) gnl_stats_kernel(const GnlArgs a)
{
    __shared__ double buf[kGnlBlock / 64];
    const int64_t s = blockIdx.x;
    const int64_t n = s / a.G;
    const int g = (int)(s % a.G);
    const int64_t E = (int64_t)a.Cg * a.J;  // (channel, chunk) entries
    const double M = (double)a.Cg * (double)a.L;
    auto entry = [&](int64_t e, double& shift, double& rows, double& S1, double& S2) {
        const int c = g * a.Cg + (int)(e % a.Cg);
        const int j = (int)(e / a.Cg);
        const int l0 = j * a.LC;
        rows = (double)(min(a.L, l0 + a.LC) - l0);
        shift = (double)static_cast<const typename Elem<ST>::type*>(a.X)[n * a.L * (int64_t)a.C + c];
        const int64_t o = (n * a.J + j) * (int64_t)a.C + c;
        S1 = (double)a.sa[o];
        S2 = (double)a.sb[o];
    };
    double sx = 0.0;
    for (int64_t e = threadIdx.x; e < E; e += kGnlBlock) {
        double sh, rows, S1, S2;
        entry(e, sh, rows, S1, S2);
        sx += rows * sh + S1;
    }
    const double mean = gnl_block_sum(sx, buf) / M;
    double m2 = 0.0;
    for (int64_t e = threadIdx.x; e < E; e += kGnlBlock) {
        double sh, rows, S1, S2;
        entry(e, sh, rows, S1, S2);
        const double d = sh - mean;
        m2 += S2 + 2.0 * d * S1 + rows * d * d;
    }
    const double M2 = gnl_block_sum(m2, buf);
    if (threadIdx.x == 0) {
        const double var = (M2 > 0.0 ? M2 : 0.0) / M;
        a.mean[s] = (float)mean;
        a.rstd[s] = (float)(1.0 / sqrt(var + (double)a.eps));
    }
}

// Backward step 2: per channel of (sample, group) blockIdx.x, the chunk sums
// added in order (the per-sample dgamma and dbeta partials), and the group
// sums A = sum gamma_c P_c, B = sum gamma_c Q_c.
__global__ void __launch_bounds__(kGnlBlock) gnl_merge_kernel(const GnlArgs a)
{
    __shared__ float buf[kGnlBlock / 64];
    const int64_t s = blockIdx.x;
    const int64_t n = s / a.G;
    const int g = (int)(s % a.G);
    float A = 0.0f, B = 0.0f;
    for (int i = threadIdx.x; i < a.Cg; i += kGnlBlock) {
        const int c = g * a.Cg + i;
        float P = 0.0f, Q = 0.0f;
        int j = 0;
        for (; j + 8 <= a.J; j += 8) {
            float vp[8], vq[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t o = (n * a.J + j + q) * (int64_t)a.C + c;
                vp[q] = a.sa[o];
                vq[q] = a.sb[o];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                P += vp[q];
                Q += vq[q];
            }
        }
        for (; j < a.J; ++j) {
            const int64_t o = (n * a.J + j) * (int64_t)a.C + c;
            P += a.sa[o];
            Q += a.sb[o];
        }
        a.part_g[n * a.Cp + c] = P;
        a.part_b[n * a.Cp + c] = Q;
        float gam;
        load_scalar_param(a.gamma, a.pdt, c, gam);
        A = __builtin_fmaf(gam, P, A);
        B = __builtin_fmaf(gam, Q, B);
    }
    A = gnl_block_sum(A, buf);
    B = gnl_block_sum(B, buf);
    if (threadIdx.x == 0) {
        a.ab[2 * s] = A;
        a.ab[2 * s + 1] = B;
    }
}

// Step 3 of both directions: MODE 0 writes y = (x - mean) rstd gamma + beta,
// MODE 1 dX = rstd (gamma dY - B / M - xhat A / M) in storage type OT.
template <int MODE, int ST, int OT, int VEC>
__global__ void __launch_bounds__(kGnlBlock) gnl_apply_kernel(const GnlArgs a)
{
    typedef typename Chunk<ST, VEC>::type CV;
    typedef typename Chunk<OT, VEC>::type OV;
    const GnlLane w(a, VEC);
    if (!w.act) return;  // no barrier below
    float mu[VEC], rs[VEC], gm[VEC], bt[VEC], c1[VEC], c2[VEC];
    const float fM = (float)a.Cg * (float)a.L;
    gnl_group_vals<VEC>(a, w, a.mean, 1, 0, mu);
    gnl_group_vals<VEC>(a, w, a.rstd, 1, 0, rs);
    gnl_params<VEC>(a.gamma, a.pdt, w.c, gm);
    if constexpr (MODE == 0) {
        gnl_params<VEC>(a.beta, a.pdt, w.c, bt);
    } else {
        gnl_group_vals<VEC>(a, w, a.ab, 2, 0, c1);
        gnl_group_vals<VEC>(a, w, a.ab, 2, 1, c2);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            c1[e] = c1[e] / fM;
            c2[e] = c2[e] / fM;
        }
    }
    // the last reads of X (and dY): plain loads in the forward, streaming
    // (non-temporal) ones in the backward, each the faster at 32 x 4096 x 320
    constexpr int LNT = MODE == 0 ? 0 : 2;
    for (int l = w.l0 + w.r; l < w.l1; l += w.rp * kGnlUnroll) {
        CV xv[kGnlUnroll], dv[kGnlUnroll];
#pragma unroll
        for (int u = 0; u < kGnlUnroll; ++u) {
            const int lu = l + u * w.rp < w.l1 ? l + u * w.rp : l;
            xv[u] = sload<ST, VEC, LNT>(a.X, w.off(a, lu));
            if constexpr (MODE == 1) dv[u] = sload<ST, VEC, LNT>(a.dY, w.off(a, lu));
        }
#pragma unroll
        for (int u = 0; u < kGnlUnroll; ++u) {
            const int lu = l + u * w.rp;
            if (lu >= w.l1) break;
            OV o;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float xh = (cget<ST, VEC>(xv[u], e) - mu[e]) * rs[e];
                if constexpr (MODE == 0) {
                    cset<OT, VEC>(o, e, __builtin_fmaf(xh, gm[e], bt[e]));
                } else {
                    const float gg = cget<ST, VEC>(dv[u], e) * gm[e];
                    cset<OT, VEC>(o, e, rs[e] * __builtin_fmaf(-xh, c1[e], gg - c2[e]));
                }
            }
            cstore<OT, VEC, 1>(MODE == 0 ? a.Y : a.dX, w.off(a, lu), o);
        }
    }
}

}  // namespace kern

// ---------------------------------------------------------------------------
// Planning and launches.
// ---------------------------------------------------------------------------

namespace {

// Streaming workgroups to aim for (the position chunks of all samples): the
// sums pass and the apply pass each take their own chunking. About four per
// CU measured best for both at 32 x 4096 x 320 (against 2, 8 and 16 for the
// sums pass and 2 for the apply pass).
constexpr int64_t kGnlSumBlocks = 1024;
constexpr int64_t kGnlApplyBlocks = 1024;
constexpr int64_t kGnlMaxChunks = 256;      // position chunks per sample

int32_t chunks_for(int64_t N, int64_t L, int64_t target)
{
    int64_t J = (target + N - 1) / N;
    if (J > kGnlMaxChunks) J = kGnlMaxChunks;
    if (J > L) J = L;
    if (J < 1) J = 1;
    // equal chunks of LC positions; the last one may be shorter
    const int64_t LC = (L + J - 1) / J;
    return (int32_t)((L + LC - 1) / LC);
}

// The same arguments with the apply pass's position chunks.
GnlArgs apply_args(const GnlArgs& a)
{
    GnlArgs b = a;
    b.J = chunks_for(a.N, a.L, kGnlApplyBlocks);
    b.LC = (int32_t)((a.L + b.J - 1) / b.J);
    return b;
}

}  // namespace

int32_t gnl_chunks(int64_t N, int64_t L) { return chunks_for(N, L, kGnlSumBlocks); }

int64_t gnl_workspace_floats(int64_t N, int64_t L, int64_t C, int64_t G)
{
    const int64_t J = gnl_chunks(N, L);
    const int64_t Cp = (C + 3) / 4 * 4;
    return 2 * N * J * C + 2 * N * Cp + 2 * N * G;
}

void gnl_geometry(int st, bool vec_ok, GnlArgs& a, int& vec)
{
    vec = vec_ok ? (st == ST_F32 ? 4 : 8) : 1;
    a.CK = a.C / vec;
    const int64_t LC = (a.L + a.J - 1) / a.J;
    a.LC = (int32_t)LC;
}

namespace {

template <int ST, int VEC>
hipError_t gnl_fwd_t(const GnlArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)a.N * a.J), (unsigned)((a.CK + kern::kGnlBlock - 1) /
                                                               kern::kGnlBlock));
    hipLaunchKernelGGL((kern::gnl_sum_kernel<0, ST, VEC>), grid, dim3(kern::kGnlBlock), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kern::gnl_stats_kernel<ST>), dim3((unsigned)((int64_t)a.N * a.G)),
                       dim3(kern::kGnlBlock), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const GnlArgs b = apply_args(a);
    const dim3 gridb((unsigned)((int64_t)b.N * b.J), grid.y);
    hipLaunchKernelGGL((kern::gnl_apply_kernel<0, ST, ST, VEC>), gridb, dim3(kern::kGnlBlock), 0,
                       s, b);
    return hipGetLastError();
}

template <int ST, int OT, int VEC>
hipError_t gnl_bwd_t(const GnlArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)a.N * a.J), (unsigned)((a.CK + kern::kGnlBlock - 1) /
                                                               kern::kGnlBlock));
    hipLaunchKernelGGL((kern::gnl_sum_kernel<1, ST, VEC>), grid, dim3(kern::kGnlBlock), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern::gnl_merge_kernel, dim3((unsigned)((int64_t)a.N * a.G)),
                       dim3(kern::kGnlBlock), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const GnlArgs b = apply_args(a);
    const dim3 gridb((unsigned)((int64_t)b.N * b.J), grid.y);
    hipLaunchKernelGGL((kern::gnl_apply_kernel<1, ST, OT, VEC>), gridb, dim3(kern::kGnlBlock), 0,
                       s, b);
    return hipGetLastError();
}

template <int ST>
hipError_t gnl_fwd_st(int vec, const GnlArgs& a, hipStream_t s)
{
    constexpr int V = ST == ST_F32 ? 4 : 8;
    return vec == 1 ? gnl_fwd_t<ST, 1>(a, s) : gnl_fwd_t<ST, V>(a, s);
}

template <int ST, int OT>
hipError_t gnl_bwd_st(int vec, const GnlArgs& a, hipStream_t s)
{
    constexpr int V = ST == ST_F32 ? 4 : 8;
    return vec == 1 ? gnl_bwd_t<ST, OT, 1>(a, s) : gnl_bwd_t<ST, OT, V>(a, s);
}

}  // namespace

hipError_t launch_gnl_fwd(int st, int vec, const GnlArgs& a, hipStream_t s)
{
    switch (st) {
    case ST_F16: return gnl_fwd_st<ST_F16>(vec, a, s);
    case ST_BF16: return gnl_fwd_st<ST_BF16>(vec, a, s);
    case ST_F32: return gnl_fwd_st<ST_F32>(vec, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gnl_bwd(int st, int ot, int vec, const GnlArgs& a, hipStream_t s)
{
    if (st == ST_F16) return ot == ST_F32 ? gnl_bwd_st<ST_F16, ST_F32>(vec, a, s)
                                          : gnl_bwd_st<ST_F16, ST_F16>(vec, a, s);
    if (st == ST_BF16) return ot == ST_F32 ? gnl_bwd_st<ST_BF16, ST_F32>(vec, a, s)
                                           : gnl_bwd_st<ST_BF16, ST_BF16>(vec, a, s);
    if (st == ST_F32) return gnl_bwd_st<ST_F32, ST_F32>(vec, a, s);
    return hipErrorInvalidValue;
}

}  // namespace mn
