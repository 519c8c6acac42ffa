// mn_groupnorm.hpp -- GroupNorm forward and backward on gfx950 (Wu and He,
// "Group Normalization"), one of the row-wise norms the [meTile] coverage
// inventory lists ("Normalization": group/channel layouts and affine
// gradients).
//
// X is [N][C][L] (L positions per channel, contiguous); the C channels form
// G groups of Cg = C / G consecutive channels, so the (sample, group) slice
// s = n * G + g is Cg contiguous channel rows of L values, and rows
// s * Cg .. s * Cg + Cg - 1 of X viewed as [N * C][L]. With M = Cg * L:
//   forward:  mean and rstd of the slice (centred variance), then
//             y = (x - mean) * rstd * gamma[c] + beta[c] per channel c;
//   backward: per channel row, P_c = sum_l dY * xhat and Q_c = sum_l dY
//             (the per-sample partials of dgamma and dbeta); the slice sums
//             A = sum_c gamma[c] P_c, B = sum_c gamma[c] Q_c; then
//             dX = rstd * (gamma[c] dY - B / M - xhat A / M).
// A column reduce (the row kernels' stage 2) adds the N per-sample partial
// rows of dgamma and dbeta in fixed order.
//
// Register path (a slice fits one workgroup): persistent workgroups, slice
// b, b + P, b + 2P, ... for workgroup b of P. The workgroup holds the slice
// in registers -- row groups of T lanes each own U channel rows, lane l
// owning CPT chunks of VEC values at column (k * T + l) * VEC -- reduces it
// and writes it from there; with PF = 1 the next slice's loads are in flight
// meanwhile (a second register set), so the chip's reads and writes overlap
// instead of coming in phases. Every load of the loop is unconditional, so
// the compiler counts them and waits for the current slice's data only,
// never for the prefetch or for earlier stores.
//
// Split path (larger slices): the work is cut into units that many
// workgroups share, and the slice-wide quantities go through memory between
// launches, each combined in a fixed order:
//   forward:  per statistics chunk (FL contiguous values of a slice) its mean
//             and centred sum of squares M2; one workgroup per slice merges
//             the chunks (the pairwise update of Chan, Golub and LeVeque:
//             counts add, M2 gains delta^2 * na * nb / n); then the apply pass
//             over row units;
//   backward: per row unit (up to UL values of one channel row) its sums of
//             dY * xhat and dY; one workgroup per slice adds each channel's
//             units in order (the dgamma, dbeta partials) and the slice sums
//             A and B; then the apply pass over row units.
// The forward keeps its chunk statistics in the output Y (overwritten by the
// apply pass), so its signature needs no workspace.
//
// Every load is unconditional (rows, columns, units and slices past the end
// are clamped to valid ones; their values are masked out), every sum has a
// fixed order, no floating-point atomics: bitwise reproducible.
#pragma once

#include "mn_kernels.hpp"

namespace mn {
namespace kern {

constexpr int kGnMaxBlock = 1024;
constexpr int kGnUnitBlock = 256;  // split path workgroups

// Chunks per lane of one split-path unit: 16-byte chunks, or 32 single
// values on the element-wise path (64 VGPRs for X and dY together).
template <int VEC>
constexpr int gn_unit_it()
{
    return VEC == 1 ? 32 : 8;
}

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

// Chunk load and store at a 32-bit element offset from a base pointer. With
// a wave-uniform base (a slice or a channel row) the compiler addresses each
// chunk with the scalar base and one 32-bit register, where a 64-bit address
// per chunk would hold twice the registers across the reductions.
// (The byte offset is formed in 32 bits, so that the address is visibly the
// base plus a zero-extended 32-bit register.)
template <int ST, int VEC, int NT>
__device__ __forceinline__ typename Chunk<ST, VEC>::type gload(const void* base, uint32_t off)
{
    typedef typename Chunk<ST, VEC>::type C;
    const uint32_t b = off * (uint32_t)sizeof(typename Elem<ST>::type);
    const C* p = reinterpret_cast<const C*>(static_cast<const char*>(base) + b);
    if constexpr ((NT & 2) != 0) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int ST, int VEC, int NT>
__device__ __forceinline__ void gstore(void* base, uint32_t off, const typename Chunk<ST, VEC>::type& v)
{
    typedef typename Chunk<ST, VEC>::type C;
    const uint32_t b = off * (uint32_t)sizeof(typename Elem<ST>::type);
    C* p = reinterpret_cast<C*>(static_cast<char*>(base) + b);
    if constexpr ((NT & 1) != 0) __builtin_nontemporal_store(v, p);
    else *p = v;
}


// A parameter element of PW bytes (binary32, or binary16 / bfloat16), loaded
// raw in one instruction without a branch (a load in the arms of a branch
// costs the compiler its count of the loads in flight, and it then waits
// for all of them), and widened by param_f32 where it is used, so that a
// persistent loop can issue it with the next slice's data. binary32 goes
// through the scalar cache where the index is wave-uniform.
template <int PW>
__device__ __forceinline__ uint32_t param_raw(const void* base, int64_t i)
{
    if constexpr (PW == 4) {
        typedef const __attribute__((address_space(4))) uint32_t cu32;
        return ((cu32*)base)[i];
    } else {
        return static_cast<const uint16_t*>(base)[i];
    }
}

// An fp32 element read through the scalar cache (a wave-uniform index into
// an array the kernel does not write): it lands in a scalar register and is
// waited for on its own counter, apart from the vector loads in flight.
__device__ __forceinline__ float scalar_f32(const float* p, int64_t i)
{
    typedef const __attribute__((address_space(4))) float cfloat;
    return ((cfloat*)p)[i];
}

template <int PW>
__device__ __forceinline__ float param_f32(uint32_t raw, int pdt)
{
    if constexpr (PW == 4) return __uint_as_float(raw);
    const float b = __uint_as_float(raw << 16);
    const float h = (float)__builtin_bit_cast(_Float16, (uint16_t)raw);
    return pdt == ST_BF16 ? b : h;
}

// Base pointer of element `off` of an array of storage type ST.
template <int ST>
__device__ __forceinline__ const void* at(const void* p, int64_t off)
{
    return static_cast<const typename Elem<ST>::type*>(p) + off;
}
template <int ST>
__device__ __forceinline__ void* at(void* p, int64_t off)
{
    return static_cast<typename Elem<ST>::type*>(p) + off;
}

// Sums of NV values per row group of T lanes (every lane of the group gets
// the same bits). Wider than a wave: the wave sums go through LDS, the lane
// l < NV of each row group adds value l's wave sums in wave order, and every
// lane reads the NV totals back. (Each lane adding all NV * T / 64 wave sums
// itself, as the row kernels do for their few sums, held them all in
// registers at once: 80 at 10 sums over 8 waves.) Two barriers; `wsum`
// holds RMAX * (T / 64) * NV floats, `tot` RMAX * NV.
template <int T, int RMAX, int NV>
__device__ __forceinline__ void gn_row_sum(float (&v)[NV], float* wsum, float* tot, int g, int l)
{
    if constexpr (T <= 64) {
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = group_sum<T>(v[i]);
    } else {
        constexpr int WPR = T / 64;
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = group_sum<64>(v[i]);
        if ((l & 63) == 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i) wsum[(g * WPR + (l >> 6)) * NV + i] = v[i];
        }
        __syncthreads();
        if (l < NV) {
            float t = wsum[(g * WPR) * NV + l];
#pragma unroll
            for (int w = 1; w < WPR; ++w) t += wsum[(g * WPR + w) * NV + l];
            tot[g * NV + l] = t;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = tot[g * NV + i];
    }
}

// This lane's channel rows within any slice: the same for every slice.
template <int T, int VEC, int CPT, int U>
struct GnRows {
    int r[U];            // channel row within the slice (clamped)
    int rv;              // bit u: row u is a row of the slice
    int l, L;

    __device__ __forceinline__ bool ok(int u, int k) const
    {
        return ((rv >> u) & 1) && (k * T + l) * VEC < L;
    }
    // element offset of chunk (u, k) within the slice (columns past the row
    // clamped to its last chunk) as a lane part and a wave-uniform part:
    // with rows of at least a wave the row's offset is uniform, so a chunk
    // costs one offset register per column k rather than per (u, k)
    __device__ __forceinline__ uint32_t voff(int u, int k) const
    {
        const uint32_t c = (uint32_t)min((k * T + l) * VEC, L - VEC);
        return T >= 64 ? c : c + (uint32_t)(r[u] * L);
    }
    __device__ __forceinline__ uint32_t soff(int u) const
    {
        return T >= 64 ? (uint32_t)(r[u] * L) : 0u;
    }
};

template <int T, int VEC, int CPT, int U>
__device__ __forceinline__ void gn_map(GnRows<T, VEC, CPT, U>& t, const GnArgs& a, int gi, int l,
                                       int rpb)
{
    // Rows of at least a wave: every lane of a wave is in the same row group,
    // so its rows (and their gamma and beta) are wave-uniform and live in
    // scalar registers.
    if (T >= 64) gi = __builtin_amdgcn_readfirstlane(gi);
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

// PW: bytes per gamma / beta element (4, or 2 for either 16-bit type)
template <int ST, int T, int VEC, int CPT, int U, int PF, int PW>
__global__ void __launch_bounds__(kGnMaxBlock) gn_fwd_kernel(const GnArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    __shared__ float buf[kGnMaxBlock / 64];
    const int tid = threadIdx.x;
    const int gi = tid / T, l = tid % T;
    const int rpb = blockDim.x / T;
    const int nw = blockDim.x >> 6;
    const int64_t M = (int64_t)a.Cg * a.L;
    const float fM = (float)a.Cg * (float)a.L;

    GnRows<T, VEC, CPT, U> t;
    gn_map(t, a, gi, l, rpb);

    struct Tile {
        HV x[U][CPT];
        uint32_t gam[U], bet[U];  // raw parameters (param_raw)
    };
    constexpr int64_t ES = sizeof(typename Elem<ST>::type);
    const uint32_t MB = (uint32_t)(M * ES);
    auto load = [&](Tile& tl, int64_t s) {
        const __amdgpu_buffer_rsrc_t xs = slice_rsrc(a.X, s * M * ES, MB);
        const int grp = (int)(s % a.G);
        // the small loads first: the compiler's waits for them then leave
        // the chunk loads in flight
#pragma unroll
        for (int u = 0; u < U; ++u) {
            tl.gam[u] = param_raw<PW>(a.gamma, grp * a.Cg + t.r[u]);
            tl.bet[u] = param_raw<PW>(a.beta, grp * a.Cg + t.r[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k) tl.x[u][k] = bload<ST, VEC, 2>(xs, t.voff(u, k), t.soff(u));
    };
    auto process = [&](Tile& tl, int64_t s) {
        const __amdgpu_buffer_rsrc_t ys = slice_rsrc(a.Y, s * M * ES, MB);
        void* yp = at<ST>(a.Y, s * M);
        float s1 = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    s1 += t.ok(u, k) ? cget<ST, VEC>(tl.x[u][k], e) : 0.0f;
        // the fp32 values of the first pass are not kept across the reduction
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k) launder(tl.x[u][k]);
        const float mu = gn_block_sum(s1, buf, nw) / fM;
        float s2 = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float c = t.ok(u, k) ? cget<ST, VEC>(tl.x[u][k], e) - mu : 0.0f;
                    s2 = __builtin_fmaf(c, c, s2);
                }
        const float rs = 1.0f / sqrtf(gn_block_sum(s2, buf, nw) / fM + a.eps);
        if (tid == 0) {
            a.mean[s] = mu;
            a.rstd[s] = rs;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float gam = param_f32<PW>(tl.gam[u], a.pdt);
            const float bet = param_f32<PW>(tl.bet[u], a.pdt);
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                launder(tl.x[u][k]);
                HV o;
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    cset<ST, VEC>(o, e, __builtin_fmaf((cget<ST, VEC>(tl.x[u][k], e) - mu) * rs,
                                                       gam, bet));
                // one slice per workgroup at a time (PF = 0): plain stores
                // under the mask, whose addresses hold fewer registers
                if constexpr (PF)
                    bstore<ST, VEC, 1>(ys, t.voff(u, k), t.soff(u), t.ok(u, k), o);
                else if (t.ok(u, k))
                    cstore<ST, VEC, 1>(yp, (int64_t)t.voff(u, k) + t.soff(u), o);
            }
        }
    };

    int64_t s = blockIdx.x;
    Tile cur;
    load(cur, s);
    if constexpr (PF) {
        for (;;) {
            const int64_t sn = s + gridDim.x;
            Tile nxt;
            load(nxt, sn < a.S ? sn : a.S - 1);
            // keep the prefetch ahead of the work on this slice (the
            // scheduler would otherwise sink it to shorten its live range)
            __builtin_amdgcn_sched_barrier(0);
            process(cur, s);
            if (sn >= a.S) break;
            cur = nxt;
            s = sn;
        }
    } else {
        for (;;) {
            process(cur, s);
            s += gridDim.x;
            if (s >= a.S) break;
            load(cur, s);
        }
    }
}

template <int ST, int OT, int T, int VEC, int CPT, int U, int PF, int PW>
__global__ void __launch_bounds__(kGnMaxBlock) gn_bwd_kernel(const GnArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    typedef typename Chunk<OT, VEC>::type OV;
    constexpr int RMAX = kGnMaxBlock / T;   // row groups at most
    constexpr int WPR = T > 64 ? T / 64 : 1;
    __shared__ float wsum[T > 64 ? RMAX * WPR * 2 * U : 1];
    __shared__ float tot[T > 64 ? RMAX * 2 * U : 1];
    // slice sums per row group, double buffered by slice parity: a wave may
    // write the next slice's while another still reads this slice's (rows
    // of at most a wave reduce without a barrier)
    __shared__ float sums[2][2][RMAX];
    const int tid = threadIdx.x;
    const int gi = tid / T, l = tid % T;
    const int rpb = blockDim.x / T;
    const int64_t M = (int64_t)a.Cg * a.L;
    const float fM = (float)a.Cg * (float)a.L;

    GnRows<T, VEC, CPT, U> t;
    gn_map(t, a, gi, l, rpb);

    struct Tile {
        HV x[U][CPT], dy[U][CPT];
        float mu, rs;
    };
    constexpr int64_t ES = sizeof(typename Elem<ST>::type);
    constexpr int64_t OS = sizeof(typename Elem<OT>::type);
    const uint32_t MB = (uint32_t)(M * ES);
    auto load = [&](Tile& tl, int64_t s) {
        const __amdgpu_buffer_rsrc_t xs = slice_rsrc(a.X, s * M * ES, MB);
        const __amdgpu_buffer_rsrc_t ds = slice_rsrc(a.dY, s * M * ES, MB);
        tl.mu = scalar_f32(a.mean, s);
        tl.rs = scalar_f32(a.rstd, s);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                tl.x[u][k] = bload<ST, VEC, 2>(xs, t.voff(u, k), t.soff(u));
                tl.dy[u][k] = bload<ST, VEC, 2>(ds, t.voff(u, k), t.soff(u));
            }
    };
    // gamma of the slice's rows, loaded as its iteration begins, ahead of
    // the next slice's chunk loads (so the wait for it leaves them in
    // flight); it is first needed after the row sums. (Loaded one slice
    // ahead with the chunks, it held registers across a whole iteration.)
    auto load_gam = [&](uint32_t (&g)[U], int64_t s) {
        const int grp = (int)(s % a.G);
#pragma unroll
        for (int u = 0; u < U; ++u) g[u] = param_raw<PW>(a.gamma, grp * a.Cg + t.r[u]);
    };
    auto process = [&](Tile& tl, const uint32_t (&graw)[U], int64_t s, int par) {
        const __amdgpu_buffer_rsrc_t dxs = slice_rsrc(a.dX, s * M * OS, (uint32_t)(M * OS));
        void* dxp = at<OT>(a.dX, s * M);
        const int64_t n = s / a.G;
        const int grp = (int)(s % a.G);
        const float mu = tl.mu, rs = tl.rs;
        float gam[U];
#pragma unroll
        for (int u = 0; u < U; ++u) gam[u] = param_f32<PW>(graw[u], a.pdt);
        // per channel row: P = sum dY * xhat, Q = sum dY
        float v[2 * U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float p = 0.0f, q = 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float xh = (cget<ST, VEC>(tl.x[u][k], e) - mu) * rs;
                    const float d = t.ok(u, k) ? cget<ST, VEC>(tl.dy[u][k], e) : 0.0f;
                    p = __builtin_fmaf(d, xh, p);
                    q += d;
                }
            v[2 * u] = p;
            v[2 * u + 1] = q;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                launder(tl.x[u][k]);
                launder(tl.dy[u][k]);
            }
        gn_row_sum<T, RMAX, 2 * U>(v, wsum, tot, gi, l);

        // per-sample partials of dgamma and dbeta (the first lane of each
        // row group writes its rows'); the slice sums by row group
        const __amdgpu_buffer_rsrc_t pg = slice_rsrc(a.part_g, n * a.Cp * 4, (uint32_t)a.Cp * 4);
        const __amdgpu_buffer_rsrc_t pb = slice_rsrc(a.part_b, n * a.Cp * 4, (uint32_t)a.Cp * 4);
        float ag = 0.0f, bg = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool rv = (t.rv >> u) & 1;
            ag = rv ? __builtin_fmaf(gam[u], v[2 * u], ag) : ag;
            bg = rv ? __builtin_fmaf(gam[u], v[2 * u + 1], bg) : bg;
            const uint32_t c = (rv && l == 0) ? (uint32_t)(grp * a.Cg + t.r[u]) * 4u : kNoStore;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[2 * u]), pg, c, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[2 * u + 1]), pb, c, 0, 0);
        }
        if (l == 0) {
            sums[par][0][gi] = ag;
            sums[par][1][gi] = bg;
        }
        __syncthreads();
        float A = sums[par][0][0], B = sums[par][1][0];
        for (int g2 = 1; g2 < rpb; ++g2) {
            A += sums[par][0][g2];
            B += sums[par][1][g2];
        }
        const float c1 = A / fM, c2 = B / fM;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                OV o;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float xh = (cget<ST, VEC>(tl.x[u][k], e) - mu) * rs;
                    const float gg = cget<ST, VEC>(tl.dy[u][k], e) * gam[u];
                    cset<OT, VEC>(o, e, rs * __builtin_fmaf(-xh, c1, gg - c2));
                }
                if constexpr (PF)
                    bstore<OT, VEC, 1>(dxs, t.voff(u, k), t.soff(u), t.ok(u, k), o);
                else if (t.ok(u, k))
                    cstore<OT, VEC, 1>(dxp, (int64_t)t.voff(u, k) + t.soff(u), o);
            }
    };

    int64_t s = blockIdx.x;
    int par = 0;
    Tile cur;
    load(cur, s);
    if constexpr (PF) {
        for (;;) {
            const int64_t sn = s + gridDim.x;
            uint32_t g[U];
            load_gam(g, s);
            Tile nxt;
            load(nxt, sn < a.S ? sn : a.S - 1);
            // keep the prefetch ahead of the work on this slice (the
            // scheduler would otherwise sink it to shorten its live range)
            __builtin_amdgcn_sched_barrier(0);
            process(cur, g, s, par);
            if (sn >= a.S) break;
            cur = nxt;
            s = sn;
            par ^= 1;
        }
    } else {
        for (;;) {
            uint32_t g[U];
            load_gam(g, s);
            process(cur, g, s, par);
            s += gridDim.x;
            if (s >= a.S) break;
            load(cur, s);
            par ^= 1;
        }
    }
}

// ---------------------------------------------------------------------------
// Split path.
// ---------------------------------------------------------------------------

// Row unit of the split path: 256-lane workgroups of RG = 256 / T row
// groups; row group gi takes unit u = blockIdx.x * RG + gi, i.e. chunk
// k = u % Kr of channel row q = u / Kr (values k * UL .. k * UL + UL - 1 of
// the row, clamped to the row), lane l the values at
// k * UL + (i * T + l) * VEC, i < IT.
template <int T, int VEC>
struct GnUnit {
    int64_t u;           // unit (clamped to the last one)
    bool uok;            // the unit exists
    int64_t q;           // channel row of X viewed as [N * C][L]
    int64_t s;           // slice of the row
    int c;               // channel
    int c0;              // first column of this lane's values in the row
    int L;

    // REV: workgroups take the units from the last one back, so that a pass
    // re-reading X first reads what the pass before it read last (and may
    // still find it in the memory-side cache)
    template <bool REV = false>
    __device__ __forceinline__ void map(const GnArgs& a, int gi, int l)
    {
        constexpr int RG = kGnUnitBlock / T;
        const int64_t bx = REV ? (int64_t)gridDim.x - 1 - blockIdx.x : (int64_t)blockIdx.x;
        const int64_t uu = bx * RG + gi;
        uok = uu < a.units;
        u = uok ? uu : a.units - 1;
        q = u / a.Kr;
        s = q / a.Cg;
        c = (int)(q % a.C);
        c0 = (int)(u - q * a.Kr) * a.UL + l * VEC;
        L = a.L;
    }
    __device__ __forceinline__ bool ok(int i) const { return uok && c0 + i * T * VEC < L; }
    // offset of value i within the channel row (clamped to its last chunk)
    __device__ __forceinline__ uint32_t off(int i) const
    {
        return (uint32_t)min(c0 + i * T * VEC, L - VEC);
    }
};

// Backward, first pass: per row unit, the sums of dY * xhat and of dY.
template <int ST, int T, int VEC>
__global__ void __launch_bounds__(kGnUnitBlock) gn_unit_sums_kernel(const GnArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    constexpr int RG = kGnUnitBlock / T;
    constexpr int IT = gn_unit_it<VEC>();
    __shared__ float red[RedBuf<T, RG, 2>::size];
    const int gi = threadIdx.x / T, l = threadIdx.x % T;
    GnUnit<T, VEC> w;
    w.map(a, gi, l);
    const float mu = a.mean[w.s], rs = a.rstd[w.s];
    const void* xr = at<ST>(a.X, w.q * w.L);
    const void* dr = at<ST>(a.dY, w.q * w.L);
    HV x[IT], dy[IT];
    // plain (temporal) loads: the dX pass reads X and dY again
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        x[i] = gload<ST, VEC, 0>(xr, w.off(i));
        dy[i] = gload<ST, VEC, 0>(dr, w.off(i));
    }
    float v[2] = {0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float xh = (cget<ST, VEC>(x[i], e) - mu) * rs;
            const float d = w.ok(i) ? cget<ST, VEC>(dy[i], e) : 0.0f;
            v[0] = __builtin_fmaf(d, xh, v[0]);
            v[1] += d;
        }
    int phase = 0;
    row_sum<T, RG, 2>(v, red, phase, gi, l);
    if (w.uok && l == 0) {
        a.unit_p[w.u] = v[0];
        a.unit_q[w.u] = v[1];
    }
}

// Backward, merge: one workgroup per slice. Lane i takes the channels
// i, i + 256, ... of the slice: each channel's units added in order give its
// dgamma and dbeta partials, and the lane's sums of gamma * P and gamma * Q
// over its channels; the workgroup adds the lanes' sums (wave trees, then
// the waves in order) to the slice sums A and B.
// (Templated on the storage type only so that each storage type's
// translation unit has its own copy.)
template <int ST>
__global__ void __launch_bounds__(kGnUnitBlock) gn_unit_merge_kernel(const GnArgs a)
{
    __shared__ float buf[kGnUnitBlock / 64];
    const int64_t s = blockIdx.x;
    const int64_t n = s / a.G;
    const int grp = (int)(s % a.G);
    float ag = 0.0f, bg = 0.0f;
    for (int c = threadIdx.x; c < a.Cg; c += kGnUnitBlock) {
        const int ch = grp * a.Cg + c;
        const int64_t q = n * a.C + ch;
        float P = 0.0f, Q = 0.0f;
        for (int k = 0; k < a.Kr; ++k) {
            P += a.unit_p[q * a.Kr + k];
            Q += a.unit_q[q * a.Kr + k];
        }
        a.part_g[n * a.Cp + ch] = P;
        a.part_b[n * a.Cp + ch] = Q;
        float gm;
        load_scalar_param(a.gamma, a.pdt, ch, gm);
        ag = __builtin_fmaf(gm, P, ag);
        bg = __builtin_fmaf(gm, Q, bg);
    }
    const float A = gn_block_sum(ag, buf, kGnUnitBlock / 64);
    const float B = gn_block_sum(bg, buf, kGnUnitBlock / 64);
    if (threadIdx.x == 0) {
        a.slice_ab[2 * s] = A;
        a.slice_ab[2 * s + 1] = B;
    }
}

// Backward, apply: dX of one row unit per row group.
template <int ST, int OT, int T, int VEC>
__global__ void __launch_bounds__(kGnUnitBlock) gn_unit_dx_kernel(const GnArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    typedef typename Chunk<OT, VEC>::type OV;
    constexpr int IT = gn_unit_it<VEC>();
    const int gi = threadIdx.x / T, l = threadIdx.x % T;
    GnUnit<T, VEC> w;
    w.map(a, gi, l);
    const void* xr = at<ST>(a.X, w.q * w.L);
    const void* dr = at<ST>(a.dY, w.q * w.L);
    void* dxr = at<OT>(a.dX, w.q * w.L);
    HV x[IT], dy[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        x[i] = gload<ST, VEC, 2>(xr, w.off(i));
        dy[i] = gload<ST, VEC, 2>(dr, w.off(i));
    }
    const float mu = a.mean[w.s], rs = a.rstd[w.s];
    const float fM = (float)a.Cg * (float)a.L;
    const float c1 = a.slice_ab[2 * w.s] / fM, c2 = a.slice_ab[2 * w.s + 1] / fM;
    float gam;
    load_scalar_param(a.gamma, a.pdt, w.c, gam);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        OV o;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float xh = (cget<ST, VEC>(x[i], e) - mu) * rs;
            const float gg = cget<ST, VEC>(dy[i], e) * gam;
            cset<OT, VEC>(o, e, rs * __builtin_fmaf(-xh, c1, gg - c2));
        }
        if (w.ok(i)) gstore<OT, VEC, 1>(dxr, w.off(i), o);
    }
}

// Forward, statistics: chunk j of slice s (values j * FL .. of the slice,
// flat across its channel rows); its mean, then its centred sum of squares
// from the registers.
template <int ST, int VEC>
__global__ void __launch_bounds__(kGnUnitBlock) gn_chunk_stats_kernel(const GnArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    constexpr int IT = gn_unit_it<VEC>();
    __shared__ float buf[kGnUnitBlock / 64];
    const int64_t M = (int64_t)a.Cg * a.L;
    const int64_t s = blockIdx.x / a.Kf;
    const int j = (int)(blockIdx.x % a.Kf);
    const int64_t first = (int64_t)j * a.FL;
    const int cnt = (int)min((int64_t)a.FL, M - first);
    const void* xc = at<ST>(a.X, s * M + first);
    HV x[IT];
    // plain (temporal) loads: the y pass reads X again, from the last unit back
#pragma unroll
    for (int i = 0; i < IT; ++i)
        x[i] = gload<ST, VEC, 0>(xc, (uint32_t)min((i * kGnUnitBlock + (int)threadIdx.x) * VEC,
                                                  cnt - VEC));
    float s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            s1 += (i * kGnUnitBlock + (int)threadIdx.x) * VEC < cnt ? cget<ST, VEC>(x[i], e) : 0.0f;
    const float mc = gn_block_sum(s1, buf, kGnUnitBlock / 64) / (float)cnt;
    float s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float d = (i * kGnUnitBlock + (int)threadIdx.x) * VEC < cnt
                                ? cget<ST, VEC>(x[i], e) - mc : 0.0f;
            s2 = __builtin_fmaf(d, d, s2);
        }
    const float m2 = gn_block_sum(s2, buf, kGnUnitBlock / 64);
    if (threadIdx.x == 0) {
        const int64_t o = 2 * (s * a.Kf + j);
        a.stat[o] = mc;
        a.stat[o + 1] = m2;
    }
}

// The pairwise update: (na, ma, qa) <- (na, ma, qa) merged with (nb, mb, qb)
// (counts, means, centred sums of squares).
__device__ __forceinline__ void gn_merge(int64_t& na, float& ma, float& qa, int64_t nb, float mb,
                                         float qb)
{
    if (nb == 0) return;
    if (na == 0) {
        na = nb;
        ma = mb;
        qa = qb;
        return;
    }
    const int64_t n = na + nb;
    const float d = mb - ma;
    const float f = (float)nb / (float)n;
    ma = __builtin_fmaf(d, f, ma);
    qa = qa + qb + d * d * ((float)na * f);
    na = n;
}

// Forward, merge: one workgroup per slice. Lane i merges a contiguous range
// of the slice's chunks in order; the 256 lane results are merged by a fixed
// pairwise tree (lane i with lane i + h, h halving); then mean and rstd.
// (Templated on the storage type as gn_unit_merge_kernel.)
template <int ST>
__global__ void __launch_bounds__(kGnUnitBlock) gn_stats_merge_kernel(const GnArgs a)
{
    __shared__ int64_t tn[kGnUnitBlock];
    __shared__ float tm[kGnUnitBlock], tq[kGnUnitBlock];
    const int64_t M = (int64_t)a.Cg * a.L;
    const int64_t s = blockIdx.x;
    const int tid = threadIdx.x;
    const int j0 = (int)((int64_t)tid * a.Kf / kGnUnitBlock);
    const int j1 = (int)((int64_t)(tid + 1) * a.Kf / kGnUnitBlock);
    int64_t n = 0;
    float m = 0.0f, q = 0.0f;
    for (int j = j0; j < j1; ++j) {
        const int64_t first = (int64_t)j * a.FL;
        const int64_t cnt = M - first < a.FL ? M - first : a.FL;
        gn_merge(n, m, q, cnt, a.stat[2 * (s * a.Kf + j)], a.stat[2 * (s * a.Kf + j) + 1]);
    }
    tn[tid] = n;
    tm[tid] = m;
    tq[tid] = q;
    __syncthreads();
    for (int h = kGnUnitBlock / 2; h > 0; h >>= 1) {
        if (tid < h) {
            int64_t na = tn[tid];
            float ma = tm[tid], qa = tq[tid];
            gn_merge(na, ma, qa, tn[tid + h], tm[tid + h], tq[tid + h]);
            tn[tid] = na;
            tm[tid] = ma;
            tq[tid] = qa;
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.mean[s] = tm[0];
        a.rstd[s] = 1.0f / sqrtf(tq[0] / (float)M + a.eps);
    }
}

// Forward, apply: y of one row unit per row group.
template <int ST, int T, int VEC>
__global__ void __launch_bounds__(kGnUnitBlock) gn_unit_y_kernel(const GnArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    constexpr int IT = gn_unit_it<VEC>();
    const int gi = threadIdx.x / T, l = threadIdx.x % T;
    GnUnit<T, VEC> w;
    w.template map<true>(a, gi, l);
    const void* xr = at<ST>(a.X, w.q * w.L);
    void* yr = at<ST>(a.Y, w.q * w.L);
    HV x[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) x[i] = gload<ST, VEC, 2>(xr, w.off(i));
    const float mu = a.mean[w.s], rs = a.rstd[w.s];
    float gam, bet;
    load_scalar_param(a.gamma, a.pdt, w.c, gam);
    load_scalar_param(a.beta, a.pdt, w.c, bet);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        HV o;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            cset<ST, VEC>(o, e, __builtin_fmaf((cget<ST, VEC>(x[i], e) - mu) * rs, gam, bet));
        if (w.ok(i)) gstore<ST, VEC, 1>(yr, w.off(i), o);
    }
}

}  // namespace kern
}  // namespace mn

namespace mn {

// Register path launch shapes (T lanes per channel row, CPT chunks per
// lane). Vector path (16-byte chunks; L a multiple of the chunk and aligned
// rows); the planner weighs every shape whose rows hold L with at most half
// of the lanes idle (and always the smallest that holds L):
//   shape  T  CPT  max_l
#define MN_GN_VEC_SHAPES(X) \
    X(0, 8, 1, 64)          \
    X(1, 16, 1, 128)        \
    X(2, 32, 1, 256)        \
    X(3, 64, 1, 512)        \
    X(4, 128, 1, 1024)      \
    X(5, 256, 1, 2048)      \
    X(6, 256, 2, 4096)      \
    X(7, 512, 1, 4096)      \
    X(8, 512, 2, 8192)      \
    X(9, 1024, 1, 8192)     \
    X(10, 1024, 2, 16384)
// Element-wise path (any L, any alignment).
#define MN_GN_ELEM_SHAPES(X) \
    X(11, 64, 4, 256)        \
    X(12, 256, 8, 2048)      \
    X(13, 1024, 16, 16384)

// Rows per row group U: 1 to 8 (backward) or 16 (forward), kept within the
// register budget of a 1024-lane workgroup (128 VGPRs), counted in chunks
// per lane per register set (16-byte chunks: 4 VGPRs; element chunks: 1).
// The backward holds X and dY, the forward X only; with the next slice in
// flight (PF = 1) there are two register sets. Rows of 1024 lanes take
// fewer (their cross-wave row sums hold more registers), rows of fewer than
// 64 lanes too (their row indices, gamma and beta are per lane, not scalar),
// and so does a binary32 dX from 16-bit data (two stores per chunk).
// binary32 chunks are twice as many for the same row, which the table's CPT
// (in 16-bit chunks) absorbs by halving the limit. Every instance within
// these limits compiles without spilling (the build's resource report).
constexpr int kGnFwdMaxU = 16;
constexpr int kGnBwdMaxU = 8;
constexpr int gn_lim(bool fwd, int vec, int t, int pf, bool wide_dx, int pw)
{
    if (vec == 1) return pf ? 8 : 16;
    if (fwd) {
        if (pf) return t >= 1024 ? 4 : t >= 64 ? 8 : 6;
        return t >= 1024 ? 4 : t >= 512 ? 8 : t >= 64 ? 20 : 10;
    }
    if (pf) return t >= 1024 ? 2 : t >= 64 ? (wide_dx ? 4 : 5) : 3;
    return t >= 1024 ? 4 : t >= 512 ? 8 : t >= 64 ? 10 : 6;
}
// pw: bytes per gamma / beta element (4 for binary32, else 2)
constexpr bool gn_fits(bool fwd, int st, int ot, int vec, int t, int cpt, int u, int pf, int pw)
{
    if (u > (fwd ? kGnFwdMaxU : kGnBwdMaxU)) return false;
    const bool wide_dx = !fwd && vec != 1 && st != ST_F32 && ot == ST_F32;
    const int lim = gn_lim(fwd, vec, t, pf, wide_dx, pw);
    return u * cpt <= ((st == ST_F32 && vec != 1) ? lim / 2 : lim);
}
// launch id: ((shape * 2 + pf) * maxU + U - 1)
constexpr int gn_id(bool fwd, int shape, int pf, int u)
{
    return (shape * 2 + pf) * (fwd ? kGnFwdMaxU : kGnBwdMaxU) + u - 1;
}

template <int ST, int OT>
hipError_t launch_gn_bwd_t(const GnPlan& p, const GnArgs& a, hipStream_t s);
template <int ST>
hipError_t launch_gn_fwd_t(const GnPlan& p, const GnArgs& a, hipStream_t s);

}  // namespace mn
