// mn_kernels.hpp -- gfx950 (CDNA4) kernel templates of the row-wise
// normalization training pair: RMSNorm, LayerNorm and fused residual-add +
// RMSNorm, forward and backward, fp16 storage with fp32 arithmetic.
//
// Semantics: [meTile] "Kernel coverage and training scope", section "Exact
// native normalization contract"; [tensorcore] "Training kernels", sections
// "RMSnorm -- Llama-style" and "LayerNorm -- standard".
//
// Layout of the work (all row kernels):
//   * A row is handled by a row group of T lanes: T = 8..64 lanes of one
//     wave64 (several rows per wave for narrow rows) or T = 128..512 lanes
//     spanning 2..8 waves (wide rows).
//   * Lane l of a row group owns CPT chunks of VEC consecutive columns; chunk
//     k starts at column (k*T + l)*VEC, so each load instruction of a wave
//     covers one contiguous span (64 x 16 B = 1 KiB for VEC = 8) and the
//     chunks a lane owns are the same in every row. VEC = 8 (one 128-bit
//     load per chunk) needs D % 8 == 0 and 16-byte aligned rows; VEC = 1 is
//     the element-wise path for every other call.
//   * Rows are processed in tiles of RPB*U rows (RPB row groups per
//     workgroup, U rows per group per step). The forward gives each
//     workgroup a contiguous range of rows (one tile in the shipped plans);
//     the backward gives workgroup b the tiles b, b+P, b+2P, ..., so the
//     workgroups in flight always cover one contiguous band of rows. With
//     PF = 1 the loads of the next tile are issued before the current tile
//     is reduced, so HBM reads stay in flight while a wave reduces and
//     writes.
//   * Row sums are reduced inside a wave by DPP (quad permutes, half-row and
//     row mirrors) and lane exchanges across 16-lane rows; row groups wider
//     than a wave combine their per-wave sums through LDS in wave order.
//     Every lane of a row group ends with the bitwise same total.
//   * The backward keeps each lane's dgamma (dbeta) partials for its columns
//     in registers across all rows of the workgroup's range, folds the row
//     groups of the workgroup in group order through LDS, and writes one
//     fp32 partial row per workgroup. A second kernel reduces the partial
//     rows of each column in a fixed order. No floating-point atomics
//     anywhere, so every result is bitwise reproducible.
//   * NT is a bit mask: bit 0 writes the streamed outputs (Y, H, dX) with
//     non-temporal stores, bit 1 reads the streamed inputs (X, R, dY, dH)
//     with non-temporal loads; neither is kept in the caches.
#pragma once

#include "mn_internal.hpp"

namespace mn {
namespace kern {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

template <int VEC> struct HVec;
template <> struct HVec<8> { typedef h8 type; };
template <> struct HVec<1> { typedef _Float16 type; };

template <int VEC>
__device__ __forceinline__ typename HVec<VEC>::type hzero()
{
    typename HVec<VEC>::type z;
    _Float16 s = (_Float16)0.0f;
    z = s;  // splat for the vector type
    return z;
}

template <int VEC>
__device__ __forceinline__ typename HVec<VEC>::type hload(const _Float16* p)
{
    return *reinterpret_cast<const typename HVec<VEC>::type*>(p);
}

// Load of a streamed input row (read once per launch); NT bit 1 marks it
// non-temporal so it does not displace reusable lines in the caches.
template <int VEC, int NT>
__device__ __forceinline__ typename HVec<VEC>::type sload(const _Float16* p)
{
    typedef typename HVec<VEC>::type HV;
    if constexpr ((NT & 2) != 0) return __builtin_nontemporal_load(reinterpret_cast<const HV*>(p));
    else return *reinterpret_cast<const HV*>(p);
}

template <int VEC, int NT>
__device__ __forceinline__ void hstore(_Float16* p, const typename HVec<VEC>::type& v)
{
    typedef typename HVec<VEC>::type HV;
    if constexpr ((NT & 1) != 0) __builtin_nontemporal_store(v, reinterpret_cast<HV*>(p));
    else *reinterpret_cast<HV*>(p) = v;
}

template <int VEC>
__device__ __forceinline__ float hget(const typename HVec<VEC>::type& v, int e)
{
    if constexpr (VEC == 8) return (float)v[e];
    else return (float)v;
}

template <int VEC>
__device__ __forceinline__ void hset(typename HVec<VEC>::type& v, int e, float f)
{
    if constexpr (VEC == 8) v[e] = (_Float16)f;   // v_cvt_f16_f32: round to nearest even
    else v = (_Float16)f;
}

// Opaque register copy: afterwards the compiler cannot reuse fp32 values it
// derived from `v` earlier, so packed fp16 registers are widened again where
// needed instead of keeping every fp32 temporary live across a reduction
// (fewer VGPRs, more waves per SIMD).
template <typename V>
__device__ __forceinline__ void launder(V& v)
{
    asm volatile("" : "+v"(v));
}

// ---------------------------------------------------------------------------
// Wave-level sums.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 8, 16, 32 or 64); every lane of a
// group receives the same bits, because each step adds the same two partial
// sums in every lane (addition is commutative). Inside a 16-lane DPP row the
// partners come from DPP quad permutes and mirrors; across rows from a lane
// exchange (ds_bpermute) with lane ^ 16 and lane ^ 32.
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(G == 8 || G == 16 || G == 32 || G == 64, "group width");
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp<0x141>(v);  // row_half_mirror: lane i <-> 7 - i within 8 lanes
    if constexpr (G >= 16) v += dpp<0x140>(v);  // row_mirror: lane i <-> 15 - i within 16
    if constexpr (G >= 32) v += __shfl_xor(v, 16);
    if constexpr (G >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Sum NV values per row group of T lanes. For T <= 64 this stays inside the
// wave; for wider groups each wave's sums go through LDS (`red`, double
// buffered by `phase` so one barrier per call suffices) and are added in
// wave order. Must be called by every thread of the workgroup (uniform
// control flow) because of the barrier.
template <int T, int RPB, int NV>
__device__ __forceinline__ void row_sum(float (&v)[NV], float* red, int& phase, int g, int l)
{
    if constexpr (T <= 64) {
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = group_sum<T>(v[i]);
    } else {
        constexpr int WPR = T / 64;
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = group_sum<64>(v[i]);
        float* buf = red + (phase & 1) * (RPB * WPR * NV);
        const int w = l >> 6;
        if ((l & 63) == 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i) buf[(g * WPR + w) * NV + i] = v[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float t = buf[(g * WPR) * NV + i];
#pragma unroll
            for (int ww = 1; ww < WPR; ++ww) t += buf[(g * WPR + ww) * NV + i];
            v[i] = t;
        }
        ++phase;
    }
}

template <int T, int RPB, int NV>
struct RedBuf {
    static constexpr int size = (T > 64) ? 2 * RPB * (T / 64) * NV : 1;
};

// ---------------------------------------------------------------------------
// Forward: Y (and H), rstd (and mean).
// ---------------------------------------------------------------------------

template <int KIND, int T, int VEC, int CPT, int U, int BLOCK, int PF, int NT>
__global__ void __launch_bounds__(BLOCK) fwd_kernel(const FwdArgs a)
{
    typedef typename HVec<VEC>::type HV;
    constexpr int RPB = BLOCK / T;
    constexpr int TILE = RPB * U;
    static_assert(BLOCK % T == 0, "block holds whole row groups");
    __shared__ float red[RedBuf<T, RPB, U>::size];

    const int tid = threadIdx.x;
    const int g = tid / T;
    const int l = tid % T;
    const int D = a.D;
    const int64_t begin = (int64_t)blockIdx.x * a.rows_per_block;
    const int64_t end = min(a.N, begin + a.rows_per_block);

    int coff[CPT];
    bool cval[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        coff[k] = (k * T + l) * VEC;
        cval[k] = coff[k] < D;
    }

    HV gam[CPT], bet[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        gam[k] = cval[k] ? hload<VEC>(a.gamma + coff[k]) : hzero<VEC>();
        if constexpr (KIND == LN) bet[k] = cval[k] ? hload<VEC>(a.beta + coff[k]) : hzero<VEC>();
    }

    struct Tile {
        HV x[U][CPT];
        HV r[U][CPT];
    };
    auto load_tile = [&](Tile& t, int64_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + u * RPB + g;
            const int64_t ro = row * (int64_t)D;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                const bool ok = row < end && cval[k];
                t.x[u][k] = ok ? sload<VEC, NT>(a.X + ro + coff[k]) : hzero<VEC>();
                if constexpr (KIND == ADD) t.r[u][k] = ok ? sload<VEC, NT>(a.R + ro + coff[k]) : hzero<VEC>();
            }
        }
    };

    const float fD = (float)D;
    int phase = 0;
    Tile cur;
    if constexpr (PF) load_tile(cur, begin);
    for (int64_t base = begin; base < end; base += TILE) {
        Tile nxt;
        if constexpr (PF) load_tile(nxt, base + TILE);
        else load_tile(cur, base);

        int64_t row[U];
        bool rv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            row[u] = base + u * RPB + g;
            rv[u] = row[u] < end;
        }

        // First reduction: sum of squares (RMS, ADD) or plain sum (LN).
        float s1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float v = hget<VEC>(cur.x[u][k], e);
                    if constexpr (KIND == ADD) v += hget<VEC>(cur.r[u][k], e);
                    if constexpr (KIND == LN) acc += v;
                    else acc += v * v;
                }
            s1[u] = acc;
        }
        row_sum<T, RPB, U>(s1, red, phase, g, l);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                launder(cur.x[u][k]);
                if constexpr (KIND == ADD) launder(cur.r[u][k]);
            }

        float mu[U], rs[U];
        if constexpr (KIND == LN) {
            // Second reduction: centred sum of squares from the registers.
            float s2[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                mu[u] = s1[u] / fD;
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < CPT; ++k)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float c = hget<VEC>(cur.x[u][k], e) - mu[u];
                        acc += cval[k] ? c * c : 0.0f;
                    }
                s2[u] = acc;
            }
            row_sum<T, RPB, U>(s2, red, phase, g, l);
#pragma unroll
            for (int u = 0; u < U; ++u) rs[u] = 1.0f / sqrtf(s2[u] / fD + a.eps);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                mu[u] = 0.0f;
                rs[u] = 1.0f / sqrtf(s1[u] / fD + a.eps);
            }
        }

#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (l == 0 && rv[u]) {
                a.rstd[row[u]] = rs[u];
                if constexpr (KIND == LN) a.mean[row[u]] = mu[u];
            }
            const int64_t ro = row[u] * (int64_t)D;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                if (!(rv[u] && cval[k])) continue;
                HV y;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float v = hget<VEC>(cur.x[u][k], e);
                    if constexpr (KIND == ADD) v += hget<VEC>(cur.r[u][k], e);
                    float o;
                    if constexpr (KIND == LN)
                        o = (v - mu[u]) * rs[u] * hget<VEC>(gam[k], e) + hget<VEC>(bet[k], e);
                    else
                        o = v * rs[u] * hget<VEC>(gam[k], e);
                    hset<VEC>(y, e, o);
                }
                hstore<VEC, NT>(a.Y + ro + coff[k], y);
                if constexpr (KIND == ADD) {
                    // binary16 addition rounds the exact sum once (to nearest even)
                    const HV h = cur.x[u][k] + cur.r[u][k];
                    hstore<VEC, NT>(a.H + ro + coff[k], h);
                }
            }
        }
        if constexpr (PF) cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// Backward stage 1: dX and per-workgroup parameter-gradient partials.
// ---------------------------------------------------------------------------

template <int KIND, int T, int VEC, int CPT, int U, int BLOCK, int PF, int NT>
__global__ void __launch_bounds__(BLOCK) bwd_kernel(const BwdArgs a)
{
    typedef typename HVec<VEC>::type HV;
    constexpr int RPB = BLOCK / T;
    constexpr int TILE = RPB * U;
    constexpr int NR = (KIND == LN) ? 2 : 1;  // sums per row: c1 (and c2)
    static_assert(BLOCK % T == 0, "block holds whole row groups");
    __shared__ float red[RedBuf<T, RPB, U * NR>::size];
    extern __shared__ float fold[];           // [NR][D] when RPB > 1

    const int tid = threadIdx.x;
    const int g = tid / T;
    const int l = tid % T;
    const int D = a.D;
    // Workgroup b owns tiles b, b + P, b + 2P, ... (P = gridDim.x): a fixed
    // set of rows, so its dgamma partial is reproducible, while the P
    // workgroups running together touch one contiguous band of rows.
    const int64_t end = a.N;
    const int64_t ntiles = (a.N + TILE - 1) / TILE;
    const int64_t tstride = (int64_t)gridDim.x * TILE;

    int coff[CPT];
    bool cval[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        coff[k] = (k * T + l) * VEC;
        cval[k] = coff[k] < D;
    }
    HV gam[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) gam[k] = cval[k] ? hload<VEC>(a.gamma + coff[k]) : hzero<VEC>();

    float accg[CPT][VEC], accb[CPT][VEC];
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            accg[k][e] = 0.0f;
            accb[k][e] = 0.0f;
        }

    struct Tile {
        HV x[U][CPT], r[U][CPT], dy[U][CPT];
        float rs[U], mu[U];
    };
    auto load_tile = [&](Tile& t, int64_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + u * RPB + g;
            const bool rok = row < end;
            t.rs[u] = rok ? a.rstd[row] : 0.0f;
            t.mu[u] = (KIND == LN && rok) ? a.mean[row] : 0.0f;
            const int64_t ro = row * (int64_t)D;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                const bool ok = rok && cval[k];
                t.x[u][k] = ok ? sload<VEC, NT>(a.X + ro + coff[k]) : hzero<VEC>();
                if constexpr (KIND == ADD) t.r[u][k] = ok ? sload<VEC, NT>(a.R + ro + coff[k]) : hzero<VEC>();
                t.dy[u][k] = ok ? sload<VEC, NT>(a.dY + ro + coff[k]) : hzero<VEC>();
            }
        }
    };

    const float fD = (float)D;
    int phase = 0;
    Tile cur;
    const int64_t first = (int64_t)blockIdx.x * TILE;
    const int64_t stop = ntiles * TILE;  // uniform loop bound for the workgroup
    if constexpr (PF) load_tile(cur, first);
    for (int64_t base = first; base < stop; base += tstride) {
        Tile nxt;
        if constexpr (PF) load_tile(nxt, base + tstride);
        else load_tile(cur, base);

        // c1 = sum(g * xhat), c2 = sum(g), g = dY * gamma
        float c[U * NR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float a1 = 0.0f, a2 = 0.0f;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float v = hget<VEC>(cur.x[u][k], e);
                    if constexpr (KIND == ADD) v += hget<VEC>(cur.r[u][k], e);
                    const float xh = (v - cur.mu[u]) * cur.rs[u];
                    const float gg = hget<VEC>(cur.dy[u][k], e) * hget<VEC>(gam[k], e);
                    a1 += gg * xh;
                    if constexpr (KIND == LN) a2 += gg;
                }
            c[u * NR] = a1;
            if constexpr (KIND == LN) c[u * NR + 1] = a2;
        }
        row_sum<T, RPB, U * NR>(c, red, phase, g, l);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                launder(cur.x[u][k]);
                launder(cur.dy[u][k]);
                if constexpr (KIND == ADD) launder(cur.r[u][k]);
            }

#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + u * RPB + g;
            const bool rok = row < end;
            const float c1 = c[u * NR] / fD;
            const float c2 = (KIND == LN) ? c[u * NR + 1] / fD : 0.0f;
            const float rs = cur.rs[u];
            const float mu = cur.mu[u];
            const int64_t ro = row * (int64_t)D;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                const bool ok = rok && cval[k];
                HV dh = hzero<VEC>();
                if constexpr (KIND == ADD) {
                    if (ok && a.dH != nullptr) dh = sload<VEC, NT>(a.dH + ro + coff[k]);
                }
                HV o;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float v = hget<VEC>(cur.x[u][k], e);
                    if constexpr (KIND == ADD) v += hget<VEC>(cur.r[u][k], e);
                    const float xh = (v - mu) * rs;
                    const float dyv = hget<VEC>(cur.dy[u][k], e);
                    const float gg = dyv * hget<VEC>(gam[k], e);
                    float d;
                    if constexpr (KIND == LN) d = rs * (gg - c2 - xh * c1);
                    else d = rs * (gg - xh * c1);
                    if constexpr (KIND == ADD) d += hget<VEC>(dh, e);
                    hset<VEC>(o, e, d);
                    accg[k][e] += dyv * xh;
                    if constexpr (KIND == LN) accb[k][e] += dyv;
                }
                if (ok) hstore<VEC, NT>(a.dX + ro + coff[k], o);
            }
        }
        if constexpr (PF) cur = nxt;
    }

    // Fold the row groups of this workgroup in group order, then write the
    // workgroup's partial row.
    float* pg = a.part_g + (int64_t)blockIdx.x * a.Dp;
    float* pb = (KIND == LN) ? a.part_b + (int64_t)blockIdx.x * a.Dp : nullptr;
    if constexpr (RPB == 1) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            if (!cval[k]) continue;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                pg[coff[k] + e] = accg[k][e];
                if constexpr (KIND == LN) pb[coff[k] + e] = accb[k][e];
            }
        }
    } else {
        for (int gg = 0; gg < RPB; ++gg) {
            if (g == gg) {
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    if (!cval[k]) continue;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const int j = coff[k] + e;
                        fold[j] = (gg == 0) ? accg[k][e] : fold[j] + accg[k][e];
                        if constexpr (KIND == LN)
                            fold[D + j] = (gg == 0) ? accb[k][e] : fold[D + j] + accb[k][e];
                    }
                }
            }
            __syncthreads();
        }
        for (int j = tid; j < D; j += BLOCK) {
            pg[j] = fold[j];
            if constexpr (KIND == LN) pb[j] = fold[D + j];
        }
    }
}

// ---------------------------------------------------------------------------
// Backward stage 2: out[j] = sum over the P partial rows of partial[p][j].
// A block covers 4*CQ columns (one float4 per thread); its SEG = 1024/CQ
// thread rows each sum one contiguous segment of the partial rows in
// ascending order, then the SEG segment sums are combined by a fixed
// pairwise tree (segment s with s + stride, stride halving). The order
// depends only on (P, D), so the result is bitwise reproducible.
// ---------------------------------------------------------------------------

template <int CQ>
__global__ void __launch_bounds__(1024) reduce_kernel(const ReduceArgs a)
{
    constexpr int SEG = 1024 / CQ;
    static_assert((SEG & (SEG - 1)) == 0, "segment count is a power of two");
    __shared__ f4 seg_sum[SEG][CQ];
    const float* part = (blockIdx.y == 0) ? a.part_g : a.part_b;
    float* out = (blockIdx.y == 0) ? a.dgamma : a.dbeta;
    const int q = threadIdx.x % CQ;
    const int s = threadIdx.x / CQ;
    const int c0 = (blockIdx.x * CQ + q) * 4;
    const int64_t per = (a.P + SEG - 1) / SEG;
    const int64_t p0 = min(a.P, (int64_t)s * per);
    const int64_t p1 = min(a.P, p0 + per);
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c0 < a.Dp) {
        const float* src = part + c0;
#pragma unroll 8
        for (int64_t p = p0; p < p1; ++p) acc += *reinterpret_cast<const f4*>(src + p * a.Dp);
    }
    seg_sum[s][q] = acc;
    __syncthreads();
#pragma unroll
    for (int st = SEG / 2; st > 0; st /= 2) {
        if (s < st) seg_sum[s][q] = seg_sum[s][q] + seg_sum[s + st][q];
        __syncthreads();
    }
    if (s == 0 && c0 < a.D) {
        const f4 t = seg_sum[0][q];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c0 + e < a.D) out[c0 + e] = t[e];
    }
}

}  // namespace kern
}  // namespace mn
