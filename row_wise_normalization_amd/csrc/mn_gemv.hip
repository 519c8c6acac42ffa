// mn_gemv.hip -- fused RMSNorm / LayerNorm + GEMV for small inference
// batches on gfx950 ([tensorcore] "Fused Norm + GEMV": Y = Norm(X) @ W with
// the normalised rows applied in registers, never written to memory).
//
// The product is bound by reading W once (K*N elements; M <= 8 rows of X are
// tiny), so it runs on the vector ALUs: per W element M fused multiply-adds,
// far below the ALU rate at HBM speed, and an MFMA tile would need W in its
// operand layout (a transposing LDS pass) for no gain at M <= 8.
//
// The normalisation is factored out of the product. With xc = x - c (c = 0
// for RMSNorm; for LayerNorm c is the row's first element, a shift that
// keeps the sums free of the cancellation an uncentred row would bring):
//   RMSNorm:   Y[m, n] = rstd_m * sum_k xc[m, k] g[k] W[k, n]
//   LayerNorm: Y[m, n] = rstd_m * (sum_k xc g W - (mean_m - c_m) sum_k g W)
//                        + sum_k b W
// so the product needs no row statistics: the rows xc*g (and, for LayerNorm,
// g and b themselves) are streamed against W as a small batch, and the
// statistics are applied once per output afterwards.
//
// Launch: blocks 0..M-1 each compute the statistics of one X row (the
// two-pass centred mean and mean square of the row-norm forward) into the
// workspace; every other block owns one tile of W (TC = 64*VEC/RPW columns
// by KB rows: each wave load covers RPW rows of TC columns, 16-byte loads,
// U loads in flight per wave). A tile block stages its KB rows of the product
// rows in LDS, streams its W rows into per-lane fp32 accumulators, adds the
// lanes of a column across the wave (butterfly) and the four waves in order,
// and writes one partial row per product row: part[ks][r][n].
//
// No second launch adds the partials. Every block that wrote something a
// tile's outputs need (its S slices, and the M statistics blocks for every
// tile) increments the tile's arrival counter once its stores have
// completed; the block whose increment completes the count adds the S
// partials of each output in ascending ks order, applies the statistics,
// rounds once to the storage type and sets the counter back to zero. The
// order of the sums does not depend on which block performs them, so the
// result is bitwise reproducible, and no block waits for another.
//
// The hand-off needs no cache maintenance. Every value handed from one
// workgroup to another (partials, statistics) is stored and loaded with
// relaxed device-scope atomics, which this architecture performs at the
// device's coherence point: the stores write through the XCD's L2, the loads
// do not return a line of it. The ordering comes from completion:
//   1. each wave of a producer waits for its stores to complete (vmcnt 0:
//      acknowledged at the coherence point) before the workgroup barrier,
//      so all of them are complete before thread 0 issues the increment;
//   2. increments of one counter are performed one after another at the
//      coherence point, so the one that completes the count comes after
//      every producer's increment, and so after every producer's stores;
//   3. the completing thread waits for its increment's return value
//      before the barrier that releases the block's other threads, and
//      only then are the loads issued.
// A load issued after a store to the same address was acknowledged at the
// coherence point reads that store (or a later one). The memory model's own
// form, an agent-scope release on the increment and an acquire for the
// completing workgroup, also writes back the XCD's whole L2 (buffer_wbl2)
// at every release: measured 2.2 times slower at M = 4 even with one release
// per workgroup and the acquire only in completing workgroups (4-5 times
// with fences per wave). The 400-call test of alternating inputs through one
// workspace checks the hand-off.
#include "mn_kernels.hpp"

namespace mn {

// Tile shapes of the 16-byte path, from timing sweeps at 4096 x 12288 and
// 4096 x 14336 (K x N): four rows of 128 columns per wave load, and tiles
// halved along K until there is about one per CU (with the K slices added
// inside the launch, fewer and longer slices beat two tiles per CU: 16 %
// faster at 4 x 4096 @ 4096 x 4096, equal at N = 12288); for one or two X
// rows and wide W, one row of 512 columns per wave load in fewer, longer
// tiles (8 % faster at M = 1, N = 14336; slower at M = 4, whose product rows
// need more registers per column, and at N = 4096, which leaves too few
// tiles).
constexpr int kGemvRpwVec = 4;
constexpr int64_t kGemvTileTarget = 256;
constexpr int64_t kGemvWideTileTarget = 192;

namespace kern {

constexpr int kGemvBlock = 256;   // four waves
constexpr int kGemvWaves = kGemvBlock / 64;

// Device-scope store and load of a value handed from one workgroup to
// another (see the hand-off above).
__device__ __forceinline__ void put_dev(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_dev(const float* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This wave's stores have completed (s_waitcnt vmcnt(0), the other counters
// left unconstrained; stores count in vmcnt on this architecture).
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Statistics of X row m = blockIdx.x: {mean (LayerNorm) or 0, rstd}.
template <int ST, bool LNF>
__device__ void gemv_row_stats(const GemvArgs& a)
{
    typedef typename Elem<ST>::type E;
    __shared__ float wsum[kGemvWaves];
    const int m = blockIdx.x;
    const int K = a.K;
    const E* x = static_cast<const E*>(a.X) + (int64_t)m * K;
    float mu = 0.0f;
    if (LNF) {
        float s = 0.0f;
#pragma unroll 8
        for (int k = threadIdx.x; k < K; k += kGemvBlock) s += (float)x[k];
        s = block_sum<kGemvBlock>(s, wsum);
        if (threadIdx.x == 0) wsum[0] = s / (float)K;
        __syncthreads();
        mu = wsum[0];
    }
    float q = 0.0f;
#pragma unroll 8
    for (int k = threadIdx.x; k < K; k += kGemvBlock) {
        const float c = (float)x[k] - mu;
        q = __builtin_fmaf(c, c, q);
    }
    q = block_sum<kGemvBlock>(q, wsum);
    if (threadIdx.x == 0) {
        put_dev(&a.stats[2 * m], mu);
        put_dev(&a.stats[2 * m + 1], 1.0f / sqrtf(q / (float)K + a.eps));
    }
}

// Parameter element k of any parameter type without a branch: two 16-bit
// loads (the halves of a binary32 value, or the same 16-bit element twice)
// and a select of the conversion.
__device__ __forceinline__ float param_any(const void* base, int pdt, int k)
{
    const uint16_t* p = static_cast<const uint16_t*>(base);
    const bool f32 = pdt == ST_F32;
    const uint32_t lo = p[f32 ? 2 * (int64_t)k : (int64_t)k];
    const uint32_t hi = p[f32 ? 2 * (int64_t)k + 1 : (int64_t)k];
    const float vf = __uint_as_float(lo | (hi << 16));
    const float vb = __uint_as_float(lo << 16);
    const float vh = (float)__builtin_bit_cast(_Float16, (uint16_t)lo);
    return f32 ? vf : (pdt == ST_BF16 ? vb : vh);
}

// Y[m][n] of column tile cb from the S partials (ks ascending) and the row
// statistics; called by the block that completed the tile's count.
template <int ST, bool LNF, int TC>
__device__ void gemv_finish(const GemvArgs& a, int cb)
{
    typedef typename Elem<ST>::type E;
    const int M = a.M, N = a.N;
    const int RE = M + (LNF ? 2 : 0);
    const int64_t step = (int64_t)RE * N;
    for (int i = threadIdx.x; i < M * TC; i += kGemvBlock) {
        const int m = i / TC;
        const int n = cb * TC + i % TC;
        if (n >= N) continue;
        // statistics first, so their loads overlap the partials'
        const float rs = get_dev(&a.stats[2 * m + 1]);
        const float d = LNF ? get_dev(&a.stats[2 * m]) -
                                  (float)static_cast<const E*>(a.X)[(int64_t)m * a.K]
                            : 0.0f;
        const float* pa = a.part + (int64_t)m * N + n;
        const float* pg = a.part + (int64_t)M * N + n;
        const float* pb = a.part + (int64_t)(M + 1) * N + n;
        float sa = 0.0f, sg = 0.0f, sb = 0.0f;
        int k = 0;
        for (; k + 8 <= a.S; k += 8) {
            float va[8], vg[8], vb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                va[j] = get_dev(pa + (k + j) * step);
                if (LNF) {
                    vg[j] = get_dev(pg + (k + j) * step);
                    vb[j] = get_dev(pb + (k + j) * step);
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sa += va[j];
                if (LNF) {
                    sg += vg[j];
                    sb += vb[j];
                }
            }
        }
        for (; k < a.S; ++k) {
            sa += get_dev(pa + k * step);
            if (LNF) {
                sg += get_dev(pg + k * step);
                sb += get_dev(pb + k * step);
            }
        }
        float y;
        if (LNF) {
            y = __builtin_fmaf(rs, __builtin_fmaf(-d, sg, sa), sb);
        } else {
            y = rs * sa;
        }
        static_cast<E*>(a.Y)[(int64_t)m * N + n] = (E)y;
    }
}

// Counter of tile cb back to zero for the next call, by the block that
// finished the tile.
__device__ __forceinline__ void gemv_reset(const GemvArgs& a, int cb)
{
    __hip_atomic_store(&a.cnt[cb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int ST, int VEC, int MM, bool LNF, int RPW, int U>
__global__ void __launch_bounds__(kGemvBlock) gemv_kernel(const GemvArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    typedef typename Elem<ST>::type E;
    constexpr int NW = kGemvWaves;
    constexpr int LPR = 64 / RPW;             // lanes per W row
    constexpr int TC = LPR * VEC;             // tile columns
    constexpr int RS = NW * RPW;              // W rows per workgroup step
    constexpr int R = MM + (LNF ? 2 : 0);     // product rows: xc*g, then g, b
    constexpr int RP = (R + 3) / 4 * 4;
    // staging buffer [KB][RP], reused for the wave sums [NW][R][TC]
    constexpr int LF = kGemvMaxKB * RP > NW * R * TC ? kGemvMaxKB * RP : NW * R * TC;
    __shared__ float4 lds4[LF / 4];
    float* const lds = reinterpret_cast<float*>(lds4);

    __shared__ int s_count;
    const int M = a.M;
    const int tid = threadIdx.x;
    const unsigned arrivals = (unsigned)(a.S + M);
    if ((int)blockIdx.x < M) {
        gemv_row_stats<ST, LNF>(a);
        // count the statistics in on every tile, and finish the tiles whose
        // count this block completes
        stores_done();
        __syncthreads();
        int* const done = reinterpret_cast<int*>(lds);
        for (int base = 0; base < a.NB; base += kGemvBlock) {
            if (tid == 0) s_count = 0;
            __syncthreads();
            const int cb = base + tid;
            if (cb < a.NB && atomicAdd(&a.cnt[cb], 1u) == arrivals - 1)
                done[atomicAdd(&s_count, 1)] = cb;
            __syncthreads();
            const int nd = s_count;
            for (int j = 0; j < nd; ++j) {
                gemv_finish<ST, LNF, TC>(a, done[j]);
                if (tid == 0) gemv_reset(a, done[j]);
            }
            __syncthreads();
        }
        return;
    }
    const int t = (int)blockIdx.x - M;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = lane / LPR;
    const int cl = lane % LPR;
    const int N = a.N, K = a.K;
    const E* X = static_cast<const E*>(a.X);
    const int cb = t % a.NB;
    const int ks = t / a.NB;
    const int k0 = ks * a.KB;
    const int kn = min(a.KB, K - k0);
    const int n0 = cb * TC + cl * VEC;
    const int r0 = wave * RPW + rg;                       // this lane's first row
    const int nb = (kn - wave * RPW + RS - 1) / RS;       // row steps of the wave
    // Every load below is unconditional: rows past the tile and columns past
    // N are clamped to the last valid ones (their values are never used), so
    // no load sits behind a branch and the loads of a batch issue together.
    const int64_t wcol = min(n0, N - VEC);
    auto wrow = [&](int i) -> int64_t {
        return (int64_t)(k0 + min(r0 + i * RS, kn - 1)) * N + wcol;
    };

    // First batch of W, then the tile's X and parameter values: one round
    // trip covers both.
    HV wa[U], wb[U];
#pragma unroll
    for (int j = 0; j < U; ++j) wa[j] = sload<ST, VEC, 2>(a.W, wrow(j));
    {
        constexpr int IT = kGemvMaxKB / kGemvBlock;
        E xr[IT][MM], cx[MM];
        float g[IT], b[IT];
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            const int64_t row = (int64_t)min(m, M - 1) * K;
            cx[m] = X[row];
#pragma unroll
            for (int it = 0; it < IT; ++it)
                xr[it][m] = X[row + k0 + min(tid + it * kGemvBlock, kn - 1)];
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int k = k0 + min(tid + it * kGemvBlock, kn - 1);
            g[it] = param_any(a.gamma, a.pdt, k);
            b[it] = LNF ? param_any(a.beta, a.pdt, k) : 0.0f;
        }
        // product rows of the tile: lds[k * RP + r]. Rows past kn are never
        // read; rows m >= M repeat row M - 1 and their sums are never stored.
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int k = tid + it * kGemvBlock;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const float c = LNF ? (float)cx[m] : 0.0f;
                lds[k * RP + m] = ((float)xr[it][m] - c) * g[it];
            }
            if (LNF) {
                lds[k * RP + MM] = g[it];
                lds[k * RP + MM + 1] = b[it];
            }
        }
    }
    __syncthreads();

    float acc[R][VEC];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[r][e] = 0.0f;
    // U rows of W per step of the lane
    auto consume = [&](const HV (&w)[U], int base) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int r = r0 + (base + j) * RS;
            if (r < kn) {
                float xv[RP];
#pragma unroll
                for (int q = 0; q < RP / 4; ++q) {
                    const float4 v = lds4[r * (RP / 4) + q];
                    xv[4 * q] = v.x;
                    xv[4 * q + 1] = v.y;
                    xv[4 * q + 2] = v.z;
                    xv[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float wv = cget<ST, VEC>(w[j], e);
#pragma unroll
                    for (int p = 0; p < R; ++p) acc[p][e] = __builtin_fmaf(xv[p], wv, acc[p][e]);
                }
            }
        }
    };
    // two register sets in turn: the next batch is in flight while one is used
    for (int base = 0; base < nb; base += 2 * U) {
#pragma unroll
        for (int j = 0; j < U; ++j) wb[j] = sload<ST, VEC, 2>(a.W, wrow(base + U + j));
        consume(wa, base);
#pragma unroll
        for (int j = 0; j < U; ++j) wa[j] = sload<ST, VEC, 2>(a.W, wrow(base + 2 * U + j));
        consume(wb, base + U);
    }

    // lanes of one column across the wave (butterfly), then the waves in order
#pragma unroll
    for (int p = 0; p < R; ++p)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
#pragma unroll
            for (int o = LPR; o < 64; o <<= 1) acc[p][e] += __shfl_xor(acc[p][e], o);
    __syncthreads();  // the staging buffer is reused below
    if (rg == 0) {
#pragma unroll
        for (int p = 0; p < R; ++p)
#pragma unroll
            for (int e = 0; e < VEC; ++e) lds[(wave * R + p) * TC + cl * VEC + e] = acc[p][e];
    }
    __syncthreads();
    const int RE = M + (LNF ? 2 : 0);   // partial rows written per slice
    for (int i = tid; i < RE * TC; i += kGemvBlock) {
        const int pr = i / TC;
        const int c = i % TC;
        const int n = cb * TC + c;
        if (n < N) {
            const int p = pr < M ? pr : MM + (pr - M);
            float s = lds[p * TC + c];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) s += lds[(ww * R + p) * TC + c];
            put_dev(&a.part[((int64_t)ks * RE + pr) * N + n], s);
        }
    }
    // count the slice in once its stores have completed; the block that
    // completes the tile's count adds the tile's partials
    stores_done();
    __syncthreads();
    if (tid == 0) s_count = atomicAdd(&a.cnt[cb], 1u) == arrivals - 1;
    __syncthreads();
    if (s_count) {
        gemv_finish<ST, LNF, TC>(a, cb);
        if (tid == 0) gemv_reset(a, cb);
    }
}

}  // namespace kern

namespace {

template <typename Kernel>
hipError_t launch_k(Kernel k, dim3 grid, dim3 block, hipStream_t s, const GemvArgs& a)
{
    void* args[] = {const_cast<GemvArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, 0, s);
}

template <int ST, int VEC, bool LNF, int RPW>
hipError_t launch_gemv_mm(int mm, dim3 grid, hipStream_t s, const GemvArgs& a)
{
    const dim3 block(kern::kGemvBlock);
    // the wide 16-byte tiles serve one or two X rows only; W loads in flight
    // per register set: 8 for one or two X rows, 4 for RMSNorm at three or
    // four, 2 for LayerNorm there (two more product rows) and for five to
    // eight (fewer loads in flight, more waves: 5-9 % faster at M = 4 with
    // 4 than 8, and 4-11 % faster at M = 8 and for LayerNorm at M = 4 with 2
    // than 4, at N = 12288)
    constexpr bool ALL = !(VEC == 8 && RPW == 1);
    switch (mm) {
    case 1: return launch_k(kern::gemv_kernel<ST, VEC, 1, LNF, RPW, 8>, grid, block, s, a);
    case 2: return launch_k(kern::gemv_kernel<ST, VEC, 2, LNF, RPW, 8>, grid, block, s, a);
    case 4:
        if constexpr (ALL) return launch_k(kern::gemv_kernel<ST, VEC, 4, LNF, RPW, LNF ? 2 : 4>, grid, block, s, a);
        break;
    case 8:
        if constexpr (ALL) return launch_k(kern::gemv_kernel<ST, VEC, 8, LNF, RPW, 2>, grid, block, s, a);
        break;
    }
    return hipErrorInvalidValue;
}

template <int ST>
hipError_t launch_gemv_st(bool ln, bool vec, int rpw, int mm, dim3 grid, hipStream_t s,
                          const GemvArgs& a)
{
    if (vec && rpw == 1) return ln ? launch_gemv_mm<ST, 8, true, 1>(mm, grid, s, a)
                                   : launch_gemv_mm<ST, 8, false, 1>(mm, grid, s, a);
    if (vec) return ln ? launch_gemv_mm<ST, 8, true, kGemvRpwVec>(mm, grid, s, a)
                       : launch_gemv_mm<ST, 8, false, kGemvRpwVec>(mm, grid, s, a);
    return ln ? launch_gemv_mm<ST, 1, true, 1>(mm, grid, s, a)
              : launch_gemv_mm<ST, 1, false, 1>(mm, grid, s, a);
}

}  // namespace

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, bool vec_ok)
{
    GemvPlan p;
    p.vec = vec_ok;
    p.MM = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    const bool wide = vec_ok && p.MM <= 2 &&
                      ((N + 511) / 512) * ((K + kGemvMaxKB - 1) / kGemvMaxKB) >= kGemvWideTileTarget;
    p.rpw = vec_ok && !wide ? kGemvRpwVec : 1;
    const int64_t cols = (vec_ok ? 64 * 8 : 64) / p.rpw;
    const int64_t target = wide ? kGemvWideTileTarget : kGemvTileTarget;
    p.NB = (int32_t)((N + cols - 1) / cols);
    // One tile per workgroup. Slices of K are halved from the LDS maximum
    // until there are enough tiles to keep every CU busy (each slice adds
    // rows of fp32 partials to write and read back), down to 64 rows.
    int64_t KB = kGemvMaxKB;
    while (KB > 64 && (int64_t)p.NB * ((K + KB - 1) / KB) < target) KB /= 2;
    p.KB = (int32_t)KB;
    p.S = (int32_t)((K + KB - 1) / KB);
    p.grid = M + (int64_t)p.NB * p.S;
    return p;
}

hipError_t launch_gemv(int st, bool ln, const GemvPlan& p, const GemvArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)p.grid);
    hipError_t e = hipErrorInvalidValue;
    switch (st) {
    case ST_F16: e = launch_gemv_st<ST_F16>(ln, p.vec, p.rpw, p.MM, grid, s, a); break;
    case ST_BF16: e = launch_gemv_st<ST_BF16>(ln, p.vec, p.rpw, p.MM, grid, s, a); break;
    }
    return e;
}

}  // namespace mn
