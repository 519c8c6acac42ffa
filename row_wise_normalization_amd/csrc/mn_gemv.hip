// mn_gemv.hip -- fused RMSNorm / LayerNorm + GEMV for small inference
// batches on gfx950 ([tensorcore] "Fused Norm + GEMV": Y = Norm(X) @ W with
// the normalised rows applied in registers, never written to memory).
//
// The product is bound by reading W once (K*N elements; M <= 8 rows of X are
// tiny). Per W element it takes M (+2 for LayerNorm) multiply-adds: for
// RMSNorm in binary16 on the matrix cores (16x16x16 products, W's operand
// layout formed by byte permutes in registers, no LDS pass; see the
// matrix-core tiles below), otherwise on the vector ALUs (LayerNorm,
// bfloat16, unaligned operands, and the wide tiles of one or two rows
// against a wide W).
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

// Blocks 0..M-1: the statistics of row blockIdx.x, then the count on every
// tile, finishing the tiles whose count this block completes. `done` is
// kGemvBlock ints of shared scratch.
template <int ST, bool LNF, int TC>
__device__ void gemv_stats_block(const GemvArgs& a, int* done, int& s_count)
{
    const int tid = threadIdx.x;
    const unsigned arrivals = (unsigned)(a.S + a.M);
    gemv_row_stats<ST, LNF>(a);
    stores_done();
    __syncthreads();
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
}

// End of a tile block: the wave sums are in lds[(wave * R + p) * TC + c]
// (p < R: the product rows, then g and b for LayerNorm); the waves are added
// in order into the slice's partial rows, the slice is counted in once its
// stores have completed, and the block that completes the tile's count adds
// the tile's partials.
template <int ST, int MM, bool LNF, int TC>
__device__ void gemv_tile_end(const GemvArgs& a, const float* lds, int cb, int ks, int& s_count)
{
    constexpr int R = MM + (LNF ? 2 : 0);
    const int M = a.M, N = a.N, tid = threadIdx.x;
    const unsigned arrivals = (unsigned)(a.S + M);
    const int RE = M + (LNF ? 2 : 0);   // partial rows written per slice
    for (int i = tid; i < RE * TC; i += kGemvBlock) {
        const int pr = i / TC;
        const int c = i % TC;
        const int n = cb * TC + c;
        if (n < N) {
            const int p = pr < M ? pr : MM + (pr - M);
            float s = lds[p * TC + c];
#pragma unroll
            for (int ww = 1; ww < kGemvWaves; ++ww) s += lds[(ww * R + p) * TC + c];
            put_dev(&a.part[((int64_t)ks * RE + pr) * N + n], s);
        }
    }
    stores_done();
    __syncthreads();
    if (tid == 0) s_count = atomicAdd(&a.cnt[cb], 1u) == arrivals - 1;
    __syncthreads();
    if (s_count) {
        gemv_finish<ST, LNF, TC>(a, cb);
        if (tid == 0) gemv_reset(a, cb);
    }
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
    if ((int)blockIdx.x < M) {
        gemv_stats_block<ST, LNF, TC>(a, reinterpret_cast<int*>(lds), s_count);
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
    gemv_tile_end<ST, MM, LNF, TC>(a, lds, cb, ks, s_count);
}

// ---------------------------------------------------------------------------
// Matrix-core tiles (binary16 X and W, the 16-byte path, at most eight
// product rows). The product of a tile is an MFMA product
//   D[m][n] += sum_k A[m][k] B[k][n]   (v_mfma_f32_16x16x16_f16, fp32 sums)
// with B = 16 rows x 16 columns of W and A = the product rows of X over the
// same 16 rows. W is read exactly as the vector-ALU kernel reads it (16-byte
// loads of 8 columns) and its elements are exact in binary16; the product
// rows are fp32 values, so each is split into two binary16 rows, hi = f16(v)
// and lo = f16(v - hi), after scaling the row of the tile by a power of two
// that puts its largest magnitude in [2^14, 2^15) (no overflow; the split
// keeps about 22 bits, the products are exact and the sums fp32). A holds
// hi and lo of product row r as its rows 2r and 2r + 1, so 2 R <= 16.
//
// Lane layout of the 16x16x16 product (lane l): A[l % 16][4 (l / 16) + i],
// B[4 (l / 16) + i][l % 16] and D[4 (l / 16) + i][l % 16], i = 0..3. A lane
// loads rows 4 (l / 16) .. + 3 of a 16-row step at columns 8 (l % 16) .. + 7
// and forms from them the B operands of eight products, one per column j of
// its eight (two byte permutes each): product j covers the tile columns
// 8 c + j, c = 0..15. Its D rows 4 (l / 16) + i are then hi and lo of the
// product rows 2 (l / 16) and 2 (l / 16) + 1, added and scaled back.
// ---------------------------------------------------------------------------
constexpr int kMfmaTC = 128;                 // tile columns: 16 lanes x 8
constexpr int kMfmaKP = kGemvMaxKB + 8;      // LDS row pitch of A, in halves
constexpr int kBufNt = 2;                    // buffer cache policy: nt
constexpr int kBufWord3 = 0x00020000;        // raw buffer, 32-bit data format
constexpr uint32_t kBufOut = 0x80000000u;    // offset past every tile: reads 0

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float mf4 __attribute__((ext_vector_type(4)));
typedef uint32_t wq __attribute__((ext_vector_type(4)));

template <int MM, bool LNF, int U>
__global__ void __launch_bounds__(kGemvBlock) gemv_mfma_kernel(const GemvArgs a)
{
    constexpr int R = MM + (LNF ? 2 : 0);
    static_assert(2 * R <= 16, "hi and lo rows of every product row fit the A operand");
    constexpr int NW = kGemvWaves;
    constexpr int TC = kMfmaTC;
    constexpr int KP = kMfmaKP;
    constexpr int AB = 16 * KP * 2;          // A rows in LDS, bytes
    constexpr int SB = NW * R * TC * 4;      // wave sums, bytes
    __shared__ float4 lds4[(AB > SB ? AB : SB) / 16];
    __shared__ float s_max[NW][R];
    __shared__ int s_sh[R];
    __shared__ int s_count;
    _Float16* const la = reinterpret_cast<_Float16*>(lds4);
    float* const lds = reinterpret_cast<float*>(lds4);

    const int M = a.M;
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < M) {
        gemv_stats_block<ST_F16, LNF, TC>(a, reinterpret_cast<int*>(lds), s_count);
        return;
    }
    const int t = (int)blockIdx.x - M;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = lane & 15;                // column group: tile columns 8 cg .. + 7
    const int kg = lane >> 4;                // rows 4 kg .. + 3 of each 16-row step
    const int N = a.N, K = a.K;
    const int cb = t % a.NB;
    const int ks = t / a.NB;
    const int k0 = ks * a.KB;
    const int kn = min(a.KB, K - k0);
    // the tile's W through a buffer resource: rows at or past kn read as 0;
    // columns past N (ragged last tile) repeat the last 8 and are not stored
    const _Float16* wt = static_cast<const _Float16*>(a.W) + (int64_t)k0 * N + (int64_t)cb * TC;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16*>(wt), 0, (int)((int64_t)kn * N * 2), kBufWord3);
    const int colc = min(cb * TC + 8 * cg, N - 8) - cb * TC;
    auto woff = [&](int rr) -> uint32_t {
        return rr < kn ? (uint32_t)(((int64_t)rr * N + colc) * 2) : kBufOut;
    };
    const int nb = (kn - 16 * wave + 16 * NW - 1) / (16 * NW);   // 16-row steps of the wave
    auto load_step = [&](wq (&w)[4], int s) {
        const int rb = 16 * (wave + NW * s) + 4 * kg;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            w[r] = __builtin_bit_cast(wq, __builtin_amdgcn_raw_buffer_load_b128(wr, woff(rb + r), 0, kBufNt));
    };

    // first steps of W in flight while the A rows are formed
    wq wa[U][4], wb[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) load_step(wa[u], u);

    // product rows of the tile (rows past kn are 0), their scales, and the
    // hi / lo rows of A in LDS: la[m * KP + k]
    int sh[R];
    {
        constexpr int IT = kGemvMaxKB / kGemvBlock;
        const _Float16* X = static_cast<const _Float16*>(a.X);
        float v[IT][R];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int k = tid + it * kGemvBlock;
            const int kk = k0 + min(k, kn - 1);
            const float g = param_any(a.gamma, a.pdt, kk);
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const int64_t row = (int64_t)min(m, M - 1) * K;
                const float c = LNF ? (float)X[row] : 0.0f;
                v[it][m] = ((float)X[row + kk] - c) * g;
            }
            if (LNF) {
                v[it][MM] = g;
                v[it][MM + 1] = param_any(a.beta, a.pdt, kk);
            }
            if (k >= kn)
#pragma unroll
                for (int r = 0; r < R; ++r) v[it][r] = 0.0f;
        }
        // largest magnitude of each row over the tile
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mx = 0.0f;
#pragma unroll
            for (int it = 0; it < IT; ++it) mx = fmaxf(mx, fabsf(v[it][r]));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            if (lane == 0) s_max[wave][r] = mx;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mx = s_max[0][r];
#pragma unroll
            for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_max[w][r]);
            // finite and nonzero: 2^sh puts the largest in [2^14, 2^15)
            const bool scale = mx > 0.0f && mx <= 3.40282347e38f;
            int ex = 0;
            if (scale) frexpf(mx, &ex);
            sh[r] = scale ? 15 - ex : 0;
            if (tid == r) s_sh[r] = sh[r];
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int k = tid + it * kGemvBlock;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float vs = ldexpf(v[it][r], sh[r]);
                const _Float16 hi = (_Float16)vs;
                const float hf = (float)hi;
                // a non-finite value keeps its hi part only (no inf - inf)
                const _Float16 lo = (hf - hf == 0.0f) ? (_Float16)(vs - hf) : (_Float16)0.0f;
                la[(2 * r) * KP + k] = hi;
                la[(2 * r + 1) * KP + k] = lo;
            }
#pragma unroll
            for (int m = 2 * R; m < 16; ++m) la[m * KP + k] = (_Float16)0.0f;
        }
    }
    __syncthreads();

    mf4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mf4{0.0f, 0.0f, 0.0f, 0.0f};
    auto mma_step = [&](const wq (&w)[4], int s) {
        const int kb = 16 * (wave + NW * s) + 4 * kg;
        const h4 af = *reinterpret_cast<const h4*>(&la[cg * KP + kb]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int d = j >> 1;
            uint32_t b0, b1;
            if (j & 1) {
                b0 = (w[0][d] >> 16) | (w[1][d] & 0xFFFF0000u);
                b1 = (w[2][d] >> 16) | (w[3][d] & 0xFFFF0000u);
            } else {
                b0 = (w[0][d] & 0xFFFFu) | (w[1][d] << 16);
                b1 = (w[2][d] & 0xFFFFu) | (w[3][d] << 16);
            }
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            const h4 bf = __builtin_bit_cast(h4, u2{b0, b1});
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(af, bf, acc[j], 0, 0, 0);
        }
    };
    // two register sets in turn: the next steps are in flight while one is used
    for (int s = 0; s < nb; s += 2 * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) load_step(wb[u], s + U + u);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s + u < nb) mma_step(wa[u], s + u);
#pragma unroll
        for (int u = 0; u < U; ++u) load_step(wa[u], s + 2 * U + u);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s + U + u < nb) mma_step(wb[u], s + U + u);
    }

    // hi + lo of product rows 2 kg and 2 kg + 1, scaled back, as wave sums
    __syncthreads();  // the A rows are reused below
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 2 * kg + h;
        if (r < R) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                lds[(wave * R + r) * TC + 8 * cg + j] =
                    ldexpf(acc[j][2 * h] + acc[j][2 * h + 1], -s_sh[r]);
        }
    }
    __syncthreads();
    gemv_tile_end<ST_F16, MM, LNF, TC>(a, lds, cb, ks, s_count);
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

hipError_t launch_gemv_mfma(int mm, dim3 grid, hipStream_t s, const GemvArgs& a)
{
    const dim3 block(kern::kGemvBlock);
    switch (mm) {
    case 1: return launch_k(kern::gemv_mfma_kernel<1, false, 2>, grid, block, s, a);
    case 2: return launch_k(kern::gemv_mfma_kernel<2, false, 2>, grid, block, s, a);
    case 4: return launch_k(kern::gemv_mfma_kernel<4, false, 2>, grid, block, s, a);
    case 8: return launch_k(kern::gemv_mfma_kernel<8, false, 2>, grid, block, s, a);
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

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, bool vec_ok, bool f16, bool ln)
{
    GemvPlan p;
    p.vec = vec_ok;
    p.MM = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
    const bool wide = vec_ok && p.MM <= 2 &&
                      ((N + 511) / 512) * ((K + kGemvMaxKB - 1) / kGemvMaxKB) >= kGemvWideTileTarget;
    // matrix-core tiles (128 columns): RMSNorm in binary16 with 16-byte
    // loads, not the shapes the wide vector-ALU tiles serve (faster for one or
    // two X rows). LayerNorm's six product rows at four X rows measured 1-5 %
    // slower on them (its longer tile set-up), so it keeps the vector ALUs.
    p.mfma = vec_ok && f16 && !ln && !wide && 2 * p.MM <= 16;
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
    if (p.mfma) return ln ? hipErrorInvalidValue : launch_gemv_mfma(p.MM, grid, s, a);
    hipError_t e = hipErrorInvalidValue;
    switch (st) {
    case ST_F16: e = launch_gemv_st<ST_F16>(ln, p.vec, p.rpw, p.MM, grid, s, a); break;
    case ST_BF16: e = launch_gemv_st<ST_BF16>(ln, p.vec, p.rpw, p.MM, grid, s, a); break;
    }
    return e;
}

}  // namespace mn
