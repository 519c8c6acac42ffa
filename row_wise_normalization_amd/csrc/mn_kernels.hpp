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
//     workgroup exactly one tile; the backward gives workgroup b the tiles
//     b, b+P, b+2P, ..., so the workgroups in flight always cover one
//     contiguous band of rows. With PF = 1 (backward) the loads of the next
//     tile are issued before the current tile is reduced, so HBM reads stay
//     in flight while a wave reduces and writes.
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

typedef float f4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Storage types. Activations use a template storage type ST: binary16
// (_Float16), bfloat16 (__bf16; gfx950 converts with v_cvt_pk_bf16_f32,
// round to nearest even) or binary32. A chunk is VEC consecutive elements,
// 16 bytes for VEC = 8 (16-bit types) or VEC = 4 (binary32), or one element.
// ---------------------------------------------------------------------------

template <int ST> struct Elem;
template <> struct Elem<ST_F16> { typedef _Float16 type; };
template <> struct Elem<ST_BF16> { typedef __bf16 type; };
template <> struct Elem<ST_F32> { typedef float type; };

template <int ST, int VEC> struct Chunk {
    typedef typename Elem<ST>::type E;
    typedef E type __attribute__((ext_vector_type(VEC)));
};
template <int ST> struct Chunk<ST, 1> { typedef typename Elem<ST>::type type; };

template <int ST, int VEC>
__device__ __forceinline__ typename Chunk<ST, VEC>::type czero()
{
    typename Chunk<ST, VEC>::type z;
    typename Elem<ST>::type s = (typename Elem<ST>::type)0.0f;
    z = s;  // splat for vector types
    return z;
}

// Load of a streamed input chunk (read once per launch); NT bit 1 marks it
// non-temporal so it does not displace reusable lines in the caches.
template <int ST, int VEC, int NT>
__device__ __forceinline__ typename Chunk<ST, VEC>::type sload(const void* base, int64_t off)
{
    typedef typename Chunk<ST, VEC>::type C;
    const C* p = reinterpret_cast<const C*>(static_cast<const typename Elem<ST>::type*>(base) + off);
    if constexpr ((NT & 2) != 0) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int ST, int VEC, int NT>
__device__ __forceinline__ void cstore(void* base, int64_t off, const typename Chunk<ST, VEC>::type& v)
{
    typedef typename Chunk<ST, VEC>::type C;
    C* p = reinterpret_cast<C*>(static_cast<typename Elem<ST>::type*>(base) + off);
    if constexpr ((NT & 1) != 0) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <int ST, int VEC>
__device__ __forceinline__ float cget(const typename Chunk<ST, VEC>::type& v, int e)
{
    if constexpr (VEC == 1) return (float)v;
    else return (float)v[e];
}

// Round an fp32 value into a chunk element (round to nearest even).
template <int ST, int VEC>
__device__ __forceinline__ void cset(typename Chunk<ST, VEC>::type& v, int e, float f)
{
    typedef typename Elem<ST>::type E;
    if constexpr (VEC == 1) v = (E)f;
    else v[e] = (E)f;
}

// bfloat16 rounding of the exact sum a + b of two bfloat16 values. The fp32
// sum s may itself be rounded; TwoSum recovers the exact remainder err with
// a + b = s + err. Rounding s to bfloat16 rounds a + b correctly unless s
// lies exactly halfway between two bfloat16 values (low 16 bits 0x8000) and
// err != 0: then the exact sum is off that midpoint on the side of err.
__device__ __forceinline__ __bf16 bf16_round_sum(float a, float b)
{
    const float s = a + b;
    const float bb = s - a;
    const float err = (a - (s - bb)) + (b - bb);
    const unsigned u = __builtin_bit_cast(unsigned, s);
    if ((u & 0xFFFFu) == 0x8000u && err != 0.0f && (u & 0x7F800000u) != 0x7F800000u) {
        const bool away = (err > 0.0f) == (s > 0.0f);
        const unsigned short h = (unsigned short)((u >> 16) + (away ? 1u : 0u));
        return __builtin_bit_cast(__bf16, h);
    }
    return (__bf16)s;
}

// The fused add's H chunk: the sum x + r rounded once to the storage type.
template <int ST, int VEC>
__device__ __forceinline__ typename Chunk<ST, VEC>::type round_sum(
    const typename Chunk<ST, VEC>::type& x, const typename Chunk<ST, VEC>::type& r)
{
    typedef typename Chunk<ST, VEC>::type C;
    if constexpr (ST == ST_F16) {
        return x + r;  // binary16 addition rounds the exact sum once
    } else if constexpr (ST == ST_F32) {
        return x + r;  // binary32 addition, likewise
    } else {
        C h;
        if constexpr (VEC == 1) {
            h = bf16_round_sum((float)x, (float)r);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) h[e] = bf16_round_sum((float)x[e], (float)r[e]);
        }
        return h;
    }
}

// Parameters (gamma, beta) are read once per workgroup and widened to fp32
// registers; their storage type pdt is a runtime value. Reading and widening
// are separate steps: the loads are issued (under a uniform branch on pdt)
// together with the first tile's loads, and widened after both are in
// flight, so a workgroup waits for memory once, not once per parameter.
//
// PRaw holds one chunk as loaded: VEC binary32 words, or VEC 16-bit values
// packed two per word (element e in the low half of word e/2 when e is even),
// or, for VEC == 1, one 16-bit value in the low half of word 0.
template <int VEC>
struct PRaw {
    uint32_t w[VEC];
};

typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

template <int VEC>
__device__ __forceinline__ void load_param_raw(const void* base, int pdt, int off, PRaw<VEC>& r)
{
    if (pdt == ST_F32) {
        const uint32_t* p = static_cast<const uint32_t*>(base) + off;
        if constexpr (VEC % 4 == 0) {
#pragma unroll
            for (int q = 0; q < VEC / 4; ++q) {
                const u4 v = *reinterpret_cast<const u4*>(p + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) r.w[4 * q + e] = v[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) r.w[e] = p[e];
        }
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(base) + off;
        if constexpr (VEC % 8 == 0) {
#pragma unroll
            for (int q = 0; q < VEC / 8; ++q) {
                const u4 v = *reinterpret_cast<const u4*>(p + 8 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) r.w[4 * q + e] = v[e];
            }
        } else if constexpr (VEC == 4) {
            const u2 v = *reinterpret_cast<const u2*>(p);
            r.w[0] = v[0];
            r.w[1] = v[1];
        } else {
            static_assert(VEC == 1, "parameter chunks of 1, 4 or a multiple of 8 elements");
            r.w[0] = p[0];
        }
    }
}

template <int VEC>
__device__ __forceinline__ uint32_t param_half(const PRaw<VEC>& r, int e)
{
    return (VEC == 1) ? (r.w[0] & 0xFFFFu) : ((r.w[e / 2] >> (16 * (e & 1))) & 0xFFFFu);
}

template <int VEC>
__device__ __forceinline__ void widen_param(const PRaw<VEC>& r, int pdt, bool valid,
                                            float (&dst)[VEC])
{
    // one uniform branch per chunk, each arm a straight run of conversions
    if (pdt == ST_F32) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) dst[e] = __uint_as_float(r.w[e]);
    } else if (pdt == ST_BF16) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) dst[e] = __uint_as_float(param_half(r, e) << 16);
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            dst[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)param_half(r, e));
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) dst[e] = valid ? dst[e] : 0.0f;
}

// One parameter element of runtime storage type pdt, widened to fp32.
__device__ __forceinline__ void load_scalar_param(const void* base, int pdt, int64_t i, float& v)
{
    if (pdt == ST_F32) v = static_cast<const float*>(base)[i];
    else if (pdt == ST_BF16) v = (float)static_cast<const __bf16*>(base)[i];
    else v = (float)static_cast<const _Float16*>(base)[i];
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

// Buffer resources: a span of one tensor (a GroupNorm slice, a tile of
// rows) as a raw buffer (base address and size in bytes in four scalar
// registers, word 3 the gfx9 raw-buffer format), so that every chunk load
// and store takes the span's base from scalar registers and one 32-bit
// offset register (with plain global addresses the compiler kept a 64-bit
// address per chunk across the reductions, which spilled the GroupNorm
// backward). An offset past the size reads 0 and drops a store: a chunk that is not to be written is
// stored at byte offset kNoStore instead of under a branch, so that every
// memory instruction of the loop is issued unconditionally and the compiler
// can count them (with a store under a divergent branch it waits for all of
// them, the prefetch included). kNoStore is a byte offset: scaled by an
// element size it would wrap to 0.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr uint32_t kNoStore = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void* p, int64_t byte_off,
                                                            uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(p) + byte_off), 0, (int)bytes, kRawBufferWord3);
}

// cache policy: 2 marks a non-temporal access
// `off` is the lane's element offset, `soff` a wave-uniform one (scalar).
template <int ST, int VEC, int NT>
__device__ __forceinline__ typename Chunk<ST, VEC>::type bload(__amdgpu_buffer_rsrc_t r,
                                                               uint32_t off, uint32_t soff)
{
    typedef typename Chunk<ST, VEC>::type C;
    constexpr int aux = (NT & 2) ? 2 : 0;
    constexpr uint32_t es = sizeof(typename Elem<ST>::type);
    const uint32_t b = off * es, sb = soff * es;
    if constexpr (sizeof(C) == 16) {
        return __builtin_bit_cast(C, __builtin_amdgcn_raw_buffer_load_b128(r, b, sb, aux));
    } else if constexpr (sizeof(C) == 4) {
        return __builtin_bit_cast(C, __builtin_amdgcn_raw_buffer_load_b32(r, b, sb, aux));
    } else {
        static_assert(sizeof(C) == 2, "chunk of 2, 4 or 16 bytes");
        return __builtin_bit_cast(C, __builtin_amdgcn_raw_buffer_load_b16(r, b, sb, aux));
    }
}

// `ok` false: the store is dropped (byte offset kNoStore). The whole offset
// goes in the offset register and the scalar offset is the constant 0: a
// store of more than 8 bytes with a scalar-register offset needs a wait
// state before the next write of its data registers, which this compiler
// did not insert (the next chunk's fp32 temporaries then replaced the first
// words of the stored data).
template <int ST, int VEC, int NT>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff,
                                       bool ok, const typename Chunk<ST, VEC>::type& v)
{
    typedef typename Chunk<ST, VEC>::type C;
    constexpr int aux = (NT & 1) ? 2 : 0;
    constexpr uint32_t es = sizeof(typename Elem<ST>::type);
    const uint32_t b = ok ? (off + soff) * es : kNoStore;
    constexpr uint32_t sb = 0;
    if constexpr (sizeof(C) == 32) {
        // binary32 dX from a 16-bit chunk of 8: two 16-byte stores
        typedef unsigned int u8v __attribute__((ext_vector_type(8)));
        const u8v w = __builtin_bit_cast(u8v, v);
        __builtin_amdgcn_raw_buffer_store_b128(u4{w[0], w[1], w[2], w[3]}, r, b, sb, aux);
        __builtin_amdgcn_raw_buffer_store_b128(u4{w[4], w[5], w[6], w[7]}, r, b + 16, sb, aux);
    } else if constexpr (sizeof(C) == 16) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, b, sb, aux);
    } else if constexpr (sizeof(C) == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, b, sb, aux);
    } else {
        static_assert(sizeof(C) == 2, "chunk of 2, 4, 16 or 32 bytes");
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, b, sb, aux);
    }
}

// Wait until every vector-memory operation issued so far has completed
// (s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima). Placed just
// before the next tile's loads are issued: the tile in registers is needed
// next anyway, and the compiler then has nothing older to wait for, so its
// own waits (it cannot count loads issued under divergent branches) no
// longer also cover the loads that are meant to stay in flight.
__device__ __forceinline__ void wait_vmem_all()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Wait until at most n vector-memory operations of this wave are
// outstanding (s_waitcnt vmcnt(n); the count is split over bits 3:0 and
// 15:14). The counter drops in issue order, so this waits for everything
// issued before the last n. It only makes the wave wait earlier: the
// compiler still places the waits that the registers it reads need.
template <int n>
__device__ __forceinline__ void wait_vmem_upto()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// tanh(u) from one exponential and one reciprocal: with
// q = 1 / (exp(2|u|) + 1), tanh(|u|) = 1 - 2q, and 1 - tanh(u)^2 = 4q(1 - q)
// (returned in `sd`; it keeps its relative precision where |tanh| is close
// to 1, and q -> 0 when the exponential overflows). Below |u| = 1/16 the
// difference 1 - 2q loses relative precision, so there tanh comes from its
// odd Taylor series u - u^3/3 + 2u^5/15, whose first omitted term is below
// 2^-32 |u|. The relative error of the returned tanh stays below about
// 2^-18 -- far inside a 16-bit ulp, not a binary32 one.
// exp(2a) as the hardware base-2 exponential of a * (2 log2 e): the same
// rounded argument as doubling a first (doubling is exact), one multiply
// fewer per element.
__device__ __forceinline__ float exp_twice(float a)
{
    return __builtin_amdgcn_exp2f(a * 2.8853900817779268f);
}

__device__ __forceinline__ float tanh_q(float u, float& sd)
{
    const float a = __builtin_fabsf(u);
    const float q = __builtin_amdgcn_rcpf(exp_twice(a) + 1.0f);
    sd = 4.0f * q * (1.0f - q);
    const float u2 = u * u;
    const float small = u * __builtin_fmaf(u2, __builtin_fmaf(u2, 2.0f / 15.0f, -1.0f / 3.0f), 1.0f);
    const float big = __builtin_copysignf(__builtin_fmaf(-2.0f, q, 1.0f), u);
    return a < 0.0625f ? small : big;
}

// The backward's tanh: 1 - tanh(u)^2 exactly as tanh_q (it scales dX), but
// tanh itself only enters the dgamma column sums, where a relative error of
// 2^-15 per term is far below what the fp32 sums can show. So below
// |u| = 1/128, where 1 - 2q would lose more than that, tanh(u) is u itself
// (relative error u^2/3 < 2^-15.6), with no polynomial: the Dynamic Tanh
// backward ran about 10 % faster at 16384 x 4096 than with tanh_q.
__device__ __forceinline__ float tanh_for_sums(float u, float& sd)
{
    const float a = __builtin_fabsf(u);
    const float q = __builtin_amdgcn_rcpf(exp_twice(a) + 1.0f);
    const float q4 = 4.0f * q;                 // exact
    sd = __builtin_fmaf(-q4, q, q4);           // 4q(1 - q), one rounding
    const float big = __builtin_copysignf(__builtin_fmaf(-2.0f, q, 1.0f), u);
    return a < 0.0078125f ? u : big;
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

template <int KIND, int ST, int T, int VEC, int CPT, int U, int BLOCK, int PF, int NT>
__global__ void __launch_bounds__(BLOCK) fwd_kernel(const FwdArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    constexpr int RPB = BLOCK / T;
    constexpr int TILE = RPB * U;
    // sums per row: none (DYT), three (POLY: sum of x^2, x^4, x^6), else one
    constexpr int NS = (KIND == DYT) ? 0 : (KIND == POLY) ? 3 : 1;
    constexpr int NSR = NS > 0 ? NS : 1;
    static_assert(BLOCK % T == 0, "block holds whole row groups");
    static_assert(PF == 0, "the forward runs one tile per workgroup: nothing to prefetch");
    __shared__ float red[RedBuf<T, RPB, U * NSR>::size];

    const int tid = threadIdx.x;
    const int g = tid / T;
    const int l = tid % T;
    const int D = a.D;
    // MOD: tiles are sample-major (each sample's S rows start a new tile), so
    // a tile never spans two samples and its rows share one scale and shift
    // row, loaded once per lane
    int64_t begin = (int64_t)blockIdx.x * TILE, end = a.N, soff = 0;
    if constexpr (KIND == MOD) {
        const int64_t tps = (a.S + TILE - 1) / TILE;
        const int64_t smp = (int64_t)blockIdx.x / tps;
        begin = smp * a.S + ((int64_t)blockIdx.x - smp * tps) * TILE;
        end = (smp + 1) * a.S;
        soff = smp * (int64_t)a.D;
    }

    int coff[CPT];
    bool cval[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        coff[k] = (k * T + l) * VEC;
        cval[k] = coff[k] < D;
    }

    constexpr bool HAS_G = KIND != POLY;
    constexpr bool HAS_B = KIND == LN || KIND == DYT;
    PRaw<VEC> graw[CPT], braw[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        if (cval[k]) {
            if constexpr (HAS_G) load_param_raw<VEC>(a.gamma, a.pdt, coff[k], graw[k]);
            if constexpr (HAS_B) load_param_raw<VEC>(a.beta, a.pdt, coff[k], braw[k]);
        }
    }
    float alpha = 0.0f, pw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (KIND == DYT) alpha = *a.alpha;
    if constexpr (KIND == POLY) {
#pragma unroll
        for (int q = 0; q < 4; ++q) pw[q] = a.poly[q];
    }

    struct Tile {
        HV x[U][CPT];
        HV r[U][CPT];
        HV sc[CPT], sh[CPT];   // MOD: the tile's sample's scale and shift
    };
    auto load_tile = [&](Tile& t, int64_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + u * RPB + g;
            const int64_t ro = row * (int64_t)D;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                const bool ok = row < end && cval[k];
                t.x[u][k] = ok ? sload<ST, VEC, NT>(a.X, ro + coff[k]) : czero<ST, VEC>();
                if constexpr (KIND == ADD) t.r[u][k] = ok ? sload<ST, VEC, NT>(a.R, ro + coff[k]) : czero<ST, VEC>();
            }
        }
        if constexpr (KIND == MOD) {
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                t.sc[k] = cval[k] ? sload<ST, VEC, 0>(a.scale, soff + coff[k]) : czero<ST, VEC>();
                t.sh[k] = cval[k] ? sload<ST, VEC, 0>(a.shift, soff + coff[k]) : czero<ST, VEC>();
            }
        }
    };

    const float fD = (float)D;
    int phase = 0;
    // parameter and tile loads are all in flight before the first wait
    Tile cur;
    load_tile(cur, begin);
    float gam[CPT][VEC], bet[CPT][VEC];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        if constexpr (HAS_G) widen_param<VEC>(graw[k], a.pdt, cval[k], gam[k]);
        if constexpr (HAS_B) widen_param<VEC>(braw[k], a.pdt, cval[k], bet[k]);
    }
    {
        const int64_t base = begin;
        int64_t row[U];
        bool rv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            row[u] = base + u * RPB + g;
            rv[u] = row[u] < end;
        }

        // First reduction: sum of squares (RMS, ADD, MOD), plain sum (LN),
        // sums of the second, fourth and sixth powers (POLY); none for DYT.
        float s1[U * NSR];
        if constexpr (NS > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float acc[NSR];
#pragma unroll
                for (int q = 0; q < NSR; ++q) acc[q] = 0.0f;
#pragma unroll
                for (int k = 0; k < CPT; ++k)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        float v = cget<ST, VEC>(cur.x[u][k], e);
                        if constexpr (KIND == ADD) v += cget<ST, VEC>(cur.r[u][k], e);
                        if constexpr (KIND == LN) {
                            acc[0] += v;
                        } else if constexpr (KIND == POLY) {
                            const float v2 = v * v;
                            const float v3 = v2 * v;
                            acc[0] = __builtin_fmaf(v, v, acc[0]);
                            acc[1] = __builtin_fmaf(v2, v2, acc[1]);
                            acc[2] = __builtin_fmaf(v3, v3, acc[2]);
                        } else {
                            acc[0] = __builtin_fmaf(v, v, acc[0]);
                        }
                    }
#pragma unroll
                for (int q = 0; q < NSR; ++q) s1[u * NSR + q] = acc[q];
            }
            row_sum<T, RPB, U * NSR>(s1, red, phase, g, l);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    launder(cur.x[u][k]);
                    if constexpr (KIND == ADD) launder(cur.r[u][k]);
                }
        }

        float mu[U], rs[U * NSR];
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
                        const float c = cget<ST, VEC>(cur.x[u][k], e) - mu[u];
                        acc = cval[k] ? __builtin_fmaf(c, c, acc) : acc;
                    }
                s2[u] = acc;
            }
            row_sum<T, RPB, U>(s2, red, phase, g, l);
#pragma unroll
            for (int u = 0; u < U; ++u) rs[u] = 1.0f / sqrtf(s2[u] / fD + a.eps);
        } else if constexpr (NS > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                mu[u] = 0.0f;
#pragma unroll
                for (int q = 0; q < NSR; ++q)
                    rs[u * NSR + q] = 1.0f / sqrtf(s1[u * NSR + q] / fD + a.eps);
            }
        }

#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (NS > 0) {
                if (l == 0 && rv[u]) {
                    if constexpr (KIND == POLY) {
#pragma unroll
                        for (int q = 0; q < 3; ++q) a.rstd[row[u] * 3 + q] = rs[u * NSR + q];
                    } else {
                        a.rstd[row[u]] = rs[u];
                    }
                    if constexpr (KIND == LN) a.mean[row[u]] = mu[u];
                }
            }
            const int64_t ro = row[u] * (int64_t)D;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                if (!(rv[u] && cval[k])) continue;
                // POLY: y = b + v (w1 r1 + v (w2 r2 + v w3 r3)), Horner form
                float k1 = 0.0f, k2 = 0.0f, k3 = 0.0f;
                if constexpr (KIND == POLY) {
                    k1 = pw[0] * rs[u * NSR];
                    k2 = pw[1] * rs[u * NSR + 1];
                    k3 = pw[2] * rs[u * NSR + 2];
                }
                HV y;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float v = cget<ST, VEC>(cur.x[u][k], e);
                    if constexpr (KIND == ADD) v += cget<ST, VEC>(cur.r[u][k], e);
                    float o;
                    if constexpr (KIND == LN) {
                        o = __builtin_fmaf((v - mu[u]) * rs[u], gam[k][e], bet[k][e]);
                    } else if constexpr (KIND == DYT) {
                        // 16-bit outputs take the one-exponential tanh; binary32
                        // outputs the library's
                        float t;
                        if constexpr (ST == ST_F32) {
                            t = tanhf(alpha * v);
                        } else {
                            float sd_unused;
                            t = tanh_q(alpha * v, sd_unused);
                        }
                        o = __builtin_fmaf(gam[k][e], t, bet[k][e]);
                    } else if constexpr (KIND == POLY) {
                        o = __builtin_fmaf(v, __builtin_fmaf(v, __builtin_fmaf(v, k3, k2), k1),
                                           pw[3]);
                    } else if constexpr (KIND == MOD) {
                        o = __builtin_fmaf(v * rs[u] * gam[k][e],
                                           1.0f + cget<ST, VEC>(cur.sc[k], e),
                                           cget<ST, VEC>(cur.sh[k], e));
                    } else {
                        o = v * rs[u] * gam[k][e];
                    }
                    cset<ST, VEC>(y, e, o);
                }
                cstore<ST, VEC, NT>(a.Y, ro + coff[k], y);
                if constexpr (KIND == ADD) {
                    // the exact sum rounded once to the storage type
                    const HV h = round_sum<ST, VEC>(cur.x[u][k], cur.r[u][k]);
                    cstore<ST, VEC, NT>(a.H, ro + coff[k], h);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Backward stage 1: dX and per-workgroup parameter-gradient partials.
// ---------------------------------------------------------------------------

// Sum of one value per lane over the whole workgroup in a fixed order: the
// wave-level tree of group_sum, then the per-wave totals in wave order.
// Every thread must call it (it has barriers); lane 0 of wave 0 gets the sum.
template <int BLOCK>
__device__ __forceinline__ float block_sum(float v, float* scratch)
{
    v = group_sum<64>(v);
    if constexpr (BLOCK > 64) {
        const int w = threadIdx.x >> 6;
        __syncthreads();
        if ((threadIdx.x & 63) == 0) scratch[w] = v;
        __syncthreads();
        if (threadIdx.x == 0) {
            float t = scratch[0];
#pragma unroll
            for (int ww = 1; ww < BLOCK / 64; ++ww) t += scratch[ww];
            v = t;
        }
    }
    return v;
}

// Constants kept in registers where the compiler cannot see their values:
// a -0 addend turns a product x * b into fma(x, b, -0), which is the rounded
// product bitwise (sign of zero included) but, unlike a multiply, takes a
// 16-bit x as a mixed-precision operand (v_fma_mix_f32: the conversion to
// fp32 costs no instruction); likewise x + c as fma(x, 1, c). With visible
// constants the compiler folds both back into a conversion and a multiply
// or an add.
struct MixConst {
    float nz, one;
};

__device__ __forceinline__ MixConst mix_const()
{
    MixConst m{-0.0f, 1.0f};
    asm volatile("" : "+v"(m.nz), "+v"(m.one));
    return m;
}

// ---------------------------------------------------------------------------
// The end of the one-launch backward of a small problem: each workgroup,
// once its partial rows are stored device-coherently, sets its flag to this
// call's epoch + 1 and reads every flag; a workgroup that finds them all set
// adds the P partial rows (P = gridDim.x, a power of two up to 64) in the
// column-reduce kernel's order, so dgamma (dbeta) is bitwise that of the
// two-launch backward.
//
// Nothing waits on another workgroup: the last flag to be stored is followed
// by its own workgroup's reads, which see every flag (each flag is stored
// only after its workgroup's partial rows completed, and read only after the
// reader's own flag completed); any other workgroup that also sees them all
// writes the same values. Every workgroup reads the epoch before storing its
// flag, so the epoch, advanced by the reducer for the next call, changes
// only after all have read it; calls on one stream run in order.
//
// The column-reduce kernel sums 64 segments, here one row each (0 past P),
// each from 0.0f, then pairwise (h = 32, 16, .., 1). P is a power of two on
// this path, and the levels h >= P add +0 to a value that is never -0, so
// they change nothing: the P-leaf tree gives the same bits. A lane holds
// NV x P x W values (W adjacent columns of each plane, one 4 W-byte load per
// row). The loads
// are device-coherent (scope bit sc1 of the buffer load: no line of the
// XCD's own L2 is returned), so no cache invalidation precedes them. Their
// byte offset walks in a vector register so that the P row offsets are not
// all held in scalar registers (which spilled them into a vector register
// of every kernel that carries this path).
// ---------------------------------------------------------------------------
constexpr int kBufferSc1 = 16;             // cache-policy operand: sc1

template <int P, int W, int BLOCK, int NV>
__device__ __forceinline__ void small_rows_sum(const BwdArgs& a, int D, int tid)
{
    static_assert(W == 1 || W == 2 || W == 4, "load width");
    __amdgpu_buffer_rsrc_t r[NV];
#pragma unroll
    for (int y = 0; y < NV; ++y)
        r[y] = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(y == 0 ? a.part_g : a.part_b),
                                                 0, P * a.Dp * (int)sizeof(float), kRawBufferWord3);
#pragma unroll 1
    for (int c = tid * W; c < D; c += BLOCK * W) {
        // both planes' loads are issued before either is added
        float v[NV][P][W];
        uint32_t off = (uint32_t)c * sizeof(float);
#pragma unroll
        for (int q = 0; q < P; ++q) {
#pragma unroll
            for (int y = 0; y < NV; ++y) {
                float x[W];
                if constexpr (W == 4) {
                    const f4 t = __builtin_bit_cast(
                        f4, __builtin_amdgcn_raw_buffer_load_b128(r[y], off, 0, kBufferSc1));
                    x[0] = t[0]; x[1] = t[1]; x[2] = t[2]; x[3] = t[3];
                } else if constexpr (W == 2) {
                    typedef float f2 __attribute__((ext_vector_type(2)));
                    const f2 t = __builtin_bit_cast(
                        f2, __builtin_amdgcn_raw_buffer_load_b64(r[y], off, 0, kBufferSc1));
                    x[0] = t[0]; x[1] = t[1];
                } else {
                    x[0] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(r[y], off, 0, kBufferSc1));
                }
#pragma unroll
                for (int e = 0; e < W; ++e) v[y][q][e] = 0.0f + x[e];
            }
            off += (uint32_t)a.Dp * sizeof(float);
            asm volatile("" : "+v"(off));  // no instruction: keeps off in a VGPR
        }
#pragma unroll
        for (int y = 0; y < NV; ++y) {
#pragma unroll
            for (int h = P / 2; h > 0; h /= 2)
#pragma unroll
                for (int q = 0; q < h; ++q)
#pragma unroll
                    for (int e = 0; e < W; ++e) v[y][q][e] = v[y][q][e] + v[y][q + h][e];
            float* out = y == 0 ? a.dgamma : a.dbeta;
#pragma unroll
            for (int e = 0; e < W; ++e)
                if (c + e < D) out[c + e] = v[y][0][e];
        }
    }
}

template <int BLOCK, int NV>
__device__ __forceinline__ void small_backward_reduce(const BwdArgs& a, int D, int tid)
{
    __shared__ int s_all;
    const int P = (int)gridDim.x;
    uint64_t e = 0;
    if (tid < 64)
        e = __hip_atomic_load(&a.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's partial rows (and the epoch) are in
    __syncthreads();
    if (tid < 64) {
        if (tid == 0)
            __hip_atomic_store(&a.sync[1 + blockIdx.x], e + 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the flag is stored
        const bool set = tid >= P || __hip_atomic_load(&a.sync[1 + tid], __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT) == e + 1;
        const uint64_t unset = __ballot(!set);
        if (tid == 0) {
            s_all = unset == 0;
            if (unset == 0)
                __hip_atomic_store(&a.sync[0], e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    if (!s_all) return;
    switch (P) {
    case 1: small_rows_sum<1, 4, BLOCK, NV>(a, D, tid); break;
    case 2: small_rows_sum<2, 4, BLOCK, NV>(a, D, tid); break;
    case 4: small_rows_sum<4, 4, BLOCK, NV>(a, D, tid); break;
    case 8: small_rows_sum<8, 4, BLOCK, NV>(a, D, tid); break;
    case 16: small_rows_sum<16, 4, BLOCK, NV>(a, D, tid); break;
    case 32: small_rows_sum<32, 2, BLOCK, NV>(a, D, tid); break;
    case 64: small_rows_sum<64, 1, BLOCK, NV>(a, D, tid); break;
    }
}

// Storage types: ST for X and R (and MOD's scale), CT for the cotangents dY
// and dH, OT for dX.
//
// Arithmetic per element (the row-constant factors are formed once per row;
// every product of a 16-bit input is a mixed-precision fma, see MixConst):
//   RMS, ADD, MOD (v = x, or x + r for ADD; w = gamma, or gamma * (1 + scale)
//   for MOD's sample; g = dY w): the row sum S = sum_j g v, so c1 =
//   mean(g xhat) = rstd S / D; then dX = rstd (g - xhat c1) [+ dH, in the
//   last fma] with xhat = v rstd.
//   LN: c1 = mean(g xhat) = rstd mean(g (x - mean)), c2 = mean(g), and
//   dX = rstd (g - c2 - xhat c1) with xhat = (x - mean) rstd, in this order
//   (exact zeros stay exact).
// The row means multiply by the rounded 1/D (one ulp of fp32 from a
// division at most).
template <int KIND, int ST, int CT, int OT, int T, int VEC, int CPT, int U, int BLOCK, int PF,
          int NT>
__global__ void __launch_bounds__(BLOCK) bwd_kernel(const BwdArgs a)
{
    typedef typename Chunk<ST, VEC>::type HV;
    typedef typename Chunk<CT, VEC>::type CV;
    typedef typename Chunk<OT, VEC>::type OV;
    constexpr int RPB = BLOCK / T;
    constexpr int TILE = RPB * U;
    // sums per row: c1 (and c2 for LN; three for POLY; none for DYT)
    // POLY's four: sum(dY * x^p) for p = 1, 2, 3 and sum(dY)
    constexpr int NR = (KIND == LN) ? 2 : (KIND == POLY) ? 4 : (KIND == DYT) ? 0 : 1;
    constexpr int NRR = NR > 0 ? NR : 1;
    // per-column partial arrays: dgamma (+ dbeta for LN and DYT, + dscale and
    // dshift for MOD); POLY has only scalar parameters
    constexpr int NV = (KIND == LN || KIND == DYT) ? 2 : (KIND == MOD) ? 3 : (KIND == POLY) ? 0 : 1;
    // per-workgroup scalar partials: dalpha (DYT), dw1..dw3 and db (POLY)
    constexpr int NSC = (KIND == DYT) ? 1 : (KIND == POLY) ? 4 : 0;
    constexpr int NQ = (KIND == POLY) ? 3 : 1;  // saved rstd values per row
    // the kinds whose row sum is S = sum(dY w v)
    constexpr bool RMSLIKE = KIND == RMS || KIND == ADD || KIND == MOD;
    static_assert(BLOCK % T == 0, "block holds whole row groups");
    __shared__ float red[RedBuf<T, RPB, U * NRR>::size];
    __shared__ float wsum[BLOCK / 64 > 0 ? BLOCK / 64 : 1];
    extern __shared__ float fold[];           // [NV][D] when RPB > 1

    const int tid = threadIdx.x;
    const int g = tid / T;
    const int l = tid % T;
    const int D = a.D;
    // Workgroup b owns tiles b, b + P, b + 2P, ... (P = gridDim.x): a fixed
    // set of rows, so its partials are reproducible, while the P workgroups
    // running together touch one contiguous band of rows. For MOD the
    // workgroups are split by sample: workgroup b serves sample b / Pb and
    // owns the tiles b % Pb, b % Pb + Pb, ... of that sample's rows, so its
    // dscale and dshift partials belong to one sample.
    int64_t row0 = 0, end = a.N, first, stop, tstride;
    if constexpr (KIND == MOD) {
        const int64_t smp = blockIdx.x / a.Pb;
        row0 = smp * a.S;
        end = row0 + a.S;
        first = row0 + (int64_t)(blockIdx.x % a.Pb) * TILE;
        stop = row0 + (a.S + TILE - 1) / TILE * TILE;
        tstride = (int64_t)a.Pb * TILE;
    } else {
        first = (int64_t)blockIdx.x * TILE;
        stop = (a.N + TILE - 1) / TILE * TILE;  // uniform loop bound for the workgroup
        tstride = (int64_t)gridDim.x * TILE;
    }

    int coff[CPT];
    bool cval[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        coff[k] = (k * T + l) * VEC;
        cval[k] = coff[k] < D;
    }
    constexpr bool HAS_G = KIND != POLY;
    PRaw<VEC> graw[CPT];
    HV scr[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        if constexpr (HAS_G)
            if (cval[k]) load_param_raw<VEC>(a.gamma, a.pdt, coff[k], graw[k]);
        if constexpr (KIND == MOD)
            scr[k] = cval[k] ? sload<ST, VEC, 0>(a.scale, (row0 / a.S) * D + coff[k])
                             : czero<ST, VEC>();
    }
    float alpha = 0.0f, pw[3] = {0.0f, 0.0f, 0.0f};
    if constexpr (KIND == DYT) alpha = *a.alpha;
    if constexpr (KIND == POLY) {
#pragma unroll
        for (int q = 0; q < 3; ++q) pw[q] = a.poly[q];
    }
    const MixConst mc = mix_const();

    float accg[CPT][VEC], accb[CPT][VEC], acch[CPT][VEC], accs[NSC > 0 ? NSC : 1];
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            accg[k][e] = 0.0f;
            accb[k][e] = 0.0f;
            acch[k][e] = 0.0f;
        }
#pragma unroll
    for (int q = 0; q < (NSC > 0 ? NSC : 1); ++q) accs[q] = 0.0f;

    // RMS, LN, ADD and MOD load every chunk unconditionally: a row past the
    // end reads the last row again and a column past D the row's first
    // chunk. Their terms vanish where they could reach a result: the row's
    // rstd (and so xhat and dY * rstd) is 0 past the end, gamma is 0 past D,
    // and the plain sums of dY (LN's dbeta, MOD's dshift) take a 0/1 row
    // mask. Nothing is stored for them, and their row sums are not used.
    // (Zero-filling the registers of masked loads instead cost about one
    // instruction per element.) DYT and POLY sum dY and x without such a
    // factor and keep the masked loads.
    constexpr bool CLAMP = RMSLIKE || KIND == LN;
    // LN only (measured 1 % slower for RMS and MOD, 1 % faster for LN): the
    // statistics loaded unconditionally and dX stored through a buffer
    // resource, so that every memory instruction of a step is issued and
    // counted, and each step waits for its own tile's loads, not for the
    // previous tile's stores (and fewer registers: 170 VGPRs instead of 200
    // for the 256-lane shape at 4096 columns)
    constexpr bool BUFST = KIND == LN;
    int coffc[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) coffc[k] = cval[k] ? coff[k] : 0;

    struct Tile {
        HV x[U][CPT], r[U][CPT];
        CV dy[U][CPT];
        float rs[U][NQ], mu[U], rm[U];
    };
    auto load_tile = [&](Tile& t, int64_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + u * RPB + g;
            const bool rok = row < end;
            if constexpr (BUFST) {
                // unconditional loads (the last row's statistics past the
                // end); process() zeroes rstd there
                const int64_t rc = rok ? row : end - 1;
                t.rs[u][0] = a.rstd[rc];
                t.mu[u] = a.mean[rc];
            } else {
                if constexpr (KIND != DYT) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) t.rs[u][q] = rok ? a.rstd[row * NQ + q] : 0.0f;
                }
                t.mu[u] = (KIND == LN && rok) ? a.mean[row] : 0.0f;
            }
            t.rm[u] = rok ? 1.0f : 0.0f;
            if constexpr (CLAMP) {
                const int64_t ro = (rok ? row : end - 1) * (int64_t)D;
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    t.x[u][k] = sload<ST, VEC, NT>(a.X, ro + coffc[k]);
                    if constexpr (KIND == ADD) t.r[u][k] = sload<ST, VEC, NT>(a.R, ro + coffc[k]);
                    t.dy[u][k] = sload<CT, VEC, NT>(a.dY, ro + coffc[k]);
                }
            } else {
                const int64_t ro = row * (int64_t)D;
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    const bool ok = rok && cval[k];
                    t.x[u][k] = ok ? sload<ST, VEC, NT>(a.X, ro + coff[k]) : czero<ST, VEC>();
                    t.dy[u][k] = ok ? sload<CT, VEC, NT>(a.dY, ro + coff[k]) : czero<CT, VEC>();
                }
            }
        }
    };

    const float invD = 1.0f / (float)D;
    int phase = 0;
    // gam: gamma; gef: the weight the row sees (MOD: gamma * (1 + scale) of
    // this workgroup's sample, else gamma); scl: 1 + scale (MOD)
    float gam[CPT][VEC], gef[CPT][VEC], scl[CPT][VEC];

    // The row value v: x, or for ADD the sum x + r rounded once to fp32.
    auto value = [&](const Tile& t, int u, int k, int e) -> float {
        if constexpr (KIND == ADD)
            return __builtin_fmaf(cget<ST, VEC>(t.x[u][k], e), mc.one, cget<ST, VEC>(t.r[u][k], e));
        else
            return cget<ST, VEC>(t.x[u][k], e);
    };

    // One tile: the row sums, then dX and the parameter-gradient terms.
    auto process = [&](Tile& cur, int64_t base) {
        // Row sums. RMS, ADD, MOD: S = sum(dY w v); LN: sum(g xhat) and
        // sum(g); POLY: sum(dY x^p) for p = 1..3 and sum(dY).
        float c[U * NRR];
        if constexpr (NR > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float acc[NRR];
#pragma unroll
                for (int q = 0; q < NRR; ++q) acc[q] = 0.0f;
                const float nmu = -cur.mu[u];
#pragma unroll
                for (int k = 0; k < CPT; ++k)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float dyv = cget<CT, VEC>(cur.dy[u][k], e);
                        if constexpr (KIND == POLY) {
                            const float v = cget<ST, VEC>(cur.x[u][k], e);
                            const float v2 = v * v;
                            acc[0] = __builtin_fmaf(dyv, v, acc[0]);
                            acc[1] = __builtin_fmaf(dyv, v2, acc[1]);
                            acc[2] = __builtin_fmaf(dyv, v2 * v, acc[2]);
                            acc[3] += dyv;
                        } else if constexpr (KIND == LN) {
                            // sum(g (x - mean)); times rstd once per row
                            const float t = __builtin_fmaf(cget<ST, VEC>(cur.x[u][k], e), mc.one,
                                                           nmu);
                            const float gg = __builtin_fmaf(dyv, gef[k][e], mc.nz);
                            acc[0] = __builtin_fmaf(gg, t, acc[0]);
                            acc[1] += gg;
                        } else {
                            const float gg = __builtin_fmaf(dyv, gef[k][e], mc.nz);
                            acc[0] = __builtin_fmaf(gg, value(cur, u, k, e), acc[0]);
                        }
                    }
#pragma unroll
                for (int q = 0; q < NRR; ++q) c[u * NRR + q] = acc[q];
            }
            row_sum<T, RPB, U * NRR>(c, red, phase, g, l);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    launder(cur.x[u][k]);
                    launder(cur.dy[u][k]);
                    if constexpr (KIND == ADD) launder(cur.r[u][k]);
                }
        }

        // LN: the tile's valid rows of dX as one raw buffer; every chunk store
        // is issued, those past D or past the last row at kNoStore (no store
        // under a branch, so the compiler can count them)
        constexpr int64_t oes = sizeof(typename Elem<OT>::type);
        const int64_t nval = (end - base < TILE) ? end - base : TILE;
        const __amdgpu_buffer_rsrc_t dxr =
            slice_rsrc(a.dX, base * D * oes, (uint32_t)(nval * D * oes));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = base + u * RPB + g;
            const bool rok = row < end;
            const float rs = (KIND == DYT) ? 0.0f : (BUFST && !rok) ? 0.0f : cur.rs[u][0];
            // row constants
            float c1 = 0.0f, c2 = 0.0f;
            if constexpr (RMSLIKE) {
                c1 = rs * (c[u * NRR] * invD);                  // mean(g xhat) = rstd S / D
            } else if constexpr (KIND == LN) {
                c1 = rs * (c[u * NRR] * invD);                  // mean(g xhat)
                c2 = c[u * NRR + 1] * invD;                     // mean(g)
            }
            const float nmu = -cur.mu[u];
            const int64_t ro = row * (int64_t)D;
            // POLY: with S_p = sum(dY x^p) and n_p = x^p r_p, mean(dY n_p) =
            // r_p S_p / D, and
            //   dX = dY (A1 + x (A2 + x A3)) - x (B1 + x^2 (B2 + x^2 B3)),
            //   A_p = p w_p r_p,  B_p = p w_p r_p^2 mean(dY n_p).
            // The row's shares of dw_p (r_p S_p) and db (S_0) are added once,
            // by the row group's first lane.
            float A1 = 0.0f, A2 = 0.0f, A3 = 0.0f, B1 = 0.0f, B2 = 0.0f, B3 = 0.0f;
            if constexpr (KIND == POLY) {
                const float c1 = c[u * NRR] * invD, c2 = c[u * NRR + 1] * invD;
                const float c3 = c[u * NRR + 2] * invD;
                const float r1 = cur.rs[u][0], r2 = cur.rs[u][1], r3 = cur.rs[u][2];
                const float m1 = r1 * c1, m2 = r2 * c2, m3 = r3 * c3;
                A1 = pw[0] * r1;
                A2 = 2.0f * pw[1] * r2;
                A3 = 3.0f * pw[2] * r3;
                B1 = A1 * r1 * m1;
                B2 = A2 * r2 * m2;
                B3 = A3 * r3 * m3;
                if (l == 0) {
                    accs[0] = __builtin_fmaf(r1, c[u * NRR], accs[0]);
                    accs[1] = __builtin_fmaf(r2, c[u * NRR + 1], accs[1]);
                    accs[2] = __builtin_fmaf(r3, c[u * NRR + 2], accs[2]);
                    accs[3] += c[u * NRR + 3];
                }
            }
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                const bool ok = rok && cval[k];
                CV dh = czero<CT, VEC>();
                if constexpr (KIND == ADD) {
                    if (ok && a.dH != nullptr) dh = sload<CT, VEC, NT>(a.dH, ro + coff[k]);
                }
                OV o;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float dyv = cget<CT, VEC>(cur.dy[u][k], e);
                    float d;
                    if constexpr (KIND == DYT) {
                        // dX needs only 1 - t^2; t enters only the dgamma
                        // sums
                        const float v = cget<ST, VEC>(cur.x[u][k], e);
                        float sd;
                        const float t = tanh_for_sums(alpha * v, sd);
                        const float gy = dyv * gam[k][e];
                        const float gs = gy * sd;
                        d = gs * alpha;
                        accg[k][e] = __builtin_fmaf(dyv, t, accg[k][e]);
                        accb[k][e] += dyv;
                        accs[0] = __builtin_fmaf(gs, v, accs[0]);
                    } else if constexpr (KIND == POLY) {
                        const float v = cget<ST, VEC>(cur.x[u][k], e);
                        const float v2 = v * v;
                        const float P = __builtin_fmaf(v, __builtin_fmaf(v, A3, A2), A1);
                        const float Q = __builtin_fmaf(v2, __builtin_fmaf(v2, B3, B2), B1);
                        d = __builtin_fmaf(dyv, P, -(v * Q));
                    } else if constexpr (KIND == LN) {
                        // (x - mean) rstd and rstd (g - c2 - xhat c1) as
                        // written: a constant row gives xhat = 0 and, with
                        // D = 1, g - c2 = 0 exactly
                        const float xh = (__builtin_fmaf(cget<ST, VEC>(cur.x[u][k], e), mc.one,
                                                         nmu) * rs);
                        const float gg = __builtin_fmaf(dyv, gam[k][e], mc.nz);
                        d = rs * __builtin_fmaf(-xh, c1, gg - c2);
                        accg[k][e] = __builtin_fmaf(dyv, xh, accg[k][e]);
                        accb[k][e] = __builtin_fmaf(dyv, cur.rm[u], accb[k][e]);
                    } else {
                        // RMS, ADD, MOD: rstd (g - xhat c1), for ADD with dH
                        // in the last fma (a dX that cancels dH against the
                        // norm term is rounded once)
                        const float v = value(cur, u, k, e);
                        const float xh = (KIND == ADD) ? v * rs : __builtin_fmaf(v, rs, mc.nz);
                        const float gg = __builtin_fmaf(dyv, gef[k][e], mc.nz);
                        const float in = __builtin_fmaf(-xh, c1, gg);
                        if constexpr (KIND == ADD) d = __builtin_fmaf(rs, in, cget<CT, VEC>(dh, e));
                        else d = rs * in;
                        if constexpr (KIND == MOD) {
                            // dgamma takes dY * xhat * (1 + scale), dscale
                            // dY * xhat * gamma, dshift dY
                            const float dx = __builtin_fmaf(dyv, xh, mc.nz);
                            accg[k][e] = __builtin_fmaf(dx, scl[k][e], accg[k][e]);
                            accb[k][e] = __builtin_fmaf(dx, gam[k][e], accb[k][e]);
                            acch[k][e] = __builtin_fmaf(dyv, cur.rm[u], acch[k][e]);
                        } else {
                            accg[k][e] = __builtin_fmaf(dyv, xh, accg[k][e]);
                        }
                    }
                    cset<OT, VEC>(o, e, d);
                }
                if constexpr (BUFST)
                    bstore<OT, VEC, NT>(dxr, (uint32_t)((u * RPB + g) * D + coff[k]), 0, ok, o);
                else if (ok)
                    cstore<OT, VEC, NT>(a.dX, ro + coff[k], o);
            }
        }
    };

    // Two tile buffers in turn: while one is reduced and written, the
    // other's loads are in flight, with no register copies between them.
    // Where registers are scarce (1024-lane workgroups, whose waves may hold
    // at most 128 VGPRs, and the element-wise variants) the loop keeps one
    // body and copies the prefetched tile instead, which the compiler
    // schedules in fewer registers.
    constexpr bool PINGPONG = VEC > 1 && BLOCK < 1024;
    Tile ta;
    load_tile(ta, first);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        if constexpr (HAS_G) widen_param<VEC>(graw[k], a.pdt, cval[k], gam[k]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (KIND == MOD) {
                scl[k][e] = 1.0f + cget<ST, VEC>(scr[k], e);
                gef[k][e] = gam[k][e] * scl[k][e];
            } else if constexpr (HAS_G) {
                gef[k][e] = gam[k][e];
            }
        }
    }
    static_assert(PF == 1, "the backward prefetches the next tile");
    // LN: the top of each step waits for the loads of the tile it is about
    // to reduce, not for the previous tile's dX stores (issued after them)
    constexpr int NSW = BUFST ? U * CPT * (((int)sizeof(OV) + 15) / 16) : 0;
    if constexpr (PINGPONG) {
        Tile tb;
        for (int64_t base = first; base < stop; base += 2 * tstride) {
            wait_vmem_upto<NSW>();
            load_tile(tb, base + tstride);
            process(ta, base);
            const int64_t b2 = base + tstride;
            if (b2 >= stop) break;
            wait_vmem_upto<NSW>();
            load_tile(ta, b2 + tstride);
            process(tb, b2);
        }
    } else {
        for (int64_t base = first; base < stop; base += tstride) {
            Tile nxt;
            wait_vmem_all();
            load_tile(nxt, base + tstride);
            process(ta, base);
            ta = nxt;
        }
    }

    // One-launch backward of a small problem (RMS, LN, ADD with a.sync set;
    // not in 1024-lane variants, whose 128 VGPRs the reduce would exceed).
    constexpr bool kOneLaunch = BLOCK < 1024 && NV > 0 && NV <= 2 && NSC == 0 && KIND != MOD;
    const bool one_launch = kOneLaunch && a.sync != nullptr;

    // Fold the row groups of this workgroup in group order, then write the
    // workgroup's partial rows: plain (write-back cached, 16-byte) stores, or
    // on the one-launch path device-coherent ones, written through to the
    // level every XCD reads.
    auto write_partials = [&](auto put) {
        float* pv[3] = {a.part_g + (int64_t)blockIdx.x * a.Dp,
                        NV > 1 ? a.part_b + (int64_t)blockIdx.x * a.Dp : nullptr,
                        NV > 2 ? a.part_h + (int64_t)blockIdx.x * a.Dp : nullptr};
        if constexpr (RPB == 1) {
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                if (!cval[k]) continue;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    put(&pv[0][coff[k] + e], accg[k][e]);
                    if constexpr (NV > 1) put(&pv[1][coff[k] + e], accb[k][e]);
                    if constexpr (NV > 2) put(&pv[2][coff[k] + e], acch[k][e]);
                }
            }
        } else {
            for (int j = tid; j < D; j += BLOCK) {
                put(&pv[0][j], fold[j]);
                if constexpr (NV > 1) put(&pv[1][j], fold[D + j]);
                if constexpr (NV > 2) put(&pv[2][j], fold[2 * D + j]);
            }
        }
    };
    if constexpr (NV > 0) {
        if constexpr (RPB > 1) {
            for (int gg = 0; gg < RPB; ++gg) {
                if (g == gg) {
#pragma unroll
                    for (int k = 0; k < CPT; ++k) {
                        if (!cval[k]) continue;
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const int j = coff[k] + e;
                            fold[j] = (gg == 0) ? accg[k][e] : fold[j] + accg[k][e];
                            if constexpr (NV > 1)
                                fold[D + j] = (gg == 0) ? accb[k][e] : fold[D + j] + accb[k][e];
                            if constexpr (NV > 2)
                                fold[2 * D + j] = (gg == 0) ? acch[k][e] : fold[2 * D + j] + acch[k][e];
                        }
                    }
                }
                __syncthreads();
            }
        }
        if (one_launch)
            write_partials([](float* q, float v) {
                __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            });
        else
            write_partials([](float* q, float v) { *q = v; });
    }
    if constexpr (kOneLaunch) {
        if (one_launch) small_backward_reduce<BLOCK, NV>(a, D, tid);
    }
    if constexpr (NSC > 0) {
#pragma unroll
        for (int q = 0; q < NSC; ++q) {
            const float t = block_sum<BLOCK>(accs[q], wsum);
            if (tid == 0) a.part_a[(int64_t)blockIdx.x * 4 + q] = t;
        }
    }
}

// ---------------------------------------------------------------------------
// Backward stage 2: out[j] = sum over the P partial rows of partial[p][j]
// (per group z of P rows when there are several groups), for every plane of
// the launch (blockIdx.y; a parameter gradient each, all in one launch).
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
    // the plane by constant indices (a dynamic index would copy the
    // arguments to scratch memory)
    const ReducePlane pl = blockIdx.y == 0 ? a.plane[0] : blockIdx.y == 1 ? a.plane[1] : a.plane[2];
    // the grid covers the largest plane: blocks past this one's columns or
    // groups have nothing to do (a whole block returns, before any barrier)
    if ((int)blockIdx.z >= pl.groups || (int)blockIdx.x * 4 * CQ >= pl.Dp) return;
    // group z: rows z*P .. z*P + P - 1 of the plane, into out[z*D ...]
    const float* part = pl.part + (int64_t)blockIdx.z * pl.P * pl.Dp;
    float* out = pl.out + (int64_t)blockIdx.z * pl.D;
    const int q = threadIdx.x % CQ;
    const int s = threadIdx.x / CQ;
    const int c0 = (blockIdx.x * CQ + q) * 4;
    const int64_t per = (pl.P + SEG - 1) / SEG;
    const int64_t p0 = min(pl.P, (int64_t)s * per);
    const int64_t p1 = min(pl.P, p0 + per);
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c0 < pl.Dp) {
        const float* src = part + c0;
#pragma unroll 8
        for (int64_t p = p0; p < p1; ++p) acc += *reinterpret_cast<const f4*>(src + p * pl.Dp);
    }
    seg_sum[s][q] = acc;
    __syncthreads();
#pragma unroll
    for (int st = SEG / 2; st > 0; st /= 2) {
        if (s < st) seg_sum[s][q] = seg_sum[s][q] + seg_sum[s + st][q];
        __syncthreads();
    }
    if (s == 0 && c0 < pl.D) {
        const f4 t = seg_sum[0][q];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c0 + e < pl.D) out[c0 + e] = t[e];
    }
}

}  // namespace kern
}  // namespace mn
