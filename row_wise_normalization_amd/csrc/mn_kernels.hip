// mn_kernels.hip -- launch tables of the gfx950 normalization kernels
// (templates in mn_kernels.hpp): which template instance serves which width,
// the grid of every launch, and the dispatch from the C ABI layer.
#include "mn_kernels.hpp"

namespace mn {
namespace {

using kern::bwd_kernel;
using kern::fwd_kernel;
using kern::reduce_kernel;

constexpr int kReduceCQ = 16;  // 64 columns per block, 64 segments

// ---------------------------------------------------------------------------
// Variant tables.
// ---------------------------------------------------------------------------

// Variant tables, one per norm kind and direction; a row is chosen by the
// smallest max_d >= D. Shapes come from timing sweeps on MI355X at
// 16384x4096, 32768x8192 and 1048576x128:
//   * the forward runs one tile per workgroup (many small workgroups keep
//     the most reads in flight);
//   * the backward runs 256 long-lived workgroups (each owns one partial
//     row of dgamma and the tiles b, b+256, ...), prefetches its next tile
//     and keeps two rows per row group in flight;
//   * streamed outputs use non-temporal stores (NT bit 0) and streamed
//     inputs non-temporal loads (NT bit 1), except the LayerNorm forward,
//     which measured slower with non-temporal loads.
// Ids are unique within a kind; 8..10 are the element-wise variants (any D,
// any alignment) shared by all kinds. Each row is instantiated for binary16,
// bfloat16 and binary32 storage (binary32: see st_vec / st_cpt below).
//
//   id   T  VEC CPT  U  BLOCK  PF NT  max_d
#define MN_FWD_RMS(X)                        \
    X(0, 8, 8, 1, 4, 256, 0, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 0, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 0, 3, 256)        \
    X(3, 64, 8, 1, 2, 256, 0, 3, 512)        \
    X(4, 128, 8, 1, 1, 256, 0, 3, 1024)      \
    X(5, 256, 8, 1, 1, 256, 0, 3, 2048)      \
    X(6, 256, 8, 2, 1, 256, 0, 3, 4096)      \
    X(7, 1024, 8, 1, 1, 1024, 0, 3, 8192)
#define MN_FWD_LN(X)                         \
    X(0, 8, 8, 1, 4, 256, 0, 1, 64)          \
    X(1, 16, 8, 1, 2, 256, 0, 1, 128)        \
    X(2, 32, 8, 1, 2, 256, 0, 1, 256)        \
    X(3, 64, 8, 1, 2, 256, 0, 1, 512)        \
    X(4, 128, 8, 1, 1, 256, 0, 1, 1024)      \
    X(5, 256, 8, 1, 1, 256, 0, 1, 2048)      \
    X(6, 256, 8, 2, 2, 256, 0, 1, 4096)      \
    X(7, 1024, 8, 1, 1, 1024, 0, 1, 8192)
#define MN_FWD_ADD(X) MN_FWD_RMS(X)
#define MN_FWD_GEN(X)                        \
    X(8, 64, 1, 16, 1, 256, 0, 1, 1024)      \
    X(9, 256, 1, 16, 1, 256, 0, 1, 4096)     \
    X(10, 512, 1, 16, 1, 512, 0, 1, 8192)

#define MN_BWD_RMS(X)                        \
    X(0, 8, 8, 1, 4, 256, 1, 3, 64)          \
    X(1, 16, 8, 1, 4, 256, 1, 3, 128)        \
    X(2, 32, 8, 1, 4, 256, 1, 3, 256)        \
    X(3, 64, 8, 1, 2, 256, 1, 3, 512)        \
    X(4, 128, 8, 1, 2, 512, 1, 3, 1024)      \
    X(5, 256, 8, 1, 2, 512, 1, 3, 2048)      \
    X(6, 512, 8, 1, 2, 512, 1, 3, 4096)      \
    X(7, 1024, 8, 1, 1, 1024, 1, 3, 8192)
#define MN_BWD_LN(X)                         \
    X(0, 8, 8, 1, 4, 256, 1, 3, 64)          \
    X(1, 16, 8, 1, 4, 256, 1, 3, 128)        \
    X(2, 32, 8, 1, 4, 256, 1, 3, 256)        \
    X(3, 64, 8, 1, 2, 256, 1, 3, 512)        \
    X(4, 64, 8, 2, 2, 256, 1, 3, 1024)       \
    X(5, 128, 8, 2, 2, 512, 1, 3, 2048)      \
    X(6, 256, 8, 2, 2, 512, 1, 3, 4096)      \
    X(7, 512, 8, 2, 1, 512, 1, 3, 8192)
#define MN_BWD_ADD(X) MN_BWD_RMS(X)
#define MN_BWD_GEN(X)                        \
    X(8, 64, 1, 16, 1, 256, 1, 1, 1024)      \
    X(9, 256, 1, 16, 1, 256, 1, 1, 4096)     \
    X(10, 512, 1, 16, 1, 512, 1, 1, 8192)

struct VariantRow {
    Variant v;
    int max_d;
};

#define MN_ROW(id, T, VEC, CPT, U, BLOCK, PF, NT, MAXD) {{id, T, VEC, CPT, U, BLOCK}, MAXD},
const VariantRow kFwdVec[3][8] = {{MN_FWD_RMS(MN_ROW)}, {MN_FWD_LN(MN_ROW)}, {MN_FWD_ADD(MN_ROW)}};
const VariantRow kBwdVec[3][8] = {{MN_BWD_RMS(MN_ROW)}, {MN_BWD_LN(MN_ROW)}, {MN_BWD_ADD(MN_ROW)}};
const VariantRow kFwdGen[] = {MN_FWD_GEN(MN_ROW)};
const VariantRow kBwdGen[] = {MN_BWD_GEN(MN_ROW)};
#undef MN_ROW

template <size_t K>
Variant pick(const VariantRow (&t)[K], int32_t D)
{
    for (size_t i = 0; i < K; ++i)
        if (D <= t[i].max_d) return t[i].v;
    return t[K - 1].v;
}

template <typename Kernel, typename Args>
hipError_t launch(Kernel k, dim3 grid, dim3 block, size_t shmem, hipStream_t s, const Args& a)
{
    void* args[] = {const_cast<Args*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, shmem, s);
}

// binary32 storage keeps 16-byte chunks: 4 elements per chunk and twice the
// chunks per lane of the 16-bit shapes, so the row coverage T*CPT*VEC and
// the bytes in flight per lane are unchanged.
constexpr int st_vec(int st, int vec) { return (st == ST_F32 && vec == 8) ? 4 : vec; }
constexpr int st_cpt(int st, int vec, int cpt) { return (st == ST_F32 && vec == 8) ? 2 * cpt : cpt; }

#define MN_FWD_CASE(id, T, VEC, CPT, U, BLOCK, PF, NT, MAXD)                                  \
    case id:                                                                                  \
        return launch(fwd_kernel<KIND, ST, T, st_vec(ST, VEC), st_cpt(ST, VEC, CPT), U, BLOCK, \
                                 PF, NT>,                                                     \
                      grid, dim3(BLOCK), 0, s, a);
#define MN_BWD_CASE(id, T, VEC, CPT, U, BLOCK, PF, NT, MAXD)                                  \
    case id:                                                                                  \
        return launch(bwd_kernel<KIND, ST, T, st_vec(ST, VEC), st_cpt(ST, VEC, CPT), U, BLOCK, \
                                 PF, NT>,                                                     \
                      grid, dim3(BLOCK), p.shmem, s, a);

template <int KIND, int ST>
hipError_t launch_fwd(const FwdPlan& p, const FwdArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)p.grid);
    if constexpr (KIND == RMS) {
        switch (p.v.id) { MN_FWD_RMS(MN_FWD_CASE) MN_FWD_GEN(MN_FWD_CASE) }
    } else if constexpr (KIND == LN) {
        switch (p.v.id) { MN_FWD_LN(MN_FWD_CASE) MN_FWD_GEN(MN_FWD_CASE) }
    } else {
        switch (p.v.id) { MN_FWD_ADD(MN_FWD_CASE) MN_FWD_GEN(MN_FWD_CASE) }
    }
    return hipErrorInvalidValue;
}

template <int KIND, int ST>
hipError_t launch_bwd(const BwdPlan& p, const BwdArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)p.P);
    if constexpr (KIND == RMS) {
        switch (p.v.id) { MN_BWD_RMS(MN_BWD_CASE) MN_BWD_GEN(MN_BWD_CASE) }
    } else if constexpr (KIND == LN) {
        switch (p.v.id) { MN_BWD_LN(MN_BWD_CASE) MN_BWD_GEN(MN_BWD_CASE) }
    } else {
        switch (p.v.id) { MN_BWD_ADD(MN_BWD_CASE) MN_BWD_GEN(MN_BWD_CASE) }
    }
    return hipErrorInvalidValue;
}

#undef MN_FWD_CASE
#undef MN_BWD_CASE

template <int KIND>
hipError_t launch_fwd_st(int st, const FwdPlan& p, const FwdArgs& a, hipStream_t s)
{
    switch (st) {
    case ST_F16: return launch_fwd<KIND, ST_F16>(p, a, s);
    case ST_BF16: return launch_fwd<KIND, ST_BF16>(p, a, s);
    case ST_F32: return launch_fwd<KIND, ST_F32>(p, a, s);
    }
    return hipErrorInvalidValue;
}

template <int KIND>
hipError_t launch_bwd_st(int st, const BwdPlan& p, const BwdArgs& a, hipStream_t s)
{
    switch (st) {
    case ST_F16: return launch_bwd<KIND, ST_F16>(p, a, s);
    case ST_BF16: return launch_bwd<KIND, ST_BF16>(p, a, s);
    case ST_F32: return launch_bwd<KIND, ST_F32>(p, a, s);
    }
    return hipErrorInvalidValue;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups (= partial rows) of the backward: one long-lived workgroup per
// CU of the 256, never more than there are rows.
int64_t bwd_blocks(int kind, int32_t D)
{
    (void)kind;
    (void)D;
    return 256;
}

}  // namespace

int32_t partial_stride(int32_t D) { return (D + 3) & ~3; }

int64_t bwd_partial_rows(int kind, int64_t N, int32_t D)
{
    return N < bwd_blocks(kind, D) ? N : bwd_blocks(kind, D);
}

FwdPlan plan_forward(int kind, int st, int64_t N, int32_t D, bool vec_ok)
{
    (void)st;
    FwdPlan p;
    p.v = vec_ok ? pick(kFwdVec[kind], D) : pick(kFwdGen, D);
    // one tile of RPB*U rows per workgroup
    p.grid = ceil_div(N, (int64_t)(p.v.BLOCK / p.v.T) * p.v.U);
    return p;
}

BwdPlan plan_backward(int kind, int st, int64_t N, int32_t D, bool vec_ok)
{
    (void)st;
    BwdPlan p;
    p.v = vec_ok ? pick(kBwdVec[kind], D) : pick(kBwdGen, D);
    p.P = bwd_partial_rows(kind, N, D);
    p.Dp = partial_stride(D);
    const int rpb = p.v.BLOCK / p.v.T;
    p.shmem = (rpb > 1) ? (size_t)D * sizeof(float) * (kind == LN ? 2 : 1) : 0;
    return p;
}

hipError_t launch_forward(int kind, int st, const FwdPlan& p, const FwdArgs& a, hipStream_t s)
{
    switch (kind) {
    case RMS: return launch_fwd_st<RMS>(st, p, a, s);
    case LN: return launch_fwd_st<LN>(st, p, a, s);
    case ADD: return launch_fwd_st<ADD>(st, p, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_backward_rows(int kind, int st, const BwdPlan& p, const BwdArgs& a,
                                hipStream_t s)
{
    switch (kind) {
    case RMS: return launch_bwd_st<RMS>(st, p, a, s);
    case LN: return launch_bwd_st<LN>(st, p, a, s);
    case ADD: return launch_bwd_st<ADD>(st, p, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)ceil_div(a.Dp, 4 * kReduceCQ), a.part_b ? 2u : 1u);
    return launch(reduce_kernel<kReduceCQ>, grid, dim3(1024), 0, s, a);
}

}  // namespace mn
