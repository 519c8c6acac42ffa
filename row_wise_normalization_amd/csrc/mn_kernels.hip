// mn_kernels.hip -- planning and dispatch of the gfx950 normalization
// kernels: picks the launch-table row for a call (tables in mn_tables.hpp),
// sizes its grid, and dispatches to the instance for its storage types
// (instantiated in mn_inst_*.hip); also launches the stage-2 reduce.
#include <algorithm>

#include "mn_kernels.hpp"
#include "mn_tables.hpp"

namespace mn {
namespace {

using kern::reduce_kernel;

constexpr int kReduceCQ = 16;  // 64 columns per block, 64 segments
// the one-launch backward adds its partial rows in this kernel's order,
// which for at most 64 rows is one row per segment
static_assert(1024 / kReduceCQ == kSmallMaxP, "one-launch reduce order");

struct VariantRow {
    Variant v;
    int max_d;
};

#define MN_ROW(id, T, VEC, CPT, U, BLOCK, PF, NT, MAXD) {{id, T, VEC, CPT, U, BLOCK}, MAXD},
const VariantRow kFwdVec[6][11] = {{MN_FWD_RMS(MN_ROW)}, {MN_FWD_LN(MN_ROW)}, {MN_FWD_ADD(MN_ROW)},
                                  {MN_FWD_DYT(MN_ROW)}, {MN_FWD_POLY(MN_ROW)}, {MN_FWD_MOD(MN_ROW)}};
const VariantRow kBwdVec[6][10] = {{MN_BWD_RMS(MN_ROW)}, {MN_BWD_LN(MN_ROW)}, {MN_BWD_ADD(MN_ROW)},
                                  {MN_BWD_DYT(MN_ROW)}, {MN_BWD_POLY(MN_ROW)}, {MN_BWD_MOD(MN_ROW)}};
const VariantRow kFwdGen[] = {MN_FWD_GEN(MN_ROW)};
const VariantRow kBwdGen[] = {MN_BWD_GEN(MN_ROW)};
#undef MN_ROW

template <size_t K>
Variant pick(const VariantRow (&t)[K], int32_t D)
{
    // tables shorter than the array end in zero rows (max_d 0), never picked
    for (size_t i = 0; i < K; ++i)
        if (D <= t[i].max_d) return t[i].v;
    return t[0].v;
}

template <typename Kernel, typename Args>
hipError_t launch(Kernel k, dim3 grid, dim3 block, size_t shmem, hipStream_t s, const Args& a)
{
    void* args[] = {const_cast<Args*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, shmem, s);
}


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
hipError_t launch_bwd_types(int st, int ct, int ot, const BwdPlan& p, const BwdArgs& a,
                            hipStream_t s)
{
#define MN_BWD_TYPE_CASE(S, C, O) \
    if (st == S && ct == C && ot == O) return launch_bwd<KIND, S, C, O>(p, a, s);
    if constexpr (KIND == RMS || KIND == LN || KIND == ADD) {
        MN_BWD_TYPES(MN_BWD_TYPE_CASE)
    } else {
        MN_BWD_TYPES_EXT(MN_BWD_TYPE_CASE)
    }
#undef MN_BWD_TYPE_CASE
    return hipErrorInvalidValue;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups (= partial rows) of the backward, never more than there are
// rows: one long-lived workgroup per CU of the 256, or two for RMSNorm rows
// of up to 3072 columns and PolyNorm rows of up to 4096 (5 % faster for
// PolyNorm at 16384 x 4096; LayerNorm, Dynamic Tanh and the fused add at
// 8192 columns were slower or unchanged with two). At 4096 columns RMSNorm
// takes one workgroup per CU with three rows per step: timed as whole steps
// (forward, backward, column reduce on rotating buffers), 0.7 % faster than
// two workgroups of two rows, with half the partial rows to reduce.
int64_t bwd_blocks(int kind, int32_t D)
{
    if (kind == RMS) return D <= 3072 ? 512 : 256;
    return (kind == POLY && D <= 4096) ? 512 : 256;
}

}  // namespace

int32_t partial_stride(int32_t D) { return (D + 3) & ~3; }

bool bwd_small(int kind, int64_t N, int32_t D)
{
    return (kind == RMS || kind == LN || kind == ADD) &&
           N * (int64_t)partial_stride(D) <= kSmallPartialFloats * 8;
}

bool bwd_one_launch(int kind, int64_t N, int32_t D)
{
    return bwd_small(kind, N, D) && D <= kSmallMaxD;
}

// every row variant that serves widths up to kSmallMaxD has fewer than 1024
// lanes (the one-launch reduce is compiled into those only)
#define MN_SMALL_OK(id, T, VEC, CPT, U, BLOCK, PF, NT, MAXD) \
    static_assert(MAXD > kSmallMaxD || BLOCK < 1024, "one-launch row variant");
MN_BWD_RMS(MN_SMALL_OK)
MN_BWD_LN(MN_SMALL_OK)
MN_BWD_ADD(MN_SMALL_OK)
MN_BWD_GEN(MN_SMALL_OK)
#undef MN_SMALL_OK

int64_t bwd_partial_rows(int kind, int64_t N, int32_t D)
{
    // Small problems: about eight rows per workgroup, rounded up to a power
    // of two (the one-launch reduce then needs no masking of absent rows;
    // workgroups past the last tile write zero rows, as they do whenever
    // there are fewer tiles than workgroups), at most 64 workgroups.
    if (bwd_small(kind, N, D)) {
        const int64_t k = (N + 7) / 8;
        int64_t p = 1;
        while (p < k && p < kSmallMaxP) p *= 2;
        return p;
    }
    return N < bwd_blocks(kind, D) ? N : bwd_blocks(kind, D);
}

int32_t mod_blocks_per_sample(int64_t B, int64_t N)
{
    // 256 workgroups shared out over the samples (at least one each), never
    // more per sample than it has rows
    const int64_t S = N / B;
    int64_t pb = B >= 256 ? 1 : 256 / B;
    if (pb > S) pb = S;
    return (int32_t)(pb < 1 ? 1 : pb);
}

int bwd_vector_partials(int kind)
{
    switch (kind) {
    case LN:
    case DYT: return 2;
    case MOD: return 3;
    case POLY: return 0;
    default: return 1;
    }
}

FwdPlan plan_forward(int kind, int st, int pdt, int64_t N, int32_t D, bool vec_ok, int64_t B)
{
    FwdPlan p;
    p.v = vec_ok ? pick(kFwdVec[kind], D) : pick(kFwdGen, D);
    // 16-bit activations with binary32 parameters: twice the rows per
    // workgroup at 4096 columns (row 15 of the RMSNorm and LayerNorm tables)
    if ((kind == RMS || kind == LN) && vec_ok && p.v.id == 6 && st != ST_F32 && pdt == ST_F32)
        for (const VariantRow& r : kFwdVec[kind])
            if (r.v.id == 15) p.v = r.v;
    // one tile of RPB*U rows per workgroup; MOD: whole tiles per sample (B
    // samples of N / B rows)
    const int64_t tile = (int64_t)(p.v.BLOCK / p.v.T) * p.v.U;
    p.grid = (kind == MOD) ? B * ceil_div(N / B, tile) : ceil_div(N, tile);
    return p;
}

BwdPlan plan_backward(int kind, int st, int64_t N, int32_t D, bool vec_ok, int64_t B)
{
    (void)st;
    BwdPlan p;
    p.v = vec_ok ? pick(kBwdVec[kind], D) : pick(kBwdGen, D);
    p.Pb = (kind == MOD) ? mod_blocks_per_sample(B, N) : 0;
    p.P = (kind == MOD) ? B * p.Pb : bwd_partial_rows(kind, N, D);
    p.Dp = partial_stride(D);
    const int rpb = p.v.BLOCK / p.v.T;
    p.shmem = (rpb > 1) ? (size_t)D * sizeof(float) * bwd_vector_partials(kind) : 0;
    return p;
}

hipError_t launch_forward(int kind, int st, const FwdPlan& p, const FwdArgs& a, hipStream_t s)
{
    switch (kind) {
    case RMS: return launch_fwd_st<RMS>(st, p, a, s);
    case LN: return launch_fwd_st<LN>(st, p, a, s);
    case ADD: return launch_fwd_st<ADD>(st, p, a, s);
    case DYT: return launch_fwd_st<DYT>(st, p, a, s);
    case POLY: return launch_fwd_st<POLY>(st, p, a, s);
    case MOD: return launch_fwd_st<MOD>(st, p, a, s);
    }
    return hipErrorInvalidValue;
}

bool backward_types_supported(int kind, int st, int ct, int ot)
{
#define MN_BWD_TYPE_OK(S, C, O) \
    if (st == S && ct == C && ot == O) return true;
    if (kind == RMS || kind == LN || kind == ADD) {
        MN_BWD_TYPES(MN_BWD_TYPE_OK)
    } else {
        MN_BWD_TYPES_EXT(MN_BWD_TYPE_OK)
    }
#undef MN_BWD_TYPE_OK
    return false;
}

hipError_t launch_backward_rows(int kind, int st, int ct, int ot, const BwdPlan& p,
                                const BwdArgs& a, hipStream_t s)
{
    switch (kind) {
    case RMS: return launch_bwd_types<RMS>(st, ct, ot, p, a, s);
    case LN: return launch_bwd_types<LN>(st, ct, ot, p, a, s);
    case ADD: return launch_bwd_types<ADD>(st, ct, ot, p, a, s);
    case DYT: return launch_bwd_types<DYT>(st, ct, ot, p, a, s);
    case POLY: return launch_bwd_types<POLY>(st, ct, ot, p, a, s);
    case MOD: return launch_bwd_types<MOD>(st, ct, ot, p, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s)
{
    if (a.planes < 1 || a.planes > kReduceMaxPlanes) return hipErrorInvalidValue;
    int64_t gx = 1, gz = 1;
    for (int y = 0; y < a.planes; ++y) {
        const ReducePlane& pl = a.plane[y];
        if (pl.Dp % 4 != 0 || pl.D > pl.Dp || pl.P < 1 || pl.groups < 1) return hipErrorInvalidValue;
        gx = std::max(gx, ceil_div(pl.Dp, 4 * kReduceCQ));
        gz = std::max(gz, (int64_t)pl.groups);
    }
    const dim3 grid((unsigned)gx, (unsigned)a.planes, (unsigned)gz);
    return launch(reduce_kernel<kReduceCQ>, grid, dim3(1024), 0, s, a);
}

}  // namespace mn
