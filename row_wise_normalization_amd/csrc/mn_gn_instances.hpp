// mn_gn_instances.hpp -- GroupNorm launchers, included by
// mn_gn_{fwd,bwd}_{f16,bf16,f32}.hip, each of which instantiates one
// direction for one activation storage type (the instances compile in
// parallel). The register-path kernels are instantiated for 4-byte and for
// 2-byte gamma / beta (PW).
#pragma once

#include "mn_groupnorm.hpp"
#include "mn_tables.hpp"

namespace mn {
namespace {

template <typename Kernel>
hipError_t gn_launch(Kernel k, int64_t grid, int block, const GnArgs& a, hipStream_t s)
{
    void* args[] = {const_cast<GnArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((unsigned)grid),
                           dim3((unsigned)block), args, 0, s);
}

// Split path row-unit kernels by lanes per unit (8 << tid).
template <int ST, int VEC, template <int, int, int> class K>
hipError_t gn_unit_launch(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    const int T = 8 << p.tid;
    const int64_t grid = (p.units + kern::kGnUnitBlock / T - 1) / (kern::kGnUnitBlock / T);
    switch (p.tid) {
    case 0: return gn_launch(K<ST, 8, VEC>::fn(), grid, kern::kGnUnitBlock, a, s);
    case 1: return gn_launch(K<ST, 16, VEC>::fn(), grid, kern::kGnUnitBlock, a, s);
    case 2: return gn_launch(K<ST, 32, VEC>::fn(), grid, kern::kGnUnitBlock, a, s);
    case 3: return gn_launch(K<ST, 64, VEC>::fn(), grid, kern::kGnUnitBlock, a, s);
    case 4: return gn_launch(K<ST, 128, VEC>::fn(), grid, kern::kGnUnitBlock, a, s);
    case 5: return gn_launch(K<ST, 256, VEC>::fn(), grid, kern::kGnUnitBlock, a, s);
    }
    return hipErrorInvalidValue;
}

template <int ST, int T, int VEC>
struct UnitSums {
    static auto fn() { return kern::gn_unit_sums_kernel<ST, T, VEC>; }
};
template <int ST, int T, int VEC>
struct UnitY {
    static auto fn() { return kern::gn_unit_y_kernel<ST, T, VEC>; }
};
template <int OT>
struct UnitDx {
    template <int ST, int T, int VEC>
    struct K {
        static auto fn() { return kern::gn_unit_dx_kernel<ST, OT, T, VEC>; }
    };
};

template <int ST, int VEC>
hipError_t gn_split_fwd(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    hipError_t e = gn_launch(kern::gn_chunk_stats_kernel<ST, VEC>, a.S * a.Kf,
                             kern::kGnUnitBlock, a, s);
    if (e == hipSuccess) e = gn_launch(kern::gn_stats_merge_kernel<ST>, a.S, kern::kGnUnitBlock, a, s);
    if (e == hipSuccess) e = gn_unit_launch<ST, VEC, UnitY>(p, a, s);
    return e;
}

template <int ST, int OT, int VEC>
hipError_t gn_split_bwd(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    hipError_t e = gn_unit_launch<ST, VEC, UnitSums>(p, a, s);
    if (e == hipSuccess) e = gn_launch(kern::gn_unit_merge_kernel<ST>, a.S, kern::kGnUnitBlock, a, s);
    if (e == hipSuccess) e = gn_unit_launch<ST, VEC, UnitDx<OT>::template K>(p, a, s);
    return e;
}

}  // namespace

// only the shapes within the register budget are instantiated
#define MN_GN_FWD_U(SH, T, VEC, CPT, PF, U)                                                   \
    case gn_id(true, SH, PF, U):                                                               \
        if constexpr (gn_fits(true, ST, ST, VEC, T, CPT, U, PF, PW))                                   \
            return gn_launch(                                                                  \
                kern::gn_fwd_kernel<ST, T, st_vec(ST, VEC), st_cpt(ST, VEC, CPT), U, PF, PW>,  \
                p.grid, p.block, a, s);                                                        \
        else                                                                                   \
            return hipErrorInvalidValue;
#define MN_GN_BWD_U(SH, T, VEC, CPT, PF, U)                                                   \
    case gn_id(false, SH, PF, U):                                                              \
        if constexpr (gn_fits(false, ST, OT, VEC, T, CPT, U, PF, PW))                                  \
            return gn_launch(                                                                  \
                kern::gn_bwd_kernel<ST, OT, T, st_vec(ST, VEC), st_cpt(ST, VEC, CPT), U, PF, PW>, \
                p.grid, p.block, a, s);                                                        \
        else                                                                                   \
            return hipErrorInvalidValue;
#define MN_GN_US8(M, SH, T, VEC, CPT, PF)                                                     \
    M(SH, T, VEC, CPT, PF, 1) M(SH, T, VEC, CPT, PF, 2) M(SH, T, VEC, CPT, PF, 3)             \
    M(SH, T, VEC, CPT, PF, 4) M(SH, T, VEC, CPT, PF, 5) M(SH, T, VEC, CPT, PF, 6)             \
    M(SH, T, VEC, CPT, PF, 7) M(SH, T, VEC, CPT, PF, 8)
#define MN_GN_US16(M, SH, T, VEC, CPT, PF)                                                    \
    MN_GN_US8(M, SH, T, VEC, CPT, PF)                                                         \
    M(SH, T, VEC, CPT, PF, 9) M(SH, T, VEC, CPT, PF, 10) M(SH, T, VEC, CPT, PF, 11)           \
    M(SH, T, VEC, CPT, PF, 12) M(SH, T, VEC, CPT, PF, 13) M(SH, T, VEC, CPT, PF, 14)          \
    M(SH, T, VEC, CPT, PF, 15) M(SH, T, VEC, CPT, PF, 16)
#define MN_GN_FWD_VEC(SH, T, CPT, MAXL) \
    MN_GN_US16(MN_GN_FWD_U, SH, T, 8, CPT, 0) MN_GN_US16(MN_GN_FWD_U, SH, T, 8, CPT, 1)
#define MN_GN_FWD_ELEM(SH, T, CPT, MAXL) \
    MN_GN_US16(MN_GN_FWD_U, SH, T, 1, CPT, 0) MN_GN_US16(MN_GN_FWD_U, SH, T, 1, CPT, 1)
#define MN_GN_BWD_VEC(SH, T, CPT, MAXL) \
    MN_GN_US8(MN_GN_BWD_U, SH, T, 8, CPT, 0) MN_GN_US8(MN_GN_BWD_U, SH, T, 8, CPT, 1)
#define MN_GN_BWD_ELEM(SH, T, CPT, MAXL) \
    MN_GN_US8(MN_GN_BWD_U, SH, T, 1, CPT, 0) MN_GN_US8(MN_GN_BWD_U, SH, T, 1, CPT, 1)

template <int ST, int PW>
hipError_t launch_gn_fwd_pw(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    switch (p.id) { MN_GN_VEC_SHAPES(MN_GN_FWD_VEC) MN_GN_ELEM_SHAPES(MN_GN_FWD_ELEM) }
    return hipErrorInvalidValue;
}

template <int ST, int OT, int PW>
hipError_t launch_gn_bwd_pw(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    switch (p.id) { MN_GN_VEC_SHAPES(MN_GN_BWD_VEC) MN_GN_ELEM_SHAPES(MN_GN_BWD_ELEM) }
    return hipErrorInvalidValue;
}

template <int ST>
hipError_t launch_gn_fwd_t(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    if (p.split)
        return p.id ? gn_split_fwd<ST, st_vec(ST, 8)>(p, a, s) : gn_split_fwd<ST, 1>(p, a, s);
    return a.pdt == ST_F32 ? launch_gn_fwd_pw<ST, 4>(p, a, s) : launch_gn_fwd_pw<ST, 2>(p, a, s);
}

template <int ST, int OT>
hipError_t launch_gn_bwd_t(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    if (p.split)
        return p.id ? gn_split_bwd<ST, OT, st_vec(ST, 8)>(p, a, s)
                    : gn_split_bwd<ST, OT, 1>(p, a, s);
    return a.pdt == ST_F32 ? launch_gn_bwd_pw<ST, OT, 4>(p, a, s)
                           : launch_gn_bwd_pw<ST, OT, 2>(p, a, s);
}

#undef MN_GN_FWD_U
#undef MN_GN_BWD_U
#undef MN_GN_US8
#undef MN_GN_US16
#undef MN_GN_FWD_VEC
#undef MN_GN_FWD_ELEM
#undef MN_GN_BWD_VEC
#undef MN_GN_BWD_ELEM

}  // namespace mn
