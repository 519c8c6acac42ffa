// mn_gn_instances.hpp -- GroupNorm launchers, included by mn_gn_{f16,bf16,f32}.hip,
// each of which instantiates them for its activation storage type.
#pragma once

#include "mn_groupnorm.hpp"
#include "mn_tables.hpp"

namespace mn {
namespace {

template <typename Kernel>
hipError_t gn_launch(Kernel k, const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    void* args[] = {const_cast<GnArgs*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((unsigned)p.grid),
                           dim3((unsigned)p.block), args, 0, s);
}

// The backward stages its first dY chunks in LDS, at most kGnStageBytes per
// workgroup (16-byte chunks only; `chunks` per lane in this instance). At
// 32 x 320 x 4096 (G = 32), 32 KB (four of a lane's ten chunks) took the
// backward from 55.5 to 51.2 us; larger stages gained little more.
constexpr int64_t kGnStageBytes = 32 * 1024;

template <typename Kernel>
hipError_t gn_launch_bwd(Kernel k, const GnPlan& p, GnArgs a, hipStream_t s, int chunks,
                         bool stage)
{
    const int64_t fit = kGnStageBytes / (16 * (int64_t)p.block);
    a.sk = stage ? (int32_t)(fit < chunks ? fit : chunks) : 0;
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((unsigned)p.grid),
                           dim3((unsigned)p.block), args, (size_t)a.sk * 16 * p.block, s);
}

}  // namespace

// only the shapes within the register budget are instantiated
#define MN_GN_FWD_U(SH, T, VEC, CPT, UL, U)                                                  \
    case SH * kGnFwdMaxU + UL:                                                               \
        if constexpr (gn_fits_fwd(ST, VEC, T, CPT, U))                                          \
            return gn_launch(                                                                \
                kern::gn_fwd_kernel<ST, T, st_vec(ST, VEC), st_cpt(ST, VEC, CPT), U>, p, a, s); \
        else                                                                                 \
            return hipErrorInvalidValue;
#define MN_GN_BWD_U(SH, T, VEC, CPT, UL, U)                                                  \
    case SH * 8 + UL:                                                                        \
        if constexpr (gn_fits(ST, VEC, T, CPT, U))                                              \
            return gn_launch_bwd(                                                            \
                kern::gn_bwd_kernel<ST, OT, T, st_vec(ST, VEC), st_cpt(ST, VEC, CPT), U>, p, a, \
                s, U * st_cpt(ST, VEC, CPT), VEC == 8);                                      \
        else                                                                                 \
            return hipErrorInvalidValue;
#define MN_GN_US(M, SH, T, VEC, CPT)                                                      \
    M(SH, T, VEC, CPT, 0, 1) M(SH, T, VEC, CPT, 1, 2) M(SH, T, VEC, CPT, 2, 3)            \
    M(SH, T, VEC, CPT, 3, 4) M(SH, T, VEC, CPT, 4, 5) M(SH, T, VEC, CPT, 5, 6)            \
    M(SH, T, VEC, CPT, 6, 7) M(SH, T, VEC, CPT, 7, 8)
#define MN_GN_US16(M, SH, T, VEC, CPT)                                                    \
    MN_GN_US(M, SH, T, VEC, CPT)                                                          \
    M(SH, T, VEC, CPT, 8, 9) M(SH, T, VEC, CPT, 9, 10) M(SH, T, VEC, CPT, 10, 11)         \
    M(SH, T, VEC, CPT, 11, 12) M(SH, T, VEC, CPT, 12, 13) M(SH, T, VEC, CPT, 13, 14)      \
    M(SH, T, VEC, CPT, 14, 15) M(SH, T, VEC, CPT, 15, 16)
#define MN_GN_FWD_VEC(SH, T, CPT, MAXL) MN_GN_US16(MN_GN_FWD_U, SH, T, 8, CPT)
#define MN_GN_FWD_ELEM(SH, T, CPT, MAXL) MN_GN_US16(MN_GN_FWD_U, SH, T, 1, CPT)
#define MN_GN_BWD_VEC(SH, T, CPT, MAXL) MN_GN_US(MN_GN_BWD_U, SH, T, 8, CPT)
#define MN_GN_BWD_ELEM(SH, T, CPT, MAXL) MN_GN_US(MN_GN_BWD_U, SH, T, 1, CPT)

template <int ST>
hipError_t launch_gn_fwd_t(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    switch (p.id) { MN_GN_VEC_SHAPES(MN_GN_FWD_VEC) MN_GN_ELEM_SHAPES(MN_GN_FWD_ELEM) }
    return hipErrorInvalidValue;
}

template <int ST, int OT>
hipError_t launch_gn_bwd_t(const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    switch (p.id) { MN_GN_VEC_SHAPES(MN_GN_BWD_VEC) MN_GN_ELEM_SHAPES(MN_GN_BWD_ELEM) }
    return hipErrorInvalidValue;
}

#undef MN_GN_FWD_U
#undef MN_GN_BWD_U
#undef MN_GN_US
#undef MN_GN_US16
#undef MN_GN_FWD_VEC
#undef MN_GN_FWD_ELEM
#undef MN_GN_BWD_VEC
#undef MN_GN_BWD_ELEM

}  // namespace mn
