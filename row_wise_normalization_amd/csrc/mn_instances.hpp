// mn_instances.hpp -- definitions of the kernel launchers, included by
// mn_inst_f16.hip, mn_inst_bf16.hip and mn_inst_f32.hip, each of which sets
// MN_INST_ST (its activation storage type) and MN_INST_BWD_TYPES (the
// backward storage combinations for it). Splitting the instances by storage
// type lets the build compile them in parallel.
#pragma once

#include "mn_kernels.hpp"
#include "mn_tables.hpp"

namespace mn {
namespace {

using kern::bwd_kernel;
using kern::fwd_kernel;

template <typename Kernel, typename Args>
hipError_t launch(Kernel k, dim3 grid, dim3 block, size_t shmem, hipStream_t s, const Args& a)
{
    void* args[] = {const_cast<Args*>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, shmem, s);
}


#define MN_FWD_CASE(id, T, VEC, CPT, U, BLOCK, PF, NT, MAXD)                                  \
    case id:                                                                                  \
        return launch(fwd_kernel<KIND, ST, T, st_vec(ST, VEC), st_cpt(ST, VEC, CPT), U, BLOCK, \
                                 PF, NT>,                                                     \
                      grid, dim3(BLOCK), 0, s, a);
#define MN_BWD_CASE(id, T, VEC, CPT, U, BLOCK, PF, NT, MAXD)                           \
    case id:                                                                           \
        return launch(bwd_kernel<KIND, ST, CT, OT, T, st_vec(ST, VEC), st_cpt(ST, VEC, CPT), \
                                 U, BLOCK, PF, NT>,                                    \
                      grid, dim3(BLOCK), p.shmem, s, a);

}  // namespace

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

template <int KIND, int ST, int CT, int OT>
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

template hipError_t launch_fwd<RMS, MN_INST_ST>(const FwdPlan&, const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<LN, MN_INST_ST>(const FwdPlan&, const FwdArgs&, hipStream_t);
template hipError_t launch_fwd<ADD, MN_INST_ST>(const FwdPlan&, const FwdArgs&, hipStream_t);

#define MN_INST_BWD(S, C, O)                                                                  \
    template hipError_t launch_bwd<RMS, S, C, O>(const BwdPlan&, const BwdArgs&, hipStream_t); \
    template hipError_t launch_bwd<LN, S, C, O>(const BwdPlan&, const BwdArgs&, hipStream_t);  \
    template hipError_t launch_bwd<ADD, S, C, O>(const BwdPlan&, const BwdArgs&, hipStream_t);
MN_INST_BWD_TYPES(MN_INST_BWD)
#undef MN_INST_BWD

}  // namespace mn
