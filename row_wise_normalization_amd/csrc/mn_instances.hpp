// mn_instances.hpp -- definitions of the kernel launchers, included by the
// mn_inst_*.hip files, each of which sets MN_INST_ST (its activation storage
// type), MN_INST_KINDS (the kinds it instantiates, as X(kind) entries) and
// MN_INST_BWD_TYPES (the backward storage combinations). Splitting the
// instances by storage type and kind group lets the build compile them in
// parallel.
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
    } else if constexpr (KIND == ADD) {
        switch (p.v.id) { MN_FWD_ADD(MN_FWD_CASE) MN_FWD_GEN(MN_FWD_CASE) }
    } else if constexpr (KIND == DYT) {
        switch (p.v.id) { MN_FWD_DYT(MN_FWD_CASE) MN_FWD_GEN(MN_FWD_CASE) }
    } else if constexpr (KIND == POLY) {
        switch (p.v.id) { MN_FWD_POLY(MN_FWD_CASE) MN_FWD_GEN(MN_FWD_CASE) }
    } else {
        switch (p.v.id) { MN_FWD_MOD(MN_FWD_CASE) MN_FWD_GEN(MN_FWD_CASE) }
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
    } else if constexpr (KIND == ADD) {
        switch (p.v.id) { MN_BWD_ADD(MN_BWD_CASE) MN_BWD_GEN(MN_BWD_CASE) }
    } else if constexpr (KIND == DYT) {
        switch (p.v.id) { MN_BWD_DYT(MN_BWD_CASE) MN_BWD_GEN(MN_BWD_CASE) }
    } else if constexpr (KIND == POLY) {
        switch (p.v.id) { MN_BWD_POLY(MN_BWD_CASE) MN_BWD_GEN(MN_BWD_CASE) }
    } else {
        switch (p.v.id) { MN_BWD_MOD(MN_BWD_CASE) MN_BWD_GEN(MN_BWD_CASE) }
    }
    return hipErrorInvalidValue;
}

#undef MN_FWD_CASE
#undef MN_BWD_CASE

#define MN_INST_FWD(K) \
    template hipError_t launch_fwd<K, MN_INST_ST>(const FwdPlan&, const FwdArgs&, hipStream_t);
MN_INST_KINDS(MN_INST_FWD)
#undef MN_INST_FWD

#define MN_INST_BWD_KIND(K, S, C, O) \
    template hipError_t launch_bwd<K, S, C, O>(const BwdPlan&, const BwdArgs&, hipStream_t);
#define MN_INST_BWD(S, C, O) MN_INST_KINDS_BWD(MN_INST_BWD_KIND, S, C, O)
MN_INST_BWD_TYPES(MN_INST_BWD)
#undef MN_INST_BWD
#undef MN_INST_BWD_KIND

}  // namespace mn
