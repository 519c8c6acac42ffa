// mn_gn_plan.hip -- GroupNorm launch planning and dispatch by storage type.
#include "mn_groupnorm.hpp"

namespace mn {

namespace {

struct GnShape {
    int id, T, CPT, max_l;
};

#define MN_GN_ROW(SH, T, CPT, MAXL) {SH, T, CPT, MAXL},
constexpr GnShape kGnVec[] = {MN_GN_VEC_SHAPES(MN_GN_ROW)};
constexpr GnShape kGnElem[] = {MN_GN_ELEM_SHAPES(MN_GN_ROW)};
#undef MN_GN_ROW

}  // namespace

bool plan_groupnorm(int st, int64_t N, int64_t C, int64_t L, int64_t G, bool vec_ok, GnPlan& p)
{
    if (N < 1 || C < 1 || L < 1 || G < 1 || C % G != 0) return false;
    const int64_t Cg = C / G;
    const GnShape* tab = vec_ok ? kGnVec : kGnElem;
    const int n = vec_ok ? (int)(sizeof(kGnVec) / sizeof(kGnVec[0]))
                         : (int)(sizeof(kGnElem) / sizeof(kGnElem[0]));
    const GnShape* sh = nullptr;
    for (int i = 0; i < n && !sh; ++i)
        if (L <= tab[i].max_l) sh = &tab[i];
    if (!sh) return false;
    // rows per row group: the fewest padding rows (rpb * U - Cg), then
    // workgroups of at most 512 lanes (more of them per CU), then the
    // smallest U (fewest registers); timing sweeps at 32 x 320 x 4096 (G = 32)
    // put the exact fit U = 5 of 512 lanes 9 % ahead of U = 4 of 768 lanes
    const int vec = vec_ok ? 8 : 1;
    int best = -1;
    int64_t best_waste = 0, best_block = 0;
    for (int U = 1; U <= 8; ++U) {
        if (!gn_fits(st, vec, sh->T, sh->CPT, U)) break;
        const int64_t rpb = (Cg + U - 1) / U;
        const int64_t block = (rpb * sh->T + 63) / 64 * 64;
        if (block > 1024) continue;
        const int64_t waste = rpb * U - Cg;
        const bool better = best < 0 || waste < best_waste ||
                            (waste == best_waste && block <= 512 && best_block > 512);
        if (better) {
            best = U;
            best_waste = waste;
            best_block = block;
        }
    }
    if (best < 0) return false;
    p.id = sh->id * 8 + best - 1;
    p.block = (int32_t)best_block;
    p.grid = N * G;
    return p.grid <= INT32_MAX;
}

hipError_t launch_gn_fwd(int st, const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    switch (st) {
    case ST_F16: return launch_gn_fwd_t<ST_F16>(p, a, s);
    case ST_BF16: return launch_gn_fwd_t<ST_BF16>(p, a, s);
    case ST_F32: return launch_gn_fwd_t<ST_F32>(p, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gn_bwd(int st, int ot, const GnPlan& p, const GnArgs& a, hipStream_t s)
{
    if (st == ST_F16) return ot == ST_F32 ? launch_gn_bwd_t<ST_F16, ST_F32>(p, a, s)
                                          : launch_gn_bwd_t<ST_F16, ST_F16>(p, a, s);
    if (st == ST_BF16) return ot == ST_F32 ? launch_gn_bwd_t<ST_BF16, ST_F32>(p, a, s)
                                           : launch_gn_bwd_t<ST_BF16, ST_BF16>(p, a, s);
    if (st == ST_F32) return launch_gn_bwd_t<ST_F32, ST_F32>(p, a, s);
    return hipErrorInvalidValue;
}

}  // namespace mn
