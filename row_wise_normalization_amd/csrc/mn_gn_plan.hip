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

bool plan_groupnorm(int st, int64_t N, int64_t C, int64_t L, int64_t G, bool vec_ok, bool fwd,
                    GnPlan& p)
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
    if (p.grid > INT32_MAX) return false;
    if (!fwd) return true;
    // The forward (same shapes as the backward) holds fewer registers per
    // row: the fewest padding rows again, then lanes that fill their waves,
    // then the smallest workgroup. At 32 x 320 x 4096 (G = 32) one row group
    // of 256 lanes per 10 x 4096 slice (four slices per CU, all 1024 in one
    // round) ran 16 % ahead of two row groups of 512 lanes (three per CU).
    int fb = -1;
    int64_t fb_waste = 0, fb_block = 0, fb_lanes = 0;
    for (int U = 1; U <= kGnFwdMaxU; ++U) {
        if (!gn_fits_fwd(st, vec, sh->T, sh->CPT, U)) break;
        const int64_t rpb = (Cg + U - 1) / U;
        const int64_t lanes = rpb * sh->T;
        const int64_t block = (lanes + 63) / 64 * 64;
        if (block > 1024) continue;
        const int64_t waste = rpb * U - Cg;
        // busy lanes per 64: a shortfall below one wave counts against
        const bool fuller = lanes * fb_block > fb_lanes * block;
        const bool same_fill = lanes * fb_block == fb_lanes * block;
        const bool better = fb < 0 || waste < fb_waste ||
                            (waste == fb_waste && (fuller || (same_fill && block < fb_block)));
        if (better) {
            fb = U;
            fb_waste = waste;
            fb_block = block;
            fb_lanes = lanes;
        }
    }
    p.id = sh->id * kGnFwdMaxU + fb - 1;
    p.block = (int32_t)fb_block;
    return true;
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
