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

// Compute units of the target: a persistent launch keeps up to 1024 lanes of
// workgroups per CU (the register budget of the shapes allows 4 waves per
// SIMD).
constexpr int64_t kGnCUs = 256;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Register path. Each CU holds 1024 lanes of these workgroups (4 waves per
// SIMD at up to 128 VGPRs), so what sets the pace is how much of the data
// each lane has in flight: the planner takes the shape, register sets and
// rows per row group with the most useful chunks in registers per lane --
// chunks per register set (X, and dY in the backward) times the sets (two
// with the next slice in flight, PF = 1) times the fraction of rows that
// are not padding (Cg / (rpb * U)) -- then PF = 1, then the smaller
// workgroup. At 32 x 320 x 4096 (G = 32) the forward holds a whole 10 x 4096
// slice in one 256-lane row group (20 chunks per lane, four slices per CU,
// all 1024 in one round: 16 % faster than two 512-lane row groups at three
// per CU, and faster than a 1024-lane workgroup with the next slice in
// flight, which has 10 chunks per lane in flight); the backward holds X and
// dY of one slice and of the next in a 1024-lane workgroup (two row groups
// of 512 lanes, five rows each). When there are no more slices than CUs,
// the workgroup with the most lanes per slice wins instead.
bool plan_registers(int st, int ot, int pw, int64_t Cg, int64_t L, int64_t S, bool vec_ok,
                    bool fwd, GnPlan& p)
{
    const GnShape* tab = vec_ok ? kGnVec : kGnElem;
    const int n = vec_ok ? (int)(sizeof(kGnVec) / sizeof(kGnVec[0]))
                         : (int)(sizeof(kGnElem) / sizeof(kGnElem[0]));
    const int vec = vec_ok ? 8 : 1;
    const int maxu = fwd ? kGnFwdMaxU : kGnBwdMaxU;
    const int tensors = fwd ? 1 : 2;
    const bool few = S <= kGnCUs;
    bool found = false, first = true;
    int bpf = 0, bid = 0;
    int64_t bblock = 0;
    double bscore = 0.0;
    for (int i = 0; i < n; ++i) {
        const GnShape& sh = tab[i];
        if (sh.max_l < L) continue;
        // the smallest shape that holds L, and any other that leaves at most
        // half of the lanes idle
        const bool cand = first || sh.max_l < 2 * L;
        first = false;
        if (!cand) continue;
        for (int pf = 1; pf >= 0; --pf) {
            for (int U = 1; U <= maxu; ++U) {
                if (!gn_fits(fwd, st, ot, vec, sh.T, sh.CPT, U, pf, pw)) break;
                const int64_t rpb = cdiv(Cg, U);
                const int64_t block = cdiv(rpb * sh.T, 64) * 64;
                if (block > kern::kGnMaxBlock) continue;
                const double useful = (double)Cg / (double)(rpb * U);
                const double score =
                    few ? (double)block * useful
                        : (double)(U * sh.CPT * tensors * (1 + pf)) * useful;
                const bool better = !found || score > bscore ||
                                    (score == bscore && (pf > bpf ||
                                                         (pf == bpf && block < bblock)));
                if (better) {
                    found = true;
                    bscore = score;
                    bpf = pf;
                    bid = gn_id(fwd, sh.id, pf, U);
                    bblock = block;
                }
            }
        }
    }
    if (!found) return false;
    p.split = false;
    p.id = bid;
    p.block = (int32_t)bblock;
    const int64_t resident = kGnCUs * (kern::kGnMaxBlock / bblock);
    p.grid = S < resident ? S : resident;
    return true;
}

}  // namespace

// Split-path geometry for 16-byte chunks (vec_ok) or single values: a row
// unit is up to IT chunks per lane of T lanes, T the smallest power of two
// from 8 to 256 that covers L in one unit (else 256 and several units per
// row); a statistics chunk is IT chunks per lane of a 256-lane workgroup.
static void split_geometry(int st, int64_t L, int64_t M, bool vec_ok, GnPlan& p)
{
    const int64_t vec = vec_ok ? (st == ST_F32 ? 4 : 8) : 1;
    const int64_t it = vec_ok ? kern::gn_unit_it<8>() : kern::gn_unit_it<1>();
    int tid = 0;
    while (tid < 5 && (int64_t)(8 << tid) * vec * it < L) ++tid;
    p.tid = tid;
    p.UL = (int32_t)((8 << tid) * vec * it);
    p.Kr = (int32_t)cdiv(L, p.UL);
    p.FL = (int32_t)(kern::kGnUnitBlock * vec * it);
    p.Kf = (int32_t)cdiv(M, p.FL);
}

int64_t gn_workspace_floats(int64_t N, int64_t C, int64_t L, int64_t G)
{
    // per-sample partials [N][Cp] twice, per-unit sums [N * C * Kr] twice
    // (Kr for the shortest units, 8192 values), slice sums [N * G][2]
    const int64_t Cp = (C + 3) / 4 * 4;
    const int64_t kr = cdiv(L, 8192);
    if (N > (INT64_MAX / 8) / (Cp + C * kr + G)) return 0;
    return 2 * N * (Cp + C * kr + G);
}

bool plan_groupnorm(int st, int ot, int pdt, int64_t N, int64_t C, int64_t L, int64_t G,
                    bool vec_ok, bool fwd, GnPlan& p)
{
    if (N < 1 || C < 1 || L < 1 || G < 1 || C % G != 0) return false;
    const int64_t Cg = C / G;
    const int64_t S = N * G;
    if (plan_registers(st, ot, pdt == ST_F32 ? 4 : 2, Cg, L, S, vec_ok, fwd, p)) return true;
    const int64_t M = Cg * L;
    if (M > INT32_MAX || L > INT32_MAX / 2) return false;
    p.split = true;
    p.id = vec_ok ? 1 : 0;
    split_geometry(st, L, M, vec_ok, p);
    p.units = N * C * p.Kr;
    const int64_t rg = kern::kGnUnitBlock / (8 << p.tid);
    if (cdiv(p.units, rg) > INT32_MAX || S * p.Kf > INT32_MAX || S > INT32_MAX) return false;
    // the workspace counts units of at least 8192 values
    if (p.Kr > cdiv(L, 8192)) return false;
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
