// mn_tables.hpp -- the launch tables of the gfx950 normalization kernels:
// which template instance serves which width and storage combination.
// Shared by the planner (mn_kernels.hip) and the per-storage instance files
// (mn_inst_*.hip), which define and instantiate the launchers.
#pragma once

#include "mn_internal.hpp"

namespace mn {

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
//     inputs non-temporal loads (NT bit 1), except the LayerNorm forward
//     away from 4096 columns, which measured slower with non-temporal loads
//     (at 4096 they measured 1 % faster in a same-box A/B).
// Rows 12 and 13 fit two common widths between the powers of two exactly
// (5120 columns, and 6144 in the forward), faster there than the next
// power-of-two row. Backward shapes away from 4096 columns come from a
// sweep at 64 M elements per call: at 3072 columns exact fits with several
// chunks per lane (RMSNorm 192 lanes x 2, LayerNorm 128 x 3; 20 % and 8 %
// faster than the 4096-column rows, where one chunk over 384 lanes was
// slower), at 5120 one row per group (RMSNorm, 7 %) and 128 lanes x 5 chunks
// (LayerNorm, 24 %), for the LayerNorm at 2048 and 8192 one row per group in
// larger workgroups (3 % and 7 %), at 4096 one 512-lane row group with two
// rows per step (1 % faster than two 256-lane groups of two chunks once its
// dX stores went through a buffer resource); the 6144-column backward keeps
// the 8192 row (exact fits within 2.5 %). The forward likewise prefers fewer lanes
// per row with more chunks per lane away from 4096 columns (4 to 8 waves per
// workgroup, one or two rows per group): 6-29 % faster than rows of 640 to
// 1024 lanes at 2048, 5120, 6144 and 8192 columns, and 32 lanes x 4 chunks at
// 1024 columns (7-13 %); it keeps the power-of-two rows at 3072 (exact fits
// within 2 %). At 512 columns the backward takes two row groups of 64 lanes
// per workgroup (9 %).
// Forward row 15 of RMSNorm and of LayerNorm (max_d 0, so never chosen by
// width) is row 6 with twice the rows per workgroup: the planner takes it
// instead of row 6 when 16-bit activations come with binary32 parameters,
// whose chunks per lane are twice as wide (at 16384 x 4096: RMSNorm 50.0 ->
// 46.8 us, LayerNorm 53.6 -> 48.8 us; with 16-bit parameters both measured
// 1-2 % slower with it).
// Ids are unique within a kind; 8..10 are the element-wise variants (any D,
// any alignment) shared by all kinds. Each row is instantiated for every
// storage combination (binary32 activations: see st_vec / st_cpt below).
//
//   id   T  VEC CPT  U  BLOCK  PF NT  max_d
#define MN_FWD_RMS(X)                        \
    X(0, 8, 8, 1, 4, 256, 0, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 0, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 0, 3, 256)        \
    X(3, 64, 8, 1, 2, 256, 0, 3, 512)        \
    X(4, 32, 8, 4, 1, 256, 0, 3, 1024)      \
    X(5, 256, 8, 1, 2, 256, 0, 3, 2048)      \
    X(6, 256, 8, 2, 1, 256, 0, 3, 4096)      \
    X(12, 320, 8, 2, 1, 320, 0, 3, 5120)     \
    X(13, 384, 8, 2, 1, 384, 0, 3, 6144)     \
    X(7, 256, 8, 4, 1, 256, 0, 3, 8192)      \
    X(15, 256, 8, 2, 2, 256, 0, 3, 0)
#define MN_FWD_LN(X)                         \
    X(0, 8, 8, 1, 4, 256, 0, 1, 64)          \
    X(1, 16, 8, 1, 2, 256, 0, 1, 128)        \
    X(2, 32, 8, 1, 2, 256, 0, 1, 256)        \
    X(3, 64, 8, 1, 2, 256, 0, 1, 512)        \
    X(4, 32, 8, 4, 1, 256, 0, 1, 1024)      \
    X(5, 64, 8, 4, 1, 256, 0, 1, 2048)      \
    X(6, 256, 8, 2, 2, 256, 0, 3, 4096)      \
    X(12, 128, 8, 5, 1, 256, 0, 1, 5120)     \
    X(13, 256, 8, 3, 1, 256, 0, 1, 6144)     \
    X(7, 256, 8, 4, 1, 256, 0, 1, 8192)      \
    X(15, 256, 8, 2, 4, 256, 0, 3, 0)
// The fused add (two inputs and two outputs per element) keeps rows of up to
// 1024 lanes away from 4096 columns: at 8192 the 256-lane row measured 4 %
// slower than the 1024-lane one.
#define MN_FWD_ADD(X)                        \
    X(0, 8, 8, 1, 4, 256, 0, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 0, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 0, 3, 256)        \
    X(3, 64, 8, 1, 2, 256, 0, 3, 512)        \
    X(4, 128, 8, 1, 1, 256, 0, 3, 1024)      \
    X(5, 256, 8, 1, 1, 256, 0, 3, 2048)      \
    X(6, 256, 8, 2, 1, 256, 0, 3, 4096)      \
    X(12, 640, 8, 1, 1, 640, 0, 3, 5120)     \
    X(13, 768, 8, 1, 1, 768, 0, 3, 6144)     \
    X(7, 1024, 8, 1, 1, 1024, 0, 3, 8192)
// The other norms. PolyNorm (three sums per row) takes the LayerNorm shapes.
// Dynamic Tanh (two parameter vectors, no reduction) and Modulated RMSNorm
// (the sample's scale and shift rows with each tile) take the RMSNorm shapes
// except where two rows per group amortise the parameter loads: at 4096
// columns a 512-lane row (3 % faster than 256 lanes x 2 chunks for DyT), and
// for MOD an exact fit of 3072 columns (128 lanes x 3 chunks, two rows per
// group: 5 % faster than the 4096-column row; 384-lane rows were 19 %
// slower), from timing sweeps at 16384 rows.
#define MN_FWD_DYT(X)                        \
    X(0, 8, 8, 1, 4, 256, 0, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 0, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 0, 3, 256)        \
    X(3, 64, 8, 1, 2, 256, 0, 3, 512)        \
    X(4, 32, 8, 4, 1, 256, 0, 3, 1024)      \
    X(5, 256, 8, 1, 2, 256, 0, 3, 2048)      \
    X(6, 512, 8, 1, 2, 512, 0, 3, 4096)      \
    X(12, 320, 8, 2, 1, 320, 0, 3, 5120)     \
    X(13, 384, 8, 2, 1, 384, 0, 3, 6144)     \
    X(7, 256, 8, 4, 1, 256, 0, 3, 8192)
// PolyNorm: the LayerNorm shapes (three sums per row), but with non-temporal
// loads as well as stores, and 128 lanes x 4 chunks at 4096 columns: a width
// sweep measured them 4-15 % faster than the LayerNorm rows at 1024-8192
// columns.
#define MN_FWD_POLY(X)                       \
    X(0, 8, 8, 1, 4, 256, 0, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 0, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 0, 3, 256)        \
    X(3, 64, 8, 1, 2, 256, 0, 3, 512)        \
    X(4, 32, 8, 4, 1, 256, 0, 3, 1024)      \
    X(5, 64, 8, 4, 1, 256, 0, 3, 2048)      \
    X(6, 128, 8, 4, 1, 256, 0, 3, 4096)      \
    X(12, 128, 8, 5, 1, 256, 0, 3, 5120)     \
    X(13, 256, 8, 3, 1, 256, 0, 3, 6144)     \
    X(7, 256, 8, 4, 1, 256, 0, 3, 8192)
#define MN_FWD_MOD(X)                        \
    X(0, 8, 8, 1, 4, 256, 0, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 0, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 0, 3, 256)        \
    X(3, 64, 8, 1, 2, 256, 0, 3, 512)        \
    X(4, 32, 8, 4, 1, 256, 0, 3, 1024)      \
    X(5, 256, 8, 1, 2, 256, 0, 3, 2048)      \
    X(14, 128, 8, 3, 2, 256, 0, 3, 3072)     \
    X(6, 256, 8, 2, 1, 256, 0, 3, 4096)      \
    X(12, 320, 8, 2, 1, 320, 0, 3, 5120)     \
    X(13, 384, 8, 2, 1, 384, 0, 3, 6144)     \
    X(7, 256, 8, 4, 1, 256, 0, 3, 8192)
#define MN_FWD_GEN(X)                        \
    X(8, 64, 1, 16, 1, 256, 0, 1, 1024)      \
    X(9, 256, 1, 16, 1, 256, 0, 1, 4096)     \
    X(10, 512, 1, 16, 1, 512, 0, 1, 8192)

#define MN_BWD_RMS(X)                        \
    X(0, 8, 8, 1, 4, 256, 1, 3, 64)          \
    X(1, 16, 8, 1, 4, 256, 1, 3, 128)        \
    X(2, 32, 8, 1, 4, 256, 1, 3, 256)        \
    X(3, 64, 8, 1, 2, 512, 1, 3, 512)        \
    X(4, 128, 8, 1, 2, 512, 1, 3, 1024)      \
    X(5, 256, 8, 1, 2, 512, 1, 3, 2048)      \
    X(14, 192, 8, 2, 1, 384, 1, 3, 3072)     \
    X(6, 512, 8, 1, 3, 512, 1, 3, 4096)      \
    X(12, 640, 8, 1, 1, 640, 1, 3, 5120)     \
    X(7, 1024, 8, 1, 1, 1024, 1, 3, 8192)
#define MN_BWD_LN(X)                         \
    X(0, 8, 8, 1, 4, 256, 1, 3, 64)          \
    X(1, 16, 8, 1, 4, 256, 1, 3, 128)        \
    X(2, 32, 8, 1, 4, 256, 1, 3, 256)        \
    X(3, 64, 8, 1, 2, 512, 1, 3, 512)        \
    X(4, 64, 8, 2, 2, 256, 1, 3, 1024)       \
    X(5, 128, 8, 2, 1, 512, 1, 3, 2048)      \
    X(14, 128, 8, 3, 1, 256, 1, 3, 3072)     \
    X(6, 512, 8, 1, 2, 512, 1, 3, 4096)      \
    X(12, 128, 8, 5, 1, 256, 1, 3, 5120)     \
    X(7, 512, 8, 2, 1, 1024, 1, 3, 8192)
// The fused add keeps two rows per group at 4096 columns (its four streams
// per element hold more registers).
#define MN_BWD_ADD(X)                        \
    X(0, 8, 8, 1, 4, 256, 1, 3, 64)          \
    X(1, 16, 8, 1, 4, 256, 1, 3, 128)        \
    X(2, 32, 8, 1, 4, 256, 1, 3, 256)        \
    X(3, 64, 8, 1, 2, 512, 1, 3, 512)        \
    X(4, 128, 8, 1, 2, 512, 1, 3, 1024)      \
    X(5, 256, 8, 1, 2, 512, 1, 3, 2048)      \
    X(14, 192, 8, 2, 1, 384, 1, 3, 3072)     \
    X(6, 512, 8, 1, 2, 512, 1, 3, 4096)      \
    X(12, 640, 8, 1, 1, 640, 1, 3, 5120)     \
    X(7, 1024, 8, 1, 1, 1024, 1, 3, 8192)
// The other norms keep two or three per-column accumulators, or four row
// sums, and (DYT) an inlined tanh per element: one row per group per step
// keeps them within 128 VGPRs without spilling.
// PolyNorm reduces four sums per row for little arithmetic per element, so
// it takes several chunks per lane (fewer lanes per row) to amortise them.
// At 4096 columns 128 lanes x 4 chunks measured 13 % faster than 256 x 2.
#define MN_BWD_POLY(X)                       \
    X(0, 8, 8, 1, 2, 256, 1, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 1, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 1, 3, 256)        \
    X(3, 64, 8, 1, 1, 256, 1, 3, 512)        \
    X(4, 64, 8, 2, 1, 256, 1, 3, 1024)       \
    X(5, 128, 8, 2, 1, 512, 1, 3, 2048)      \
    X(6, 128, 8, 4, 1, 512, 1, 3, 4096)      \
    X(12, 320, 8, 2, 1, 320, 1, 3, 5120)     \
    X(7, 512, 8, 2, 1, 512, 1, 3, 8192)
// Dynamic Tanh at 4096 columns: 256 lanes x 2 chunks, two row groups per
// workgroup (4 % faster than one 512-lane group).
#define MN_BWD_DYT(X)                        \
    X(0, 8, 8, 1, 2, 256, 1, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 1, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 1, 3, 256)        \
    X(3, 64, 8, 1, 1, 256, 1, 3, 512)        \
    X(4, 128, 8, 1, 1, 512, 1, 3, 1024)      \
    X(5, 256, 8, 1, 1, 512, 1, 3, 2048)      \
    X(6, 256, 8, 2, 1, 512, 1, 3, 4096)      \
    X(12, 640, 8, 1, 1, 640, 1, 3, 5120)     \
    X(7, 1024, 8, 1, 1, 1024, 1, 3, 8192)
// Modulated RMSNorm: an exact fit of 3072 columns, 128 lanes x 3 chunks
// (19 % faster than the 4096-column row of 512 lanes).
#define MN_BWD_MOD(X)                        \
    X(0, 8, 8, 1, 2, 256, 1, 3, 64)          \
    X(1, 16, 8, 1, 2, 256, 1, 3, 128)        \
    X(2, 32, 8, 1, 2, 256, 1, 3, 256)        \
    X(3, 64, 8, 1, 1, 256, 1, 3, 512)        \
    X(4, 128, 8, 1, 1, 512, 1, 3, 1024)      \
    X(5, 256, 8, 1, 1, 512, 1, 3, 2048)      \
    X(14, 128, 8, 3, 1, 256, 1, 3, 3072)     \
    X(6, 512, 8, 1, 1, 512, 1, 3, 4096)      \
    X(12, 640, 8, 1, 1, 640, 1, 3, 5120)     \
    X(7, 1024, 8, 1, 1, 1024, 1, 3, 8192)
#define MN_BWD_GEN(X)                        \
    X(8, 64, 1, 16, 1, 256, 1, 1, 1024)      \
    X(9, 256, 1, 16, 1, 256, 1, 1, 4096)     \
    X(10, 512, 1, 16, 1, 512, 1, 1, 8192)

// Storage combinations of the backward (X/R, dY/dH, dX), one list per
// activation type: cotangents in the activation type or binary32 and dX in
// the activation type or binary32; binary32 activations take cotangents of
// any type and give a binary32 dX.
#define MN_BWD_TYPES_F16(X)                                                     \
    X(ST_F16, ST_F16, ST_F16) X(ST_F16, ST_F16, ST_F32) X(ST_F16, ST_F32, ST_F16) \
    X(ST_F16, ST_F32, ST_F32)
#define MN_BWD_TYPES_BF16(X)                                                         \
    X(ST_BF16, ST_BF16, ST_BF16) X(ST_BF16, ST_BF16, ST_F32) X(ST_BF16, ST_F32, ST_BF16) \
    X(ST_BF16, ST_F32, ST_F32)
#define MN_BWD_TYPES_F32(X) \
    X(ST_F32, ST_F32, ST_F32) X(ST_F32, ST_F16, ST_F32) X(ST_F32, ST_BF16, ST_F32)
#define MN_BWD_TYPES(X) MN_BWD_TYPES_F16(X) MN_BWD_TYPES_BF16(X) MN_BWD_TYPES_F32(X)

// The other norms (DYT, POLY, MOD): cotangents in the activation type, dX in
// the activation type or binary32.
#define MN_BWD_TYPES_EXT_F16(X) X(ST_F16, ST_F16, ST_F16) X(ST_F16, ST_F16, ST_F32)
#define MN_BWD_TYPES_EXT_BF16(X) X(ST_BF16, ST_BF16, ST_BF16) X(ST_BF16, ST_BF16, ST_F32)
#define MN_BWD_TYPES_EXT_F32(X) X(ST_F32, ST_F32, ST_F32)
#define MN_BWD_TYPES_EXT(X) \
    MN_BWD_TYPES_EXT_F16(X) MN_BWD_TYPES_EXT_BF16(X) MN_BWD_TYPES_EXT_F32(X)

// binary32 storage keeps 16-byte chunks: 4 elements per chunk and twice the
// chunks per lane of the 16-bit shapes, so the row coverage T*CPT*VEC and
// the bytes in flight per lane are unchanged.
constexpr int st_vec(int st, int vec) { return (st == ST_F32 && vec == 8) ? 4 : vec; }
constexpr int st_cpt(int st, int vec, int cpt) { return (st == ST_F32 && vec == 8) ? 2 * cpt : cpt; }

// Launch one planned forward / backward-stage-1 kernel; defined and
// explicitly instantiated per activation storage type and kind group in
// mn_inst_*.hip.
template <int KIND, int ST>
hipError_t launch_fwd(const FwdPlan& p, const FwdArgs& a, hipStream_t s);
template <int KIND, int ST, int CT, int OT>
hipError_t launch_bwd(const BwdPlan& p, const BwdArgs& a, hipStream_t s);

}  // namespace mn
