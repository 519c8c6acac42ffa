// mn_internal.hpp -- argument blocks, launch plans and launcher declarations
// shared by the C-ABI layer (mn_api.cpp) and the kernels (mn_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mn {

// Norm kinds: the training pair (RMS, LN, ADD) and the other row-wise norms
// (DYT: Dynamic Tanh, POLY: PolyNorm, MOD: Modulated RMSNorm).
enum Kind : int { RMS = 0, LN = 1, ADD = 2, DYT = 3, POLY = 4, MOD = 5 };

// Storage types; the values match mn_dtype in mn_norm.h.
enum Stor : int { ST_F16 = 0, ST_BF16 = 1, ST_F32 = 2 };

inline int stor_bytes(int st) { return st == ST_F32 ? 4 : 2; }

// Forward arguments. Pointers not used by a kind are null. Activations
// (X, R, Y, H, and MOD's scale and shift) share one storage type (a template
// parameter of the kernel); gamma and beta share the parameter storage type
// `pdt`.
struct FwdArgs {
    const void* X;
    const void* R;           // ADD
    const void* gamma;       // all but POLY
    const void* beta;        // LN, DYT
    const float* alpha;      // DYT: the scalar alpha (device)
    const float* poly;       // POLY: w1, w2, w3, b (device)
    const void* scale;       // MOD: [B][D]
    const void* shift;       // MOD: [B][D]
    void* Y;
    void* H;                 // ADD
    float* mean;             // LN
    float* rstd;             // [N] (POLY: [N][3])
    int64_t N;
    int64_t S;               // MOD: rows per sample
    int32_t D;
    int32_t pdt;             // storage type of gamma / beta
    float eps;
};

// Backward (stage 1) arguments. X and R share the activation storage type,
// dY and dH the cotangent storage type; dX has its own.
struct BwdArgs {
    const void* X;
    const void* R;           // ADD
    const void* gamma;       // all but POLY
    const void* dY;
    const void* dH;          // ADD, may be null (zero cotangent)
    const float* mean;       // LN
    const float* rstd;       // [N] (POLY: [N][3])
    const float* alpha;      // DYT
    const float* poly;       // POLY: w1, w2, w3, b
    const void* scale;       // MOD: [B][D], activation storage type
    void* dX;
    float* part_g;           // [P][Dp] dgamma partials
    float* part_b;           // [P][Dp] dbeta (LN, DYT) or dscale (MOD) partials
    float* part_h;           // MOD: [P][Dp] dshift partials
    float* part_a;           // DYT, POLY: [P][4] scalar partials
    int64_t N;
    int64_t S;               // MOD: rows per sample
    int32_t D;
    int32_t Dp;              // partial row stride (D rounded up to 4)
    int32_t pdt;             // storage type of gamma
    int32_t Pb;              // MOD: workgroups per sample (workgroup b serves sample b / Pb)
    // one-launch backward of small problems (null otherwise): the hand-off
    // words [epoch][flag per workgroup] and the parameter gradients
    uint64_t* sync;
    float* dgamma;
    float* dbeta;            // LN
};

// Column-reduce (stage 2) arguments. One launch reduces up to
// kReduceMaxPlanes planes, each of its own shape: for plane y and group
// z < groups, out[z * D + j] = sum over the P rows p of
// part[(z * P + p) * Dp + j].
struct ReducePlane {
    const float* part;
    float* out;
    int64_t P;               // partial rows per group
    int32_t D;
    int32_t Dp;              // partial row stride (a multiple of 4)
    int32_t groups;
};
constexpr int kReduceMaxPlanes = 3;
struct ReduceArgs {
    ReducePlane plane[kReduceMaxPlanes];
    int32_t planes;
};

// Row-kernel variant: threads per row (T), elements per load (VEC, 8 or 1),
// loads per thread per row (CPT), rows per row-group per iteration (U) and
// workgroup size (BLOCK).
struct Variant {
    int id;
    int T, VEC, CPT, U, BLOCK;
};

struct FwdPlan {
    Variant v;
    int64_t grid;            // one tile of (BLOCK / T) * U rows per workgroup
};

struct BwdPlan {
    Variant v;
    int64_t P;               // workgroups == partial rows
    int32_t Pb;              // MOD: workgroups per sample
    int32_t Dp;
    size_t shmem;            // dynamic LDS bytes of the block-level fold
};

// Partial-buffer geometry; depends only on (kind, N, D), and for MOD on the
// sample count B.
int64_t bwd_partial_rows(int kind, int64_t N, int32_t D);
// Small problems of RMSNorm, LayerNorm and the fused add (N * Dp at most
// 8 * kSmallPartialFloats): at most kSmallMaxP partial rows, added inside
// the row launch by the workgroup that finds every partial row written, so
// that the whole backward is one launch. The workspace then ends with the
// hand-off words: an epoch and one flag per workgroup (kSmallSyncBytes).
constexpr int64_t kSmallPartialFloats = 16384;
constexpr int64_t kSmallMaxP = 64;
constexpr size_t kSmallSyncBytes = (8 * (1 + kSmallMaxP) + 15) / 16 * 16;
bool bwd_small(int kind, int64_t N, int32_t D);
// The full backward is one launch for small problems whose rows have at most
// kSmallMaxD columns (every row variant up to that width has fewer than 1024
// lanes, the variants that carry the in-kernel reduce).
constexpr int32_t kSmallMaxD = 5120;
bool bwd_one_launch(int kind, int64_t N, int32_t D);
int32_t mod_blocks_per_sample(int64_t B, int64_t N);
int bwd_vector_partials(int kind);
int32_t partial_stride(int32_t D);

FwdPlan plan_forward(int kind, int st, int pdt, int64_t N, int32_t D, bool vec_ok, int64_t B);
BwdPlan plan_backward(int kind, int st, int64_t N, int32_t D, bool vec_ok, int64_t B = 1);

hipError_t launch_forward(int kind, int st, const FwdPlan& p, const FwdArgs& a, hipStream_t s);
// Backward storage combinations (activations st, cotangents ct, dX ot).
bool backward_types_supported(int kind, int st, int ct, int ot);
hipError_t launch_backward_rows(int kind, int st, int ct, int ot, const BwdPlan& p,
                                const BwdArgs& a, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);

// GroupNorm over X [N][C][L]: G groups of Cg = C / G consecutive channels;
// the (sample, group) slice s = n * G + g is Cg * L contiguous values.
//
// Slices that fit one workgroup's registers take one kernel per direction
// (persistent workgroups, one slice at a time, the next slice's loads in
// flight). Larger slices take the split path: the forward as per-chunk
// statistics, a fixed-order merge per slice and an apply pass; the backward
// as per-chunk channel sums, a per-slice merge (dgamma, dbeta partials and
// the slice sums) and an apply pass. A chunk ("unit") of the split path's
// row kernels is up to kGnUnitIt chunks per lane of one channel row.
struct GnArgs {
    const void* X;           // [N][C][L], storage type of the launch
    const void* gamma;       // [C], type pdt
    const void* beta;        // [C], type pdt (forward)
    const void* dY;          // [N][C][L] (backward)
    void* Y;                 // forward output
    void* dX;                // backward output, type OT of the launch
    float* mean;             // [N][G]
    float* rstd;             // [N][G]
    float* part_g;           // [N][Cp] per-sample sums of dY * xhat per channel
    float* part_b;           // [N][Cp] per-sample sums of dY per channel
    // split path
    float* unit_p;           // backward: [N * C * Kr] per-unit sums of dY * xhat
    float* unit_q;           // backward: [N * C * Kr] per-unit sums of dY
    float* slice_ab;         // backward: [N * G][2] the slice sums A, B
    float* stat;             // forward: [N * G * Kf][2] per-chunk mean and M2
    int64_t S;               // slices, N * G
    int64_t units;           // row units, N * C * Kr
    int32_t C, L, G, Cg, Cp, pdt;
    int32_t Kr;              // row units per channel row
    int32_t UL;              // values per row unit (the last one of a row may be shorter)
    int32_t Kf;              // statistics chunks per slice
    int32_t FL;              // values per statistics chunk (the last one may be shorter)
    float eps;
};

struct GnPlan {
    bool split;              // the split path (slice larger than one workgroup)
    int id;                  // register path: launch shape (T, VEC, CPT, U, prefetch);
                             // split path: 1 for 16-byte chunks, 0 element-wise
    int32_t block;           // register path: threads, a multiple of 64, at most 1024
    int64_t grid;            // register path: persistent workgroups, at most N * G
    int tid;                 // split path: lanes per row unit, 8 << tid
    int32_t Kr, UL, Kf, FL;  // split path geometry (see GnArgs)
    int64_t units;
};

// Plans either path for a valid shape (false only when a count exceeds the
// launch limits; `ot` is the dX type, the activation type for the forward;
// `pdt` the gamma / beta type); the workspace is gn_workspace_floats(N, C, L, G) floats
// for both paths.
bool plan_groupnorm(int st, int ot, int pdt, int64_t N, int64_t C, int64_t L, int64_t G,
                    bool vec_ok, bool fwd, GnPlan& p);
int64_t gn_workspace_floats(int64_t N, int64_t C, int64_t L, int64_t G);
hipError_t launch_gn_fwd(int st, const GnPlan& p, const GnArgs& a, hipStream_t s);
hipError_t launch_gn_bwd(int st, int ot, const GnPlan& p, const GnArgs& a, hipStream_t s);

// GroupNorm over channels-last X [N][L][C] (C contiguous per position): a
// sums pass over position chunks, a per-(sample, group) merge, an apply
// pass (mn_gnl.hip). The workspace is gnl_workspace_floats(N, L, C, G)
// floats: sa, sb [N][J][C] chunk sums, then (backward) part_g, part_b
// [N][Cp] and ab [N * G][2].
struct GnlArgs {
    const void* X;           // [N][L][C], storage type of the launch
    const void* gamma;       // [C], type pdt
    const void* beta;        // [C], type pdt (forward)
    const void* dY;          // [N][L][C] (backward)
    void* Y;                 // forward output
    void* dX;                // backward output, type OT of the launch
    float* mean;             // [N][G]
    float* rstd;             // [N][G]
    float* sa;               // [N][J][C] chunk sums (see mn_gnl.hip)
    float* sb;               // [N][J][C]
    float* part_g;           // backward: [N][Cp] per-sample sums of dY * xhat
    float* part_b;           // backward: [N][Cp] per-sample sums of dY
    float* ab;               // backward: [N * G][2] the group sums A, B
    int64_t N;
    int32_t L, C, G, Cg, Cp, pdt;
    int32_t J;               // position chunks per sample
    int32_t LC;              // positions per chunk (the last one may be shorter)
    int32_t CK;              // chunks of VEC channels per position
    float eps;
};
int32_t gnl_chunks(int64_t N, int64_t L);
int64_t gnl_workspace_floats(int64_t N, int64_t L, int64_t C, int64_t G);
// VEC (8 for 16-bit, 4 for binary32 storage, when C is a multiple of it and
// every activation pointer is 16-byte aligned; else 1) and the derived CK, LC.
void gnl_geometry(int st, bool vec_ok, GnlArgs& a, int& vec);
hipError_t launch_gnl_fwd(int st, int vec, const GnlArgs& a, hipStream_t s);
hipError_t launch_gnl_bwd(int st, int ot, int vec, const GnlArgs& a, hipStream_t s);

// Fused normalization + GEMV (inference): Y [M][N] = Norm(X [M][K]) @ W [K][N].
constexpr int kGemvMaxKB = 512;  // rows of W per tile (LDS slice of the product rows)
constexpr int kGemvMaxM = 8;
constexpr int kGemvStatFloats = 64;  // workspace head: {mean, rstd} per X row
// Arrival counters after the statistics, one per column tile (tiles are at
// least 64 columns wide), in an area of fixed size so that no shape's
// partials ever land on another shape's counters: N <= 64 * kGemvCountWords.
constexpr int64_t kGemvCountWords = 16384;

struct GemvArgs {
    const void* X;           // [M][K], storage type of the launch
    const void* gamma;       // [K], type pdt
    const void* beta;        // [K], type pdt (LayerNorm) or null
    const void* W;           // [K][N], storage type of the launch
    float* stats;            // [M][2] row statistics (workspace head)
    uint32_t* cnt;           // [NB] arrival counters, zero between calls
    float* part;             // [S][RE][N] fp32 partial products, RE = M (+2 LayerNorm)
    void* Y;                 // [M][N], storage type of the launch
    int32_t M, N, K, pdt;
    float eps;
    int32_t KB;              // W rows per tile
    int32_t S;               // K slices = ceil(K / KB)
    int32_t NB;              // column blocks
};

struct GemvPlan {
    bool vec;                // 16-byte W loads (N % 8 == 0, aligned)
    bool mfma;               // matrix-core tiles (binary16, 128 columns)
    int32_t MM;              // rows instantiated: 1, 2, 4 or 8 >= M
    int32_t rpw;             // W rows per wave load (tile columns 64 * VEC / rpw)
    int32_t NB, KB, S;
    int64_t grid;
};

GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, bool vec_ok, bool f16, bool ln);
hipError_t launch_gemv(int st, bool ln, const GemvPlan& p, const GemvArgs& a, hipStream_t s);

}  // namespace mn
