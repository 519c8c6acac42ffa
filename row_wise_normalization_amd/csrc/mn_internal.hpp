// mn_internal.hpp -- argument blocks, launch plans and launcher declarations
// shared by the C-ABI layer (mn_api.cpp) and the kernels (mn_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mn {

enum Kind : int { RMS = 0, LN = 1, ADD = 2 };

// Storage types; the values match mn_dtype in mn_norm.h.
enum Stor : int { ST_F16 = 0, ST_BF16 = 1, ST_F32 = 2 };

inline int stor_bytes(int st) { return st == ST_F32 ? 4 : 2; }

// Forward arguments. Pointers not used by a kind are null. Activations
// (X, R, Y, H) share one storage type (a template parameter of the kernel);
// gamma and beta share the parameter storage type `pdt`.
struct FwdArgs {
    const void* X;
    const void* R;           // ADD
    const void* gamma;
    const void* beta;        // LN
    void* Y;
    void* H;                 // ADD
    float* mean;             // LN
    float* rstd;
    int64_t N;
    int32_t D;
    int32_t pdt;             // storage type of gamma / beta
    float eps;
};

// Backward (stage 1) arguments. X and R share the activation storage type,
// dY and dH the cotangent storage type; dX has its own.
struct BwdArgs {
    const void* X;
    const void* R;           // ADD
    const void* gamma;
    const void* dY;
    const void* dH;          // ADD, may be null (zero cotangent)
    const float* mean;       // LN
    const float* rstd;
    void* dX;
    float* part_g;           // [P][Dp] dgamma partials
    float* part_b;           // [P][Dp] dbeta partials (LN)
    int64_t N;
    int32_t D;
    int32_t Dp;              // partial row stride (D rounded up to 4)
    int32_t pdt;             // storage type of gamma
};

// Column-reduce (stage 2) arguments.
struct ReduceArgs {
    const float* part_g;
    const float* part_b;     // null unless LN
    float* dgamma;
    float* dbeta;
    int64_t P;               // partial rows
    int32_t D;
    int32_t Dp;
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
    int32_t Dp;
    size_t shmem;            // dynamic LDS bytes of the block-level fold
};

// Partial-buffer geometry; depends only on (kind, N, D).
int64_t bwd_partial_rows(int kind, int64_t N, int32_t D);
int32_t partial_stride(int32_t D);

FwdPlan plan_forward(int kind, int st, int64_t N, int32_t D, bool vec_ok);
BwdPlan plan_backward(int kind, int st, int64_t N, int32_t D, bool vec_ok);

hipError_t launch_forward(int kind, int st, const FwdPlan& p, const FwdArgs& a, hipStream_t s);
// Backward storage combinations (activations st, cotangents ct, dX ot).
bool backward_types_supported(int st, int ct, int ot);
hipError_t launch_backward_rows(int kind, int st, int ct, int ot, const BwdPlan& p,
                                const BwdArgs& a, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);

}  // namespace mn
