// mn_internal.hpp -- argument blocks, launch plans and launcher declarations
// shared by the C-ABI layer (mn_api.cpp) and the kernels (mn_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mn {

enum Kind : int { RMS = 0, LN = 1, ADD = 2 };

// Forward arguments. Pointers not used by a kind are null.
struct FwdArgs {
    const _Float16* X;
    const _Float16* R;       // ADD
    const _Float16* gamma;
    const _Float16* beta;    // LN
    _Float16* Y;
    _Float16* H;             // ADD
    float* mean;             // LN
    float* rstd;
    int64_t N;
    int32_t D;
    float eps;
    int64_t rows_per_block;  // contiguous rows owned by one workgroup
};

// Backward (stage 1) arguments.
struct BwdArgs {
    const _Float16* X;
    const _Float16* R;       // ADD
    const _Float16* gamma;
    const _Float16* dY;
    const _Float16* dH;      // ADD, may be null (zero cotangent)
    const float* mean;       // LN
    const float* rstd;
    _Float16* dX;
    float* part_g;           // [P][Dp] dgamma partials
    float* part_b;           // [P][Dp] dbeta partials (LN)
    int64_t N;
    int32_t D;
    int32_t Dp;              // partial row stride (D rounded up to 4)
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
    int64_t grid;
    int64_t rows_per_block;
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

FwdPlan plan_forward(int kind, int64_t N, int32_t D, bool vec_ok);
BwdPlan plan_backward(int kind, int64_t N, int32_t D, bool vec_ok);

hipError_t launch_forward(int kind, const FwdPlan& p, const FwdArgs& a, hipStream_t s);
hipError_t launch_backward_rows(int kind, const BwdPlan& p, const BwdArgs& a, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);

}  // namespace mn
