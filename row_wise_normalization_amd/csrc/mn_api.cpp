// mn_api.cpp -- the C ABI declared in include/mn_norm.h: argument
// validation, launch planning and dispatch to the kernels. Validation runs on
// the host before anything is enqueued, so every error return leaves device
// memory untouched.
#include "mn_norm.h"

#include <cmath>
#include <cstring>
#include <string>

#include "mn_internal.hpp"

namespace {

thread_local std::string g_last_device_error;

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, size_t bytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Span{a, p ? a + bytes : a};
}

bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

bool shape_ok(int64_t N, int64_t D)
{
    if (N < 1 || D < 1 || D > MN_MAX_COLS) return false;
    // element offsets are formed in int64 and byte spans in uintptr_t
    return N <= (INT64_MAX / 8) / D;
}

bool eps_ok(float eps) { return std::isfinite(eps) && eps > 0.0f; }

bool dtype_ok(int t) { return t == MN_F16 || t == MN_BF16 || t == MN_F32; }

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Outputs must not overlap any input or each other (no in-place mutation).
template <size_t NI, size_t NO>
bool alias_free(const Span (&in)[NI], const Span (&out)[NO])
{
    for (size_t o = 0; o < NO; ++o) {
        if (out[o].lo == out[o].hi) continue;
        for (size_t i = 0; i < NI; ++i)
            if (in[i].lo != in[i].hi && overlap(out[o], in[i])) return false;
        for (size_t p = o + 1; p < NO; ++p)
            if (out[p].lo != out[p].hi && overlap(out[o], out[p])) return false;
    }
    return true;
}

// 128-bit chunks need whole 16-byte chunks per row: D a multiple of 8
// elements for the 16-bit storage types, of 4 for binary32.
bool chunks_fit(int st, int64_t D) { return D % (st == mn::ST_F32 ? 4 : 8) == 0; }

size_t workspace_bytes(int kind, int64_t N, int64_t D)
{
    if (!shape_ok(N, D) || kind < 0 || kind > 2) return 0;
    const int64_t P = mn::bwd_partial_rows(kind, N, (int32_t)D);
    const int64_t Dp = mn::partial_stride((int32_t)D);
    return (size_t)P * (size_t)Dp * sizeof(float) * (kind == mn::LN ? 2u : 1u);
}

mn_status device_status(hipError_t e)
{
    if (e == hipSuccess) return MN_OK;
    g_last_device_error = hipGetErrorString(e);
    return MN_ERR_DEVICE;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------
// Forward.
// ---------------------------------------------------------------------------

mn_status forward(int kind, const void* X, const void* R, const void* gamma, const void* beta,
                  void* H, void* Y, float* mean, float* rstd, int64_t N, int64_t D, float eps,
                  int st, int pdt, void* stream)
{
    if (!X || !gamma || !Y || !rstd) return MN_ERR_NULL;
    if (kind == mn::LN && (!beta || !mean)) return MN_ERR_NULL;
    if (kind == mn::ADD && (!R || !H)) return MN_ERR_NULL;
    if (!dtype_ok(st) || !dtype_ok(pdt)) return MN_ERR_DTYPE;
    if (!shape_ok(N, D)) return MN_ERR_SHAPE;
    if (!eps_ok(eps)) return MN_ERR_EPS;

    const size_t nd = (size_t)N * (size_t)D * (size_t)mn::stor_bytes(st);
    const size_t dp = (size_t)D * (size_t)mn::stor_bytes(pdt);
    const Span in[] = {span(X, nd), span(R, nd), span(gamma, dp), span(beta, dp)};
    const Span out[] = {span(Y, nd), span(H, nd), span(rstd, (size_t)N * 4u),
                        span(mean, (size_t)N * 4u)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;

    const bool vec_ok = chunks_fit(st, D) && aligned16(X) && aligned16(R) && aligned16(gamma) &&
                        aligned16(beta) && aligned16(Y) && aligned16(H);
    const mn::FwdPlan plan = mn::plan_forward(kind, st, N, (int32_t)D, vec_ok);
    if (plan.grid > INT32_MAX) return MN_ERR_SHAPE;  // one workgroup per tile of rows
    mn::FwdArgs a;
    a.X = X;
    a.R = R;
    a.gamma = gamma;
    a.beta = beta;
    a.Y = Y;
    a.H = H;
    a.mean = mean;
    a.rstd = rstd;
    a.N = N;
    a.D = (int32_t)D;
    a.pdt = pdt;
    a.eps = eps;
    return device_status(mn::launch_forward(kind, st, plan, a, as_stream(stream)));
}

// ---------------------------------------------------------------------------
// Backward.
// ---------------------------------------------------------------------------

struct BwdIn {
    const void *X, *R, *gamma, *dY, *dH;
    const float *mean, *rstd;
    void* dX;
};

// Storage types of one backward call: activations (X, R), parameters
// (gamma), cotangents (dY, dH) and dX.
struct BwdTypes {
    int st, pdt, ct, ot;
};

mn_status backward_rows(int kind, const BwdIn& b, int64_t N, int64_t D, const BwdTypes& t,
                        void* ws, size_t ws_bytes, const float* dgamma, const float* dbeta,
                        void* stream)
{
    if (!b.X || !b.gamma || !b.dY || !b.rstd || !b.dX) return MN_ERR_NULL;
    if (kind == mn::LN && !b.mean) return MN_ERR_NULL;
    if (kind == mn::ADD && !b.R) return MN_ERR_NULL;
    if (!dtype_ok(t.st) || !dtype_ok(t.pdt) || !dtype_ok(t.ct) || !dtype_ok(t.ot) ||
        !mn::backward_types_supported(t.st, t.ct, t.ot))
        return MN_ERR_DTYPE;
    const int st = t.st;
    if (!shape_ok(N, D)) return MN_ERR_SHAPE;
    const size_t need = workspace_bytes(kind, N, D);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MN_ERR_WORKSPACE;

    const size_t nd = (size_t)N * (size_t)D * (size_t)mn::stor_bytes(st);
    const size_t ndc = (size_t)N * (size_t)D * (size_t)mn::stor_bytes(t.ct);
    const size_t ndo = (size_t)N * (size_t)D * (size_t)mn::stor_bytes(t.ot);
    const size_t dp = (size_t)D * (size_t)mn::stor_bytes(t.pdt);
    const Span in[] = {span(b.X, nd), span(b.R, nd), span(b.gamma, dp), span(b.dY, ndc),
                       span(b.dH, ndc), span(b.mean, (size_t)N * 4u),
                       span(b.rstd, (size_t)N * 4u)};
    const Span out[] = {span(b.dX, ndo), span(ws, need), span(dgamma, (size_t)D * 4u),
                        span(dbeta, (size_t)D * 4u)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;

    const bool vec_ok = chunks_fit(st, D) && aligned16(b.X) && aligned16(b.R) &&
                        aligned16(b.gamma) && aligned16(b.dY) && aligned16(b.dH) &&
                        aligned16(b.dX);
    const mn::BwdPlan plan = mn::plan_backward(kind, st, N, (int32_t)D, vec_ok);
    mn::BwdArgs a;
    a.X = b.X;
    a.R = b.R;
    a.gamma = b.gamma;
    a.dY = b.dY;
    a.dH = b.dH;
    a.mean = b.mean;
    a.rstd = b.rstd;
    a.dX = b.dX;
    a.part_g = static_cast<float*>(ws);
    a.part_b = (kind == mn::LN) ? static_cast<float*>(ws) + plan.P * plan.Dp : nullptr;
    a.N = N;
    a.D = (int32_t)D;
    a.Dp = plan.Dp;
    a.pdt = t.pdt;
    return device_status(
        mn::launch_backward_rows(kind, st, t.ct, t.ot, plan, a, as_stream(stream)));
}

mn_status reduce_partials(int kind, int64_t N, int64_t D, const void* ws, size_t ws_bytes,
                          float* dgamma, float* dbeta, void* stream)
{
    if (!dgamma || (kind == mn::LN && !dbeta)) return MN_ERR_NULL;
    if (kind < 0 || kind > 2) return MN_ERR_SHAPE;
    if (!shape_ok(N, D)) return MN_ERR_SHAPE;
    const size_t need = workspace_bytes(kind, N, D);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MN_ERR_WORKSPACE;
    const Span in[] = {span(ws, need)};
    const Span out[] = {span(dgamma, (size_t)D * 4u),
                        span(kind == mn::LN ? dbeta : nullptr, (size_t)D * 4u)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;

    mn::ReduceArgs a;
    a.P = mn::bwd_partial_rows(kind, N, (int32_t)D);
    a.Dp = mn::partial_stride((int32_t)D);
    a.D = (int32_t)D;
    a.part_g = static_cast<const float*>(ws);
    a.part_b = (kind == mn::LN) ? static_cast<const float*>(ws) + a.P * a.Dp : nullptr;
    a.dgamma = dgamma;
    a.dbeta = (kind == mn::LN) ? dbeta : nullptr;
    return device_status(mn::launch_reduce(a, as_stream(stream)));
}

const BwdTypes kF16{MN_F16, MN_F16, MN_F16, MN_F16};

mn_status backward(int kind, const BwdIn& b, float* dgamma, float* dbeta, int64_t N, int64_t D,
                   const BwdTypes& t, void* ws, size_t ws_bytes, void* stream)
{
    if (!dgamma || (kind == mn::LN && !dbeta)) return MN_ERR_NULL;
    mn_status s = backward_rows(kind, b, N, D, t, ws, ws_bytes, dgamma, dbeta, stream);
    if (s != MN_OK) return s;
    return reduce_partials(kind, N, D, ws, ws_bytes, dgamma, dbeta, stream);
}

}  // namespace

extern "C" {

// --- binary16 entry points ---------------------------------------------------

mn_status mn_rmsnorm_forward(const mn_f16* X, const mn_f16* gamma, mn_f16* Y, float* rstd,
                             int64_t N, int64_t D, float eps, void* stream)
{
    return forward(mn::RMS, X, nullptr, gamma, nullptr, nullptr, Y, nullptr, rstd, N, D, eps,
                   MN_F16, MN_F16, stream);
}

mn_status mn_layernorm_forward(const mn_f16* X, const mn_f16* gamma, const mn_f16* beta,
                               mn_f16* Y, float* mean, float* rstd, int64_t N, int64_t D,
                               float eps, void* stream)
{
    return forward(mn::LN, X, nullptr, gamma, beta, nullptr, Y, mean, rstd, N, D, eps, MN_F16,
                   MN_F16, stream);
}

mn_status mn_add_rmsnorm_forward(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                 mn_f16* H, mn_f16* Y, float* rstd, int64_t N, int64_t D,
                                 float eps, void* stream)
{
    return forward(mn::ADD, X, R, gamma, nullptr, H, Y, nullptr, rstd, N, D, eps, MN_F16,
                   MN_F16, stream);
}

mn_status mn_rmsnorm_backward(const mn_f16* X, const mn_f16* gamma, const float* rstd,
                              const mn_f16* dY, mn_f16* dX, float* dgamma, int64_t N, int64_t D,
                              void* workspace, size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX};
    return backward(mn::RMS, b, dgamma, nullptr, N, D, kF16, workspace, workspace_bytes,
                    stream);
}

mn_status mn_layernorm_backward(const mn_f16* X, const mn_f16* gamma, const float* mean,
                                const float* rstd, const mn_f16* dY, mn_f16* dX, float* dgamma,
                                float* dbeta, int64_t N, int64_t D, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, nullptr, gamma, dY, nullptr, mean, rstd, dX};
    return backward(mn::LN, b, dgamma, dbeta, N, D, kF16, workspace, workspace_bytes,
                    stream);
}

mn_status mn_add_rmsnorm_backward(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                  const float* rstd, const mn_f16* dY, const mn_f16* dH,
                                  mn_f16* dX, float* dgamma, int64_t N, int64_t D,
                                  void* workspace, size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, R, gamma, dY, dH, nullptr, rstd, dX};
    return backward(mn::ADD, b, dgamma, nullptr, N, D, kF16, workspace, workspace_bytes,
                    stream);
}

mn_status mn_rmsnorm_backward_rows(const mn_f16* X, const mn_f16* gamma, const float* rstd,
                                   const mn_f16* dY, mn_f16* dX, int64_t N, int64_t D,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX};
    return backward_rows(mn::RMS, b, N, D, kF16, workspace, workspace_bytes, nullptr,
                         nullptr, stream);
}

mn_status mn_layernorm_backward_rows(const mn_f16* X, const mn_f16* gamma, const float* mean,
                                     const float* rstd, const mn_f16* dY, mn_f16* dX, int64_t N,
                                     int64_t D, void* workspace, size_t workspace_bytes,
                                     void* stream)
{
    const BwdIn b{X, nullptr, gamma, dY, nullptr, mean, rstd, dX};
    return backward_rows(mn::LN, b, N, D, kF16, workspace, workspace_bytes, nullptr,
                         nullptr, stream);
}

mn_status mn_add_rmsnorm_backward_rows(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                       const float* rstd, const mn_f16* dY, const mn_f16* dH,
                                       mn_f16* dX, int64_t N, int64_t D, void* workspace,
                                       size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, R, gamma, dY, dH, nullptr, rstd, dX};
    return backward_rows(mn::ADD, b, N, D, kF16, workspace, workspace_bytes, nullptr,
                         nullptr, stream);
}

// --- entry points with explicit storage types --------------------------------

mn_status mn_rmsnorm_forward_ex(const void* X, const void* gamma, void* Y, float* rstd, int64_t N,
                                int64_t D, float eps, mn_dtype act, mn_dtype param, void* stream)
{
    return forward(mn::RMS, X, nullptr, gamma, nullptr, nullptr, Y, nullptr, rstd, N, D, eps,
                   act, param, stream);
}

mn_status mn_layernorm_forward_ex(const void* X, const void* gamma, const void* beta, void* Y,
                                  float* mean, float* rstd, int64_t N, int64_t D, float eps,
                                  mn_dtype act, mn_dtype param, void* stream)
{
    return forward(mn::LN, X, nullptr, gamma, beta, nullptr, Y, mean, rstd, N, D, eps, act, param,
                   stream);
}

mn_status mn_add_rmsnorm_forward_ex(const void* X, const void* R, const void* gamma, void* H,
                                    void* Y, float* rstd, int64_t N, int64_t D, float eps,
                                    mn_dtype act, mn_dtype param, void* stream)
{
    return forward(mn::ADD, X, R, gamma, nullptr, H, Y, nullptr, rstd, N, D, eps, act, param,
                   stream);
}

mn_status mn_rmsnorm_backward_ex(const void* X, const void* gamma, const float* rstd,
                                 const void* dY, void* dX, float* dgamma, int64_t N, int64_t D,
                                 mn_dtype act, mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                 void* workspace, size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX};
    return backward(mn::RMS, b, dgamma, nullptr, N, D, BwdTypes{act, param, cot, dxt},
                    workspace, workspace_bytes, stream);
}

mn_status mn_layernorm_backward_ex(const void* X, const void* gamma, const float* mean,
                                   const float* rstd, const void* dY, void* dX, float* dgamma,
                                   float* dbeta, int64_t N, int64_t D, mn_dtype act,
                                   mn_dtype param, mn_dtype cot, mn_dtype dxt, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, nullptr, gamma, dY, nullptr, mean, rstd, dX};
    return backward(mn::LN, b, dgamma, dbeta, N, D, BwdTypes{act, param, cot, dxt}, workspace,
                    workspace_bytes, stream);
}

mn_status mn_add_rmsnorm_backward_ex(const void* X, const void* R, const void* gamma,
                                     const float* rstd, const void* dY, const void* dH, void* dX,
                                     float* dgamma, int64_t N, int64_t D, mn_dtype act,
                                     mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                     void* workspace, size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, R, gamma, dY, dH, nullptr, rstd, dX};
    return backward(mn::ADD, b, dgamma, nullptr, N, D, BwdTypes{act, param, cot, dxt},
                    workspace, workspace_bytes, stream);
}

mn_status mn_rmsnorm_backward_rows_ex(const void* X, const void* gamma, const float* rstd,
                                      const void* dY, void* dX, int64_t N, int64_t D,
                                      mn_dtype act, mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                      void* workspace, size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX};
    return backward_rows(mn::RMS, b, N, D, BwdTypes{act, param, cot, dxt}, workspace,
                         workspace_bytes, nullptr, nullptr, stream);
}

mn_status mn_layernorm_backward_rows_ex(const void* X, const void* gamma, const float* mean,
                                        const float* rstd, const void* dY, void* dX, int64_t N,
                                        int64_t D, mn_dtype act, mn_dtype param, mn_dtype cot,
                                        mn_dtype dxt, void* workspace, size_t workspace_bytes,
                                        void* stream)
{
    const BwdIn b{X, nullptr, gamma, dY, nullptr, mean, rstd, dX};
    return backward_rows(mn::LN, b, N, D, BwdTypes{act, param, cot, dxt}, workspace,
                         workspace_bytes, nullptr, nullptr, stream);
}

mn_status mn_add_rmsnorm_backward_rows_ex(const void* X, const void* R, const void* gamma,
                                          const float* rstd, const void* dY, const void* dH,
                                          void* dX, int64_t N, int64_t D, mn_dtype act,
                                          mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                          void* workspace, size_t workspace_bytes, void* stream)
{
    const BwdIn b{X, R, gamma, dY, dH, nullptr, rstd, dX};
    return backward_rows(mn::ADD, b, N, D, BwdTypes{act, param, cot, dxt}, workspace,
                         workspace_bytes, nullptr, nullptr, stream);
}

// --- workspace, stage 2, diagnostics ----------------------------------------

mn_status mn_norm_reduce_partials(mn_norm_kind kind, int64_t N, int64_t D, const void* workspace,
                                  size_t workspace_bytes, float* dgamma, float* dbeta,
                                  void* stream)
{
    return reduce_partials((int)kind, N, D, workspace, workspace_bytes, dgamma, dbeta, stream);
}

size_t mn_norm_workspace_bytes(mn_norm_kind kind, int64_t N, int64_t D)
{
    return workspace_bytes((int)kind, N, D);
}

const char* mn_status_string(mn_status s)
{
    switch (s) {
    case MN_OK: return "ok";
    case MN_ERR_NULL: return "a required pointer is NULL";
    case MN_ERR_SHAPE: return "shape out of range: need N >= 1 and 1 <= D <= 8192";
    case MN_ERR_EPS: return "eps must be a positive finite float";
    case MN_ERR_ALIAS: return "an output overlaps an input or another output";
    case MN_ERR_WORKSPACE: return "workspace missing, too small or not 16-byte aligned";
    case MN_ERR_DEVICE: return "the HIP runtime rejected a launch";
    case MN_ERR_DTYPE: return "unknown storage type or unsupported combination";
    }
    return "unknown status";
}

const char* mn_last_device_error(void) { return g_last_device_error.c_str(); }

}  // extern "C"
