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

// Largest sample count of the Modulated RMSNorm (its backward keeps one set
// of partial rows per sample).
constexpr int64_t kMaxSamples = 4096;

bool samples_ok(int kind, int64_t B, int64_t N)
{
    if (kind != mn::MOD) return true;
    return B >= 1 && B <= kMaxSamples && N % B == 0;
}

int64_t partial_rows(int kind, int64_t N, int64_t D, int64_t B)
{
    if (kind == mn::MOD) return B * mn::mod_blocks_per_sample(B, N);
    return mn::bwd_partial_rows(kind, N, (int32_t)D);
}

bool has_scalar_partials(int kind) { return kind == mn::DYT || kind == mn::POLY; }

// Workspace: per-workgroup fp32 partial rows [P][Dp] for each per-column
// parameter gradient, then (DYT, POLY) [P][4] scalar partials, then (small
// problems of RMS, LN, ADD, whose backward is one launch) the hand-off words.
size_t workspace_bytes(int kind, int64_t N, int64_t D, int64_t B = 1)
{
    if (!shape_ok(N, D) || kind < 0 || kind > mn::MOD || !samples_ok(kind, B, N)) return 0;
    const int64_t P = partial_rows(kind, N, D, B);
    const int64_t Dp = mn::partial_stride((int32_t)D);
    size_t bytes = (size_t)P * (size_t)Dp * sizeof(float) * (size_t)mn::bwd_vector_partials(kind);
    if (has_scalar_partials(kind)) bytes += (size_t)P * 4u * sizeof(float);
    if (mn::bwd_small(kind, N, (int32_t)D)) bytes += mn::kSmallSyncBytes;
    return bytes;
}

mn_status device_status(hipError_t e)
{
    if (e == hipSuccess) return MN_OK;
    g_last_device_error = hipGetErrorString(e);
    return MN_ERR_DEVICE;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

namespace mn {
// MN_ERR_DEVICE with the runtime's text kept for mn_last_device_error (for
// the other translation units of the library).
mn_status record_device_error(hipError_t e) { return device_status(e); }
}  // namespace mn

namespace {

// ---------------------------------------------------------------------------
// Forward.
// ---------------------------------------------------------------------------

struct FwdIn {
    const void* X = nullptr;
    const void* R = nullptr;         // ADD
    const void* gamma = nullptr;     // all but POLY
    const void* beta = nullptr;      // LN, DYT
    const float* alpha = nullptr;    // DYT
    const float* poly = nullptr;     // POLY: w1, w2, w3, b
    const void* scale = nullptr;     // MOD
    const void* shift = nullptr;     // MOD
    void* H = nullptr;               // ADD
    void* Y = nullptr;
    float* mean = nullptr;           // LN
    float* rstd = nullptr;           // all but DYT (POLY: [N][3])
    int64_t B = 1;                   // MOD: samples
};

mn_status forward(int kind, const FwdIn& f, int64_t N, int64_t D, float eps, int st, int pdt,
                  void* stream)
{
    if (!f.X || !f.Y) return MN_ERR_NULL;
    if (kind != mn::POLY && !f.gamma) return MN_ERR_NULL;
    if (kind != mn::DYT && !f.rstd) return MN_ERR_NULL;
    if ((kind == mn::LN || kind == mn::DYT) && !f.beta) return MN_ERR_NULL;
    if (kind == mn::LN && !f.mean) return MN_ERR_NULL;
    if (kind == mn::ADD && (!f.R || !f.H)) return MN_ERR_NULL;
    if (kind == mn::DYT && !f.alpha) return MN_ERR_NULL;
    if (kind == mn::POLY && !f.poly) return MN_ERR_NULL;
    if (kind == mn::MOD && (!f.scale || !f.shift)) return MN_ERR_NULL;
    if (!dtype_ok(st) || !dtype_ok(pdt)) return MN_ERR_DTYPE;
    if (!shape_ok(N, D) || !samples_ok(kind, f.B, N)) return MN_ERR_SHAPE;
    if (kind != mn::DYT && !eps_ok(eps)) return MN_ERR_EPS;

    const size_t es = (size_t)mn::stor_bytes(st);
    const size_t nd = (size_t)N * (size_t)D * es;
    const size_t dp = (size_t)D * (size_t)mn::stor_bytes(pdt);
    const size_t bd = (kind == mn::MOD) ? (size_t)f.B * (size_t)D * es : 0;
    const size_t nstat = (size_t)N * 4u * (kind == mn::POLY ? 3u : 1u);
    const Span in[] = {span(f.X, nd), span(f.R, nd), span(f.gamma, dp), span(f.beta, dp),
                       span(f.alpha, 4), span(f.poly, 16), span(f.scale, bd), span(f.shift, bd)};
    const Span out[] = {span(f.Y, nd), span(f.H, nd), span(f.rstd, nstat),
                        span(f.mean, (size_t)N * 4u)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;

    const bool vec_ok = chunks_fit(st, D) && aligned16(f.X) && aligned16(f.R) &&
                        aligned16(f.gamma) && aligned16(f.beta) && aligned16(f.Y) &&
                        aligned16(f.H) && aligned16(f.scale) && aligned16(f.shift);
    const mn::FwdPlan plan = mn::plan_forward(kind, st, pdt, N, (int32_t)D, vec_ok, f.B);
    if (plan.grid > INT32_MAX) return MN_ERR_SHAPE;  // one workgroup per tile of rows
    mn::FwdArgs a;
    a.X = f.X;
    a.R = f.R;
    a.gamma = f.gamma;
    a.beta = f.beta;
    a.alpha = f.alpha;
    a.poly = f.poly;
    a.scale = f.scale;
    a.shift = f.shift;
    a.Y = f.Y;
    a.H = f.H;
    a.mean = f.mean;
    a.rstd = f.rstd;
    a.N = N;
    a.S = (kind == mn::MOD) ? N / f.B : 0;
    a.D = (int32_t)D;
    a.pdt = pdt;
    a.eps = eps;
    return device_status(mn::launch_forward(kind, st, plan, a, as_stream(stream)));
}

// ---------------------------------------------------------------------------
// Backward.
// ---------------------------------------------------------------------------

struct BwdIn {
    const void* X = nullptr;
    const void* R = nullptr;         // ADD
    const void* gamma = nullptr;     // all but POLY
    const void* dY = nullptr;
    const void* dH = nullptr;        // ADD (may be NULL)
    const float* mean = nullptr;     // LN
    const float* rstd = nullptr;     // all but DYT
    const float* alpha = nullptr;    // DYT
    const float* poly = nullptr;     // POLY
    const void* scale = nullptr;     // MOD
    void* dX = nullptr;
    int64_t B = 1;                   // MOD
};

// Parameter gradients (fp32).
struct BwdOut {
    float* dgamma = nullptr;         // all but POLY
    float* dbeta = nullptr;          // LN, DYT; MOD: dscale [B][D]
    float* dshift = nullptr;         // MOD [B][D]
    float* dscalar = nullptr;        // DYT: dalpha [1]; POLY: d(w1, w2, w3, b) [4]
};

// Storage types of one backward call: activations (X, R), parameters
// (gamma), cotangents (dY, dH) and dX.
struct BwdTypes {
    int st, pdt, ct, ot;
};

// Byte spans of the parameter-gradient outputs.
void out_spans(int kind, const BwdOut& o, int64_t D, int64_t B, Span (&sp)[4])
{
    const size_t dv = (size_t)D * 4u;
    const size_t bdv = (size_t)B * (size_t)D * 4u;
    sp[0] = span(o.dgamma, dv);
    sp[1] = span(o.dbeta, kind == mn::MOD ? bdv : dv);
    sp[2] = span(o.dshift, bdv);
    sp[3] = span(o.dscalar, kind == mn::POLY ? 16u : 4u);
}

// `one_launch` (the full backward): for a small problem (mn::bwd_one_launch)
// the row launch adds the partial rows itself and writes dgamma (dbeta);
// *done says whether it did.
mn_status backward_rows(int kind, const BwdIn& b, int64_t N, int64_t D, const BwdTypes& t,
                        void* ws, size_t ws_bytes, const BwdOut& o, void* stream,
                        bool one_launch = false, bool* done = nullptr)
{
    if (!b.X || !b.dY || !b.dX) return MN_ERR_NULL;
    if (kind != mn::POLY && !b.gamma) return MN_ERR_NULL;
    if (kind != mn::DYT && !b.rstd) return MN_ERR_NULL;
    if (kind == mn::LN && !b.mean) return MN_ERR_NULL;
    if (kind == mn::ADD && !b.R) return MN_ERR_NULL;
    if (kind == mn::DYT && !b.alpha) return MN_ERR_NULL;
    if (kind == mn::POLY && !b.poly) return MN_ERR_NULL;
    if (kind == mn::MOD && !b.scale) return MN_ERR_NULL;
    if (!dtype_ok(t.st) || !dtype_ok(t.pdt) || !dtype_ok(t.ct) || !dtype_ok(t.ot) ||
        !mn::backward_types_supported(kind, t.st, t.ct, t.ot))
        return MN_ERR_DTYPE;
    if (!shape_ok(N, D) || !samples_ok(kind, b.B, N)) return MN_ERR_SHAPE;
    const int st = t.st;
    const size_t need = workspace_bytes(kind, N, D, b.B);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MN_ERR_WORKSPACE;

    const size_t es = (size_t)mn::stor_bytes(st);
    const size_t nd = (size_t)N * (size_t)D * es;
    const size_t ndc = (size_t)N * (size_t)D * (size_t)mn::stor_bytes(t.ct);
    const size_t ndo = (size_t)N * (size_t)D * (size_t)mn::stor_bytes(t.ot);
    const size_t dp = (size_t)D * (size_t)mn::stor_bytes(t.pdt);
    const size_t bd = (kind == mn::MOD) ? (size_t)b.B * (size_t)D * es : 0;
    const size_t nstat = (size_t)N * 4u * (kind == mn::POLY ? 3u : 1u);
    const Span in[] = {span(b.X, nd), span(b.R, nd), span(b.gamma, dp), span(b.dY, ndc),
                       span(b.dH, ndc), span(b.mean, (size_t)N * 4u), span(b.rstd, nstat),
                       span(b.alpha, 4), span(b.poly, 16), span(b.scale, bd)};
    Span ps[4];
    out_spans(kind, o, D, b.B, ps);
    const Span out[] = {span(b.dX, ndo), span(ws, need), ps[0], ps[1], ps[2], ps[3]};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;

    const bool vec_ok = chunks_fit(st, D) && aligned16(b.X) && aligned16(b.R) &&
                        aligned16(b.gamma) && aligned16(b.dY) && aligned16(b.dH) &&
                        aligned16(b.dX) && aligned16(b.scale);
    const mn::BwdPlan plan = mn::plan_backward(kind, st, N, (int32_t)D, vec_ok, b.B);
    float* w = static_cast<float*>(ws);
    const int64_t PD = plan.P * plan.Dp;
    const int nv = mn::bwd_vector_partials(kind);
    mn::BwdArgs a;
    a.X = b.X;
    a.R = b.R;
    a.gamma = b.gamma;
    a.dY = b.dY;
    a.dH = b.dH;
    a.mean = b.mean;
    a.rstd = b.rstd;
    a.alpha = b.alpha;
    a.poly = b.poly;
    a.scale = b.scale;
    a.dX = b.dX;
    a.part_g = nv > 0 ? w : nullptr;
    a.part_b = nv > 1 ? w + PD : nullptr;
    a.part_h = nv > 2 ? w + 2 * PD : nullptr;
    a.part_a = has_scalar_partials(kind) ? w + nv * PD : nullptr;
    a.N = N;
    a.S = (kind == mn::MOD) ? N / b.B : 0;
    a.D = (int32_t)D;
    a.Dp = plan.Dp;
    a.pdt = t.pdt;
    a.Pb = plan.Pb;
    a.sync = nullptr;
    a.dgamma = nullptr;
    a.dbeta = nullptr;
    one_launch = one_launch && mn::bwd_one_launch(kind, N, (int32_t)D) && plan.v.BLOCK < 1024;
    if (done) *done = one_launch;
    if (one_launch) {
        a.sync = reinterpret_cast<uint64_t*>(w + nv * PD);
        a.dgamma = o.dgamma;
        a.dbeta = kind == mn::LN ? o.dbeta : nullptr;
    }
    return device_status(
        mn::launch_backward_rows(kind, st, t.ct, t.ot, plan, a, as_stream(stream)));
}

// Stage 2 for every kind: the fixed-order column sums of the partial rows.
mn_status reduce_partials(int kind, int64_t N, int64_t D, int64_t B, const void* ws,
                          size_t ws_bytes, const BwdOut& o, void* stream)
{
    if (kind < 0 || kind > mn::MOD) return MN_ERR_SHAPE;
    if (kind != mn::POLY && !o.dgamma) return MN_ERR_NULL;
    if ((kind == mn::LN || kind == mn::DYT || kind == mn::MOD) && !o.dbeta) return MN_ERR_NULL;
    if (kind == mn::MOD && !o.dshift) return MN_ERR_NULL;
    if (has_scalar_partials(kind) && !o.dscalar) return MN_ERR_NULL;
    if (!shape_ok(N, D) || !samples_ok(kind, B, N)) return MN_ERR_SHAPE;
    const size_t need = workspace_bytes(kind, N, D, B);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MN_ERR_WORKSPACE;
    Span ps[4];
    out_spans(kind, o, D, B, ps);
    const Span in[] = {span(ws, need)};
    const Span out[] = {ps[0], ps[1], ps[2], ps[3]};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;

    const int64_t P = partial_rows(kind, N, D, B);
    const int32_t Dp = mn::partial_stride((int32_t)D);
    const int64_t PD = P * Dp;
    const int nv = mn::bwd_vector_partials(kind);
    const float* w = static_cast<const float*>(ws);
    // every parameter gradient of the call in one launch, one plane each
    mn::ReduceArgs a{};
    auto add = [&](const float* part, float* out, int64_t rows, int32_t d, int32_t dp,
                   int32_t groups) {
        a.plane[a.planes++] = mn::ReducePlane{part, out, rows, d, dp, groups};
    };
    if (nv > 0) add(w, o.dgamma, P, (int32_t)D, Dp, 1);
    if (kind == mn::LN || kind == mn::DYT) add(w + PD, o.dbeta, P, (int32_t)D, Dp, 1);
    if (kind == mn::MOD) {
        // dscale and dshift: the partial rows of each sample's workgroups
        add(w + PD, o.dbeta, P / B, (int32_t)D, Dp, (int32_t)B);
        add(w + 2 * PD, o.dshift, P / B, (int32_t)D, Dp, (int32_t)B);
    }
    if (has_scalar_partials(kind)) add(w + nv * PD, o.dscalar, P, kind == mn::POLY ? 4 : 1, 4, 1);
    return device_status(mn::launch_reduce(a, as_stream(stream)));
}

const BwdTypes kF16{MN_F16, MN_F16, MN_F16, MN_F16};

// ---------------------------------------------------------------------------
// Fused normalization + GEMV.
// ---------------------------------------------------------------------------

bool gemv_shape_ok(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || M > mn::kGemvMaxM || N < 1 || K < 1 || N > 64 * mn::kGemvCountWords) return false;
    return N <= INT32_MAX / 8 && K <= INT32_MAX / 8 && K <= (INT64_MAX / 8) / N;
}

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (!gemv_shape_ok(M, N, K)) return 0;
    // the largest slice count of any load path (16-byte, with or without the
    // matrix-core tiles, or element-wise)
    int64_t S = mn::plan_gemv(M, N, K, false, false, false).S;
    for (int f16 = 0; f16 < 2; ++f16)
        for (int ln = 0; ln < 2; ++ln) {
            const int64_t s = mn::plan_gemv(M, N, K, N % 8 == 0, f16, ln).S;
            S = s > S ? s : S;
        }
    // statistics, the tiles' arrival counters, then S slices of M + 2 partial
    // rows (LayerNorm's two extra)
    return sizeof(float) * ((size_t)mn::kGemvStatFloats + (size_t)mn::kGemvCountWords +
                            (size_t)S * (size_t)(M + 2) * (size_t)N);
}

mn_status norm_gemv(bool ln, const void* X, const void* gamma, const void* beta, const void* W,
                    void* Y, int64_t M, int64_t N, int64_t K, float eps, int st, int pdt,
                    void* ws, size_t ws_bytes, void* stream)
{
    if (!X || !gamma || !W || !Y || (ln && !beta)) return MN_ERR_NULL;
    if (!dtype_ok(st) || !dtype_ok(pdt) || st == MN_F32) return MN_ERR_DTYPE;
    if (!gemv_shape_ok(M, N, K)) return MN_ERR_SHAPE;
    if (!eps_ok(eps)) return MN_ERR_EPS;
    const size_t need = gemv_workspace_bytes(M, N, K);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MN_ERR_WORKSPACE;
    const size_t es = (size_t)mn::stor_bytes(st);
    const size_t kp = (size_t)K * (size_t)mn::stor_bytes(pdt);
    const Span in[] = {span(X, (size_t)M * K * es), span(gamma, kp), span(beta, kp),
                       span(W, (size_t)K * N * es)};
    const Span out[] = {span(Y, (size_t)M * N * es), span(ws, need)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;

    const bool vec_ok = N % 8 == 0 && aligned16(W);
    const mn::GemvPlan plan = mn::plan_gemv(M, N, K, vec_ok, st == MN_F16, ln);
    mn::GemvArgs a;
    a.X = X;
    a.gamma = gamma;
    a.beta = ln ? beta : nullptr;
    a.W = W;
    a.stats = static_cast<float*>(ws);
    a.cnt = reinterpret_cast<uint32_t*>(static_cast<float*>(ws) + mn::kGemvStatFloats);
    a.part = static_cast<float*>(ws) + mn::kGemvStatFloats + mn::kGemvCountWords;
    a.Y = Y;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.pdt = pdt;
    a.eps = eps;
    a.KB = plan.KB;
    a.S = plan.S;
    a.NB = plan.NB;
    return device_status(mn::launch_gemv(st, ln, plan, a, as_stream(stream)));
}

// ---------------------------------------------------------------------------
// GroupNorm.
// ---------------------------------------------------------------------------

int64_t gn_cp(int64_t C) { return (C + 3) / 4 * 4; }

bool gn_shape_ok(int64_t N, int64_t C, int64_t L, int64_t G)
{
    if (N < 1 || C < 1 || L < 1 || G < 1 || C % G != 0) return false;
    if (C > INT32_MAX / 4 || L > INT32_MAX) return false;
    return N <= (INT64_MAX / 4) / C / L;
}

size_t gn_workspace_bytes(int64_t N, int64_t C, int64_t L, int64_t G)
{
    if (!gn_shape_ok(N, C, L, G)) return 0;
    const int64_t f = mn::gn_workspace_floats(N, C, L, G);
    return f > 0 ? (size_t)f * sizeof(float) : 0;
}

bool gn_vec_ok(int st, int64_t L, const void* a, const void* b, const void* c = nullptr,
               const void* d = nullptr)
{
    return chunks_fit(st, L) && aligned16(a) && aligned16(b) && aligned16(c) && aligned16(d);
}

void gn_common(mn::GnArgs& a, const mn::GnPlan& plan, int64_t N, int64_t C, int64_t L,
               int64_t G)
{
    a.S = N * G;
    a.C = (int32_t)C;
    a.L = (int32_t)L;
    a.G = (int32_t)G;
    a.Cg = (int32_t)(C / G);
    a.Cp = (int32_t)gn_cp(C);
    if (plan.split) {
        a.units = plan.units;
        a.Kr = plan.Kr;
        a.UL = plan.UL;
        a.Kf = plan.Kf;
        a.FL = plan.FL;
    }
}

mn_status groupnorm_forward(const void* X, const void* gamma, const void* beta, void* Y,
                            float* mean, float* rstd, int64_t N, int64_t C, int64_t L, int64_t G,
                            float eps, int st, int pdt, void* stream)
{
    if (!X || !gamma || !beta || !Y || !mean || !rstd) return MN_ERR_NULL;
    if (!dtype_ok(st) || !dtype_ok(pdt)) return MN_ERR_DTYPE;
    if (!gn_shape_ok(N, C, L, G)) return MN_ERR_SHAPE;
    const bool vec = gn_vec_ok(st, L, X, Y);
    mn::GnPlan plan;
    if (!mn::plan_groupnorm(st, st, pdt, N, C, L, G, vec, true, plan)) return MN_ERR_SHAPE;
    if (!eps_ok(eps)) return MN_ERR_EPS;
    const size_t es = (size_t)mn::stor_bytes(st), ps = (size_t)mn::stor_bytes(pdt);
    const size_t nx = (size_t)N * (size_t)C * (size_t)L;
    const Span in[] = {span(X, nx * es), span(gamma, (size_t)C * ps), span(beta, (size_t)C * ps)};
    const Span out[] = {span(Y, nx * es), span(mean, (size_t)(N * G) * 4),
                        span(rstd, (size_t)(N * G) * 4)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;
    mn::GnArgs a{};
    a.X = X;
    a.gamma = gamma;
    a.beta = beta;
    a.Y = Y;
    a.mean = mean;
    a.rstd = rstd;
    a.pdt = pdt;
    a.eps = eps;
    gn_common(a, plan, N, C, L, G);
    if (plan.split) {
        // the chunk statistics go into Y (16-byte aligned within it) until
        // the apply pass overwrites it
        const uintptr_t y = reinterpret_cast<uintptr_t>(Y);
        const uintptr_t st16 = (y + 15) & ~(uintptr_t)15;
        const size_t need = (size_t)(st16 - y) + 8 * (size_t)(N * G) * (size_t)plan.Kf;
        if (need > nx * es) return MN_ERR_SHAPE;
        a.stat = reinterpret_cast<float*>(st16);
    }
    return device_status(mn::launch_gn_fwd(st, plan, a, as_stream(stream)));
}

mn_status groupnorm_backward(const void* X, const void* gamma, const float* mean,
                             const float* rstd, const void* dY, void* dX, float* dgamma,
                             float* dbeta, int64_t N, int64_t C, int64_t L, int64_t G, int st,
                             int pdt, int ot, void* ws, size_t ws_bytes, void* stream)
{
    if (!X || !gamma || !mean || !rstd || !dY || !dX || !dgamma || !dbeta) return MN_ERR_NULL;
    if (!dtype_ok(st) || !dtype_ok(pdt) || !(ot == st || ot == MN_F32)) return MN_ERR_DTYPE;
    if (!gn_shape_ok(N, C, L, G)) return MN_ERR_SHAPE;
    const bool vec = gn_vec_ok(st, L, X, dY, dX);
    mn::GnPlan plan;
    if (!mn::plan_groupnorm(st, ot, pdt, N, C, L, G, vec, false, plan)) return MN_ERR_SHAPE;
    const size_t need = gn_workspace_bytes(N, C, L, G);
    if (need == 0) return MN_ERR_SHAPE;
    if (!ws || ws_bytes < need || !aligned16(ws)) return MN_ERR_WORKSPACE;
    const size_t es = (size_t)mn::stor_bytes(st), ps = (size_t)mn::stor_bytes(pdt);
    const size_t os = (size_t)mn::stor_bytes(ot);
    const size_t nx = (size_t)N * (size_t)C * (size_t)L;
    const Span in[] = {span(X, nx * es), span(gamma, (size_t)C * ps),
                       span(mean, (size_t)(N * G) * 4), span(rstd, (size_t)(N * G) * 4),
                       span(dY, nx * es)};
    const Span out[] = {span(dX, nx * os), span(dgamma, (size_t)C * 4),
                        span(dbeta, (size_t)C * 4), span(ws, need)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;
    mn::GnArgs a{};
    a.X = X;
    a.gamma = gamma;
    a.dY = dY;
    a.dX = dX;
    a.mean = const_cast<float*>(mean);
    a.rstd = const_cast<float*>(rstd);
    gn_common(a, plan, N, C, L, G);
    // workspace: part_g, part_b [N][Cp]; then (split path) unit_p, unit_q
    // [N * C * Kr] and the slice sums [N * G][2]
    float* w = static_cast<float*>(ws);
    a.part_g = w;
    a.part_b = w + N * a.Cp;
    if (plan.split) {
        a.unit_p = w + 2 * N * a.Cp;
        a.unit_q = a.unit_p + plan.units;
        a.slice_ab = a.unit_q + plan.units;
    }
    a.pdt = pdt;
    hipStream_t s = as_stream(stream);
    hipError_t e = mn::launch_gn_bwd(st, ot, plan, a, s);
    if (e != hipSuccess) return device_status(e);
    // dgamma, dbeta: the N per-sample partial rows, added in fixed order
    mn::ReduceArgs r{};
    r.plane[0] = mn::ReducePlane{a.part_g, dgamma, N, (int32_t)C, a.Cp, 1};
    r.plane[1] = mn::ReducePlane{a.part_b, dbeta, N, (int32_t)C, a.Cp, 1};
    r.planes = 2;
    return device_status(mn::launch_reduce(r, s));
}

// GroupNorm over channels-last X [N][L][C]: the launch limits (grid y
// covers ceil(C / 256) channel blocks of the element-wise path, grid x the
// N * J position chunks) on top of the channels-first shape bounds.
bool gnl_shape_ok(int64_t N, int64_t L, int64_t C, int64_t G)
{
    if (!gn_shape_ok(N, C, L, G)) return false;
    if ((C + 255) / 256 > 65535) return false;
    return N * (int64_t)mn::gnl_chunks(N, L) <= (int64_t)UINT32_MAX && N * G <= (int64_t)UINT32_MAX;
}

size_t gnl_workspace_bytes(int64_t N, int64_t L, int64_t C, int64_t G)
{
    if (!gnl_shape_ok(N, L, C, G)) return 0;
    return (size_t)mn::gnl_workspace_floats(N, L, C, G) * sizeof(float);
}

void gnl_common(mn::GnlArgs& a, int st, bool vec_ok, int& vec, int64_t N, int64_t L, int64_t C,
                int64_t G, void* ws)
{
    a.N = N;
    a.L = (int32_t)L;
    a.C = (int32_t)C;
    a.G = (int32_t)G;
    a.Cg = (int32_t)(C / G);
    a.Cp = (int32_t)gn_cp(C);
    a.J = mn::gnl_chunks(N, L);
    mn::gnl_geometry(st, vec_ok, a, vec);
    // workspace: sa, sb [N][J][C]; then part_g, part_b [N][Cp]; ab [N * G][2]
    float* w = static_cast<float*>(ws);
    const int64_t njc = N * (int64_t)a.J * C;
    a.sa = w;
    a.sb = w + njc;
    a.part_g = w + 2 * njc;
    a.part_b = a.part_g + N * a.Cp;
    a.ab = a.part_b + N * a.Cp;
}

mn_status groupnorm_nlc_forward(const void* X, const void* gamma, const void* beta, void* Y,
                                float* mean, float* rstd, int64_t N, int64_t L, int64_t C,
                                int64_t G, float eps, int st, int pdt, void* ws, size_t ws_bytes,
                                void* stream)
{
    if (!X || !gamma || !beta || !Y || !mean || !rstd) return MN_ERR_NULL;
    if (!dtype_ok(st) || !dtype_ok(pdt)) return MN_ERR_DTYPE;
    if (!gnl_shape_ok(N, L, C, G)) return MN_ERR_SHAPE;
    if (!eps_ok(eps)) return MN_ERR_EPS;
    const size_t need = gnl_workspace_bytes(N, L, C, G);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MN_ERR_WORKSPACE;
    const size_t es = (size_t)mn::stor_bytes(st), ps = (size_t)mn::stor_bytes(pdt);
    const size_t nx = (size_t)N * (size_t)C * (size_t)L;
    const Span in[] = {span(X, nx * es), span(gamma, (size_t)C * ps), span(beta, (size_t)C * ps)};
    const Span out[] = {span(Y, nx * es), span(mean, (size_t)(N * G) * 4),
                        span(rstd, (size_t)(N * G) * 4), span(ws, need)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;
    mn::GnlArgs a{};
    a.X = X;
    a.gamma = gamma;
    a.beta = beta;
    a.Y = Y;
    a.mean = mean;
    a.rstd = rstd;
    a.pdt = pdt;
    a.eps = eps;
    int vec = 1;
    gnl_common(a, st,
               chunks_fit(st, C) && aligned16(X) && aligned16(Y) && aligned16(gamma) &&
                   aligned16(beta),
               vec, N, L, C, G, ws);
    return device_status(mn::launch_gnl_fwd(st, vec, a, as_stream(stream)));
}

mn_status groupnorm_nlc_backward(const void* X, const void* gamma, const float* mean,
                                 const float* rstd, const void* dY, void* dX, float* dgamma,
                                 float* dbeta, int64_t N, int64_t L, int64_t C, int64_t G, int st,
                                 int pdt, int ot, void* ws, size_t ws_bytes, void* stream)
{
    if (!X || !gamma || !mean || !rstd || !dY || !dX || !dgamma || !dbeta) return MN_ERR_NULL;
    if (!dtype_ok(st) || !dtype_ok(pdt) || !(ot == st || ot == MN_F32)) return MN_ERR_DTYPE;
    if (!gnl_shape_ok(N, L, C, G)) return MN_ERR_SHAPE;
    const size_t need = gnl_workspace_bytes(N, L, C, G);
    if (!ws || ws_bytes < need || !aligned16(ws)) return MN_ERR_WORKSPACE;
    const size_t es = (size_t)mn::stor_bytes(st), ps = (size_t)mn::stor_bytes(pdt);
    const size_t os = (size_t)mn::stor_bytes(ot);
    const size_t nx = (size_t)N * (size_t)C * (size_t)L;
    const Span in[] = {span(X, nx * es), span(gamma, (size_t)C * ps),
                       span(mean, (size_t)(N * G) * 4), span(rstd, (size_t)(N * G) * 4),
                       span(dY, nx * es)};
    const Span out[] = {span(dX, nx * os), span(dgamma, (size_t)C * 4),
                        span(dbeta, (size_t)C * 4), span(ws, need)};
    if (!alias_free(in, out)) return MN_ERR_ALIAS;
    mn::GnlArgs a{};
    a.X = X;
    a.gamma = gamma;
    a.dY = dY;
    a.dX = dX;
    a.mean = const_cast<float*>(mean);
    a.rstd = const_cast<float*>(rstd);
    a.pdt = pdt;
    int vec = 1;
    gnl_common(a, st,
               chunks_fit(st, C) && aligned16(X) && aligned16(dY) && aligned16(dX) &&
                   aligned16(gamma),
               vec, N, L, C, G, ws);
    hipStream_t s = as_stream(stream);
    hipError_t e = mn::launch_gnl_bwd(st, ot, vec, a, s);
    if (e != hipSuccess) return device_status(e);
    // dgamma, dbeta: the N per-sample partial rows, added in fixed order
    mn::ReduceArgs r{};
    r.plane[0] = mn::ReducePlane{a.part_g, dgamma, N, (int32_t)C, a.Cp, 1};
    r.plane[1] = mn::ReducePlane{a.part_b, dbeta, N, (int32_t)C, a.Cp, 1};
    r.planes = 2;
    return device_status(mn::launch_reduce(r, s));
}

mn_status backward(int kind, const BwdIn& b, const BwdOut& o, int64_t N, int64_t D,
                   const BwdTypes& t, void* ws, size_t ws_bytes, void* stream)
{
    if (kind != mn::POLY && !o.dgamma) return MN_ERR_NULL;
    if ((kind == mn::LN || kind == mn::DYT || kind == mn::MOD) && !o.dbeta) return MN_ERR_NULL;
    if (kind == mn::MOD && !o.dshift) return MN_ERR_NULL;
    if (has_scalar_partials(kind) && !o.dscalar) return MN_ERR_NULL;
    bool one = false;
    mn_status s = backward_rows(kind, b, N, D, t, ws, ws_bytes, o, stream, true, &one);
    if (s != MN_OK || one) return s;
    return reduce_partials(kind, N, D, b.B, ws, ws_bytes, o, stream);
}

}  // namespace

namespace {

FwdIn fwd_in(const void* X, const void* R, const void* gamma, const void* beta, void* H, void* Y,
             float* mean, float* rstd)
{
    FwdIn f;
    f.X = X;
    f.R = R;
    f.gamma = gamma;
    f.beta = beta;
    f.H = H;
    f.Y = Y;
    f.mean = mean;
    f.rstd = rstd;
    return f;
}

BwdIn bwd_in(const void* X, const void* R, const void* gamma, const void* dY, const void* dH,
             const float* mean, const float* rstd, void* dX)
{
    BwdIn b;
    b.X = X;
    b.R = R;
    b.gamma = gamma;
    b.dY = dY;
    b.dH = dH;
    b.mean = mean;
    b.rstd = rstd;
    b.dX = dX;
    return b;
}

BwdOut bwd_out(float* dgamma, float* dbeta = nullptr, float* dshift = nullptr,
               float* dscalar = nullptr)
{
    BwdOut o;
    o.dgamma = dgamma;
    o.dbeta = dbeta;
    o.dshift = dshift;
    o.dscalar = dscalar;
    return o;
}

}  // namespace

extern "C" {

// --- binary16 entry points ---------------------------------------------------


mn_status mn_rmsnorm_forward(const mn_f16* X, const mn_f16* gamma, mn_f16* Y, float* rstd,
                             int64_t N, int64_t D, float eps, void* stream)
{
    return forward(mn::RMS, fwd_in(X, nullptr, gamma, nullptr, nullptr, Y, nullptr, rstd), N, D,
                   eps, MN_F16, MN_F16, stream);
}

mn_status mn_layernorm_forward(const mn_f16* X, const mn_f16* gamma, const mn_f16* beta,
                               mn_f16* Y, float* mean, float* rstd, int64_t N, int64_t D,
                               float eps, void* stream)
{
    return forward(mn::LN, fwd_in(X, nullptr, gamma, beta, nullptr, Y, mean, rstd), N, D, eps,
                   MN_F16, MN_F16, stream);
}

mn_status mn_add_rmsnorm_forward(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                 mn_f16* H, mn_f16* Y, float* rstd, int64_t N, int64_t D,
                                 float eps, void* stream)
{
    return forward(mn::ADD, fwd_in(X, R, gamma, nullptr, H, Y, nullptr, rstd), N, D, eps, MN_F16,
                   MN_F16, stream);
}

mn_status mn_rmsnorm_backward(const mn_f16* X, const mn_f16* gamma, const float* rstd,
                              const mn_f16* dY, mn_f16* dX, float* dgamma, int64_t N, int64_t D,
                              void* workspace, size_t workspace_bytes, void* stream)
{
    return backward(mn::RMS, bwd_in(X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX),
                    bwd_out(dgamma), N, D, kF16, workspace, workspace_bytes, stream);
}

mn_status mn_layernorm_backward(const mn_f16* X, const mn_f16* gamma, const float* mean,
                                const float* rstd, const mn_f16* dY, mn_f16* dX, float* dgamma,
                                float* dbeta, int64_t N, int64_t D, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    return backward(mn::LN, bwd_in(X, nullptr, gamma, dY, nullptr, mean, rstd, dX),
                    bwd_out(dgamma, dbeta), N, D, kF16, workspace, workspace_bytes, stream);
}

mn_status mn_add_rmsnorm_backward(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                  const float* rstd, const mn_f16* dY, const mn_f16* dH,
                                  mn_f16* dX, float* dgamma, int64_t N, int64_t D,
                                  void* workspace, size_t workspace_bytes, void* stream)
{
    return backward(mn::ADD, bwd_in(X, R, gamma, dY, dH, nullptr, rstd, dX), bwd_out(dgamma), N,
                    D, kF16, workspace, workspace_bytes, stream);
}

mn_status mn_rmsnorm_backward_rows(const mn_f16* X, const mn_f16* gamma, const float* rstd,
                                   const mn_f16* dY, mn_f16* dX, int64_t N, int64_t D,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    return backward_rows(mn::RMS, bwd_in(X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX), N,
                         D, kF16, workspace, workspace_bytes, BwdOut(), stream);
}

mn_status mn_layernorm_backward_rows(const mn_f16* X, const mn_f16* gamma, const float* mean,
                                     const float* rstd, const mn_f16* dY, mn_f16* dX, int64_t N,
                                     int64_t D, void* workspace, size_t workspace_bytes,
                                     void* stream)
{
    return backward_rows(mn::LN, bwd_in(X, nullptr, gamma, dY, nullptr, mean, rstd, dX), N, D,
                         kF16, workspace, workspace_bytes, BwdOut(), stream);
}

mn_status mn_add_rmsnorm_backward_rows(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                       const float* rstd, const mn_f16* dY, const mn_f16* dH,
                                       mn_f16* dX, int64_t N, int64_t D, void* workspace,
                                       size_t workspace_bytes, void* stream)
{
    return backward_rows(mn::ADD, bwd_in(X, R, gamma, dY, dH, nullptr, rstd, dX), N, D, kF16,
                         workspace, workspace_bytes, BwdOut(), stream);
}

// --- entry points with explicit storage types --------------------------------

mn_status mn_rmsnorm_forward_ex(const void* X, const void* gamma, void* Y, float* rstd, int64_t N,
                                int64_t D, float eps, mn_dtype act, mn_dtype param, void* stream)
{
    return forward(mn::RMS, fwd_in(X, nullptr, gamma, nullptr, nullptr, Y, nullptr, rstd), N, D,
                   eps, act, param, stream);
}

mn_status mn_layernorm_forward_ex(const void* X, const void* gamma, const void* beta, void* Y,
                                  float* mean, float* rstd, int64_t N, int64_t D, float eps,
                                  mn_dtype act, mn_dtype param, void* stream)
{
    return forward(mn::LN, fwd_in(X, nullptr, gamma, beta, nullptr, Y, mean, rstd), N, D, eps,
                   act, param, stream);
}

mn_status mn_add_rmsnorm_forward_ex(const void* X, const void* R, const void* gamma, void* H,
                                    void* Y, float* rstd, int64_t N, int64_t D, float eps,
                                    mn_dtype act, mn_dtype param, void* stream)
{
    return forward(mn::ADD, fwd_in(X, R, gamma, nullptr, H, Y, nullptr, rstd), N, D, eps, act,
                   param, stream);
}

mn_status mn_rmsnorm_backward_ex(const void* X, const void* gamma, const float* rstd,
                                 const void* dY, void* dX, float* dgamma, int64_t N, int64_t D,
                                 mn_dtype act, mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                 void* workspace, size_t workspace_bytes, void* stream)
{
    return backward(mn::RMS, bwd_in(X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX),
                    bwd_out(dgamma), N, D, BwdTypes{act, param, cot, dxt}, workspace,
                    workspace_bytes, stream);
}

mn_status mn_layernorm_backward_ex(const void* X, const void* gamma, const float* mean,
                                   const float* rstd, const void* dY, void* dX, float* dgamma,
                                   float* dbeta, int64_t N, int64_t D, mn_dtype act,
                                   mn_dtype param, mn_dtype cot, mn_dtype dxt, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    return backward(mn::LN, bwd_in(X, nullptr, gamma, dY, nullptr, mean, rstd, dX),
                    bwd_out(dgamma, dbeta), N, D, BwdTypes{act, param, cot, dxt}, workspace,
                    workspace_bytes, stream);
}

mn_status mn_add_rmsnorm_backward_ex(const void* X, const void* R, const void* gamma,
                                     const float* rstd, const void* dY, const void* dH, void* dX,
                                     float* dgamma, int64_t N, int64_t D, mn_dtype act,
                                     mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                     void* workspace, size_t workspace_bytes, void* stream)
{
    return backward(mn::ADD, bwd_in(X, R, gamma, dY, dH, nullptr, rstd, dX), bwd_out(dgamma), N,
                    D, BwdTypes{act, param, cot, dxt}, workspace, workspace_bytes, stream);
}

mn_status mn_rmsnorm_backward_rows_ex(const void* X, const void* gamma, const float* rstd,
                                      const void* dY, void* dX, int64_t N, int64_t D,
                                      mn_dtype act, mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                      void* workspace, size_t workspace_bytes, void* stream)
{
    return backward_rows(mn::RMS, bwd_in(X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX), N,
                         D, BwdTypes{act, param, cot, dxt}, workspace, workspace_bytes, BwdOut(),
                         stream);
}

mn_status mn_layernorm_backward_rows_ex(const void* X, const void* gamma, const float* mean,
                                        const float* rstd, const void* dY, void* dX, int64_t N,
                                        int64_t D, mn_dtype act, mn_dtype param, mn_dtype cot,
                                        mn_dtype dxt, void* workspace, size_t workspace_bytes,
                                        void* stream)
{
    return backward_rows(mn::LN, bwd_in(X, nullptr, gamma, dY, nullptr, mean, rstd, dX), N, D,
                         BwdTypes{act, param, cot, dxt}, workspace, workspace_bytes, BwdOut(),
                         stream);
}

mn_status mn_add_rmsnorm_backward_rows_ex(const void* X, const void* R, const void* gamma,
                                          const float* rstd, const void* dY, const void* dH,
                                          void* dX, int64_t N, int64_t D, mn_dtype act,
                                          mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                          void* workspace, size_t workspace_bytes, void* stream)
{
    return backward_rows(mn::ADD, bwd_in(X, R, gamma, dY, dH, nullptr, rstd, dX), N, D,
                         BwdTypes{act, param, cot, dxt}, workspace, workspace_bytes, BwdOut(),
                         stream);
}

// --- the other row-wise norms ------------------------------------------------

mn_status mn_dyt_forward_ex(const void* X, const float* alpha, const void* gamma,
                            const void* beta, void* Y, int64_t N, int64_t D, mn_dtype act,
                            mn_dtype param, void* stream)
{
    FwdIn f = fwd_in(X, nullptr, gamma, beta, nullptr, Y, nullptr, nullptr);
    f.alpha = alpha;
    return forward(mn::DYT, f, N, D, 1.0f, act, param, stream);
}

mn_status mn_dyt_backward_ex(const void* X, const float* alpha, const void* gamma, const void* dY,
                             void* dX, float* dalpha, float* dgamma, float* dbeta, int64_t N,
                             int64_t D, mn_dtype act, mn_dtype param, mn_dtype dxt,
                             void* workspace, size_t workspace_bytes, void* stream)
{
    BwdIn b = bwd_in(X, nullptr, gamma, dY, nullptr, nullptr, nullptr, dX);
    b.alpha = alpha;
    return backward(mn::DYT, b, bwd_out(dgamma, dbeta, nullptr, dalpha), N, D,
                    BwdTypes{act, param, act, dxt}, workspace, workspace_bytes, stream);
}

mn_status mn_polynorm_forward_ex(const void* X, const float* params, void* Y, float* rstd,
                                 int64_t N, int64_t D, float eps, mn_dtype act, void* stream)
{
    FwdIn f = fwd_in(X, nullptr, nullptr, nullptr, nullptr, Y, nullptr, rstd);
    f.poly = params;
    return forward(mn::POLY, f, N, D, eps, act, MN_F32, stream);
}

mn_status mn_polynorm_backward_ex(const void* X, const float* params, const float* rstd,
                                  const void* dY, void* dX, float* dparams, int64_t N, int64_t D,
                                  mn_dtype act, mn_dtype dxt, void* workspace,
                                  size_t workspace_bytes, void* stream)
{
    BwdIn b = bwd_in(X, nullptr, nullptr, dY, nullptr, nullptr, rstd, dX);
    b.poly = params;
    return backward(mn::POLY, b, bwd_out(nullptr, nullptr, nullptr, dparams), N, D,
                    BwdTypes{act, MN_F32, act, dxt}, workspace, workspace_bytes, stream);
}

mn_status mn_mod_rmsnorm_forward_ex(const void* X, const void* gamma, const void* scale,
                                    const void* shift, void* Y, float* rstd, int64_t B,
                                    int64_t N, int64_t D, float eps, mn_dtype act, mn_dtype param,
                                    void* stream)
{
    FwdIn f = fwd_in(X, nullptr, gamma, nullptr, nullptr, Y, nullptr, rstd);
    f.scale = scale;
    f.shift = shift;
    f.B = B;
    return forward(mn::MOD, f, N, D, eps, act, param, stream);
}

mn_status mn_mod_rmsnorm_backward_ex(const void* X, const void* gamma, const void* scale,
                                     const float* rstd, const void* dY, void* dX, float* dgamma,
                                     float* dscale, float* dshift, int64_t B, int64_t N,
                                     int64_t D, mn_dtype act, mn_dtype param, mn_dtype dxt,
                                     void* workspace, size_t workspace_bytes, void* stream)
{
    BwdIn b = bwd_in(X, nullptr, gamma, dY, nullptr, nullptr, rstd, dX);
    b.scale = scale;
    b.B = B;
    return backward(mn::MOD, b, bwd_out(dgamma, dscale, dshift), N, D,
                    BwdTypes{act, param, act, dxt}, workspace, workspace_bytes, stream);
}

// --- GroupNorm ---------------------------------------------------------------

mn_status mn_groupnorm_forward_ex(const void* X, const void* gamma, const void* beta, void* Y,
                                  float* mean, float* rstd, int64_t N, int64_t C, int64_t L,
                                  int64_t G, float eps, mn_dtype act, mn_dtype param,
                                  void* stream)
{
    return groupnorm_forward(X, gamma, beta, Y, mean, rstd, N, C, L, G, eps, act, param, stream);
}

mn_status mn_groupnorm_backward_ex(const void* X, const void* gamma, const float* mean,
                                   const float* rstd, const void* dY, void* dX, float* dgamma,
                                   float* dbeta, int64_t N, int64_t C, int64_t L, int64_t G,
                                   mn_dtype act, mn_dtype param, mn_dtype dxt, void* workspace,
                                   size_t workspace_bytes, void* stream)
{
    return groupnorm_backward(X, gamma, mean, rstd, dY, dX, dgamma, dbeta, N, C, L, G, act,
                              param, dxt, workspace, workspace_bytes, stream);
}

size_t mn_groupnorm_workspace_bytes(int64_t N, int64_t C, int64_t L, int64_t G)
{
    return gn_workspace_bytes(N, C, L, G);
}

mn_status mn_groupnorm_nlc_forward_ex(const void* X, const void* gamma, const void* beta, void* Y,
                                      float* mean, float* rstd, int64_t N, int64_t L, int64_t C,
                                      int64_t G, float eps, mn_dtype act, mn_dtype param,
                                      void* workspace, size_t workspace_bytes, void* stream)
{
    return groupnorm_nlc_forward(X, gamma, beta, Y, mean, rstd, N, L, C, G, eps, act, param,
                                 workspace, workspace_bytes, stream);
}

mn_status mn_groupnorm_nlc_backward_ex(const void* X, const void* gamma, const float* mean,
                                       const float* rstd, const void* dY, void* dX,
                                       float* dgamma, float* dbeta, int64_t N, int64_t L,
                                       int64_t C, int64_t G, mn_dtype act, mn_dtype param,
                                       mn_dtype dxt, void* workspace, size_t workspace_bytes,
                                       void* stream)
{
    return groupnorm_nlc_backward(X, gamma, mean, rstd, dY, dX, dgamma, dbeta, N, L, C, G, act,
                                  param, dxt, workspace, workspace_bytes, stream);
}

size_t mn_groupnorm_nlc_workspace_bytes(int64_t N, int64_t L, int64_t C, int64_t G)
{
    return gnl_workspace_bytes(N, L, C, G);
}

// --- fused normalization + GEMV (inference) ---------------------------------

mn_status mn_fused_rmsnorm_gemv(const mn_f16* X, const mn_f16* gamma, const mn_f16* W, mn_f16* Y,
                                int64_t M, int64_t N, int64_t K, float eps, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    return norm_gemv(false, X, gamma, nullptr, W, Y, M, N, K, eps, MN_F16, MN_F16, workspace,
                     workspace_bytes, stream);
}

mn_status mn_fused_layernorm_gemv(const mn_f16* X, const mn_f16* gamma, const mn_f16* beta,
                                  const mn_f16* W, mn_f16* Y, int64_t M, int64_t N, int64_t K,
                                  float eps, void* workspace, size_t workspace_bytes,
                                  void* stream)
{
    return norm_gemv(true, X, gamma, beta, W, Y, M, N, K, eps, MN_F16, MN_F16, workspace,
                     workspace_bytes, stream);
}

mn_status mn_fused_rmsnorm_gemv_ex(const void* X, const void* gamma, const void* W, void* Y,
                                   int64_t M, int64_t N, int64_t K, float eps, mn_dtype act,
                                   mn_dtype param, void* workspace, size_t workspace_bytes,
                                   void* stream)
{
    return norm_gemv(false, X, gamma, nullptr, W, Y, M, N, K, eps, act, param, workspace,
                     workspace_bytes, stream);
}

mn_status mn_fused_layernorm_gemv_ex(const void* X, const void* gamma, const void* beta,
                                     const void* W, void* Y, int64_t M, int64_t N, int64_t K,
                                     float eps, mn_dtype act, mn_dtype param, void* workspace,
                                     size_t workspace_bytes, void* stream)
{
    return norm_gemv(true, X, gamma, beta, W, Y, M, N, K, eps, act, param, workspace,
                     workspace_bytes, stream);
}

size_t mn_norm_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    return gemv_workspace_bytes(M, N, K);
}

// --- workspace, stage 2, diagnostics ----------------------------------------

mn_status mn_norm_reduce_partials(mn_norm_kind kind, int64_t N, int64_t D, const void* workspace,
                                  size_t workspace_bytes, float* dgamma, float* dbeta,
                                  void* stream)
{
    // the split stages are exported for the training pair only
    if ((int)kind < 0 || (int)kind > mn::ADD) return MN_ERR_SHAPE;
    return reduce_partials((int)kind, N, D, 1, workspace, workspace_bytes,
                           bwd_out(dgamma, kind == MN_LAYERNORM ? dbeta : nullptr), stream);
}

size_t mn_norm_workspace_bytes(mn_norm_kind kind, int64_t N, int64_t D)
{
    if (kind == MN_MOD_RMSNORM) return 0;  // depends on the sample count
    return workspace_bytes((int)kind, N, D);
}

int mn_norm_backward_launches(mn_norm_kind kind, int64_t N, int64_t D)
{
    if (kind == MN_MOD_RMSNORM) return shape_ok(N, D) ? 2 : 0;
    if (workspace_bytes((int)kind, N, D) == 0) return 0;
    return mn::bwd_one_launch((int)kind, N, (int32_t)D) ? 1 : 2;
}

size_t mn_mod_rmsnorm_workspace_bytes(int64_t B, int64_t N, int64_t D)
{
    return workspace_bytes(mn::MOD, N, D, B);
}

const char* mn_status_string(mn_status s)
{
    switch (s) {
    case MN_OK: return "ok";
    case MN_ERR_NULL: return "a required pointer is NULL";
    case MN_ERR_SHAPE: return "shape out of range for this entry point (its declaration states the bounds)";
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
