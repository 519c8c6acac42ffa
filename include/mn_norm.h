/*
 * mn_norm.h -- C ABI of the MI355X (gfx950) row-wise normalization training
 * library: RMSNorm, LayerNorm and fused residual-add + RMSNorm, forward and
 * backward, over row-major [N, D] binary16 activations.
 *
 * Sources of the semantics (web pages, cited by title and section):
 *   [meTile]     "Kernel coverage and training scope", section "Exact native
 *                normalization contract": formulas, the unrounded fused sum,
 *                both cotangents of the fused add, bounds (positive rows,
 *                1..8192 columns, positive finite epsilon), FP32 statistics
 *                and parameter gradients, no accumulation into existing
 *                gradient buffers, no in-place mutation, deterministic
 *                parameter reduction without atomics.
 *   [tensorcore] "Training kernels", sections "RMSnorm -- Llama-style" and
 *                "LayerNorm -- standard": argument order (X, gamma, [beta],
 *                Y, saved statistics, N, D, eps), fp16 X/gamma/beta/Y/dY/dX,
 *                fp32 saved rstd/mean [N] and fp32 dgamma [D], status return.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a device pointer owned by the caller. The
 *     library allocates nothing and frees nothing.
 *   - Row-major, contiguous: element (i, j) of an [N, D] tensor is at i*D + j.
 *     gamma, beta, dgamma, dbeta are [D]; mean and rstd are [N].
 *   - mn_f16 is an IEEE binary16 bit pattern. Arithmetic inside is fp32;
 *     fp16 results are rounded to nearest, ties to even.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).
 *     Work is enqueued asynchronously; no call synchronizes the host.
 *   - Validation happens before anything is enqueued; on any error nothing
 *     is written and nothing is launched:
 *       MN_ERR_NULL      a required pointer is NULL
 *       MN_ERR_SHAPE     N < 1, D outside [1, MN_MAX_COLS], N * D * 8 beyond
 *                        INT64_MAX, or (forward) more than 2^31 - 1 tiles of
 *                        rows (a tile holds at least 4 rows)
 *       MN_ERR_EPS       eps is not a positive finite float
 *       MN_ERR_ALIAS     an output's byte range overlaps an input's or
 *                        another output's ([meTile]: no in-place mutation)
 *       MN_ERR_WORKSPACE workspace NULL, smaller than
 *                        mn_norm_workspace_bytes(), or not 16-byte aligned
 *       MN_ERR_DEVICE    the HIP runtime rejected a launch
 *       MN_ERR_DTYPE     a storage type outside mn_dtype, or a backward
 *                        combination the *_ex calls do not provide
 *   - Results are bitwise deterministic for a given (N, D), pointer
 *     alignment class and device: every reduction has a fixed order and no
 *     floating-point atomics are used.
 *   - Calls whose tensor pointers are all 16-byte aligned, with D % 8 == 0
 *     for 16-bit storage or D % 4 == 0 for binary32, take the 128-bit vector
 *     kernels; any other call takes the element-wise kernels (same formulas,
 *     different fp32 summation order).
 */
#ifndef MN_NORM_H
#define MN_NORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t mn_f16;

typedef enum {
    MN_OK = 0,
    MN_ERR_NULL = 1,
    MN_ERR_SHAPE = 2,
    MN_ERR_EPS = 3,
    MN_ERR_ALIAS = 4,
    MN_ERR_WORKSPACE = 5,
    MN_ERR_DEVICE = 6,
    MN_ERR_DTYPE = 7
} mn_status;

/* Storage types of the *_ex entry points. Arithmetic is fp32 for all.
 * mn_dtype and mn_norm_kind are plain 32-bit integers (the size of an enum
 * argument on every supported ABI) with named values, so that any value a
 * caller passes is well defined in the library and an unknown one returns
 * MN_ERR_DTYPE (MN_ERR_SHAPE, or 0 bytes, for an unknown kind). */
typedef int32_t mn_dtype;
enum {
    MN_F16 = 0,   /* IEEE binary16 */
    MN_BF16 = 1,  /* bfloat16: the upper 16 bits of an IEEE binary32 */
    MN_F32 = 2    /* IEEE binary32 */
};

typedef int32_t mn_norm_kind;
enum {
    MN_RMSNORM = 0,
    MN_LAYERNORM = 1,
    MN_ADD_RMSNORM = 2,
    MN_DYT = 3,          /* Dynamic Tanh */
    MN_POLYNORM = 4,
    MN_MOD_RMSNORM = 5   /* Modulated RMSNorm */
};

/* [meTile] contract bound: 1..8192 columns. */
#define MN_MAX_COLS 8192

/* ---------------------------------------------------------------------------
 * RMSNorm. [meTile] contract, rms_norm_forward; [tensorcore] RMSnorm Math:
 *   rstd[i] = 1 / sqrt(mean_j(X[i,j]^2) + eps)
 *   Y[i,j]  = fp16(X[i,j] * rstd[i] * gamma[j])
 * Inputs X [N,D], gamma [D]; outputs Y [N,D] fp16, rstd [N] fp32 (saved for
 * the backward).
 * ------------------------------------------------------------------------- */
mn_status mn_rmsnorm_forward(const mn_f16* X, const mn_f16* gamma, mn_f16* Y, float* rstd,
                             int64_t N, int64_t D, float eps, void* stream);

/* RMSNorm backward. [meTile] contract (the derivative of the exact formula,
 * evaluated with the forward's saved fp32 statistics); [tensorcore]
 * tc_rmsnorm_backward. With xhat = X*rstd and g = dY*gamma:
 *   dX[i,j]   = fp16(rstd[i] * (g[i,j] - xhat[i,j] * mean_j(g*xhat)))
 *   dgamma[j] = sum_i dY[i,j] * xhat[i,j]      (fp32, overwritten)
 * rstd is the forward's saved array; X and rstd must be unchanged since the
 * forward. dgamma is reduced in two fixed-order stages through `workspace`
 * (caller-owned device memory of at least
 * mn_norm_workspace_bytes(MN_RMSNORM, N, D) bytes, contents on entry
 * ignored, clobbered on exit). For small problems (N * round_up(D, 4) up
 * to 131,072, rows of up to 5120 columns) both stages run in one launch:
 * the last workgroup to finish
 * its partial row adds them all, in the same order as the second stage
 * (bitwise the same dgamma), found through an epoch and per-workgroup flags
 * kept at the end of the workspace. These words need no clearing: a
 * workgroup reduces early only if every flag not yet written already holds
 * the 64-bit epoch word + 1, which neither cleared memory nor the words left
 * by earlier calls of the same shape do. The same holds for the
 * LayerNorm and fused-add backwards and their typed (_ex) forms. */
mn_status mn_rmsnorm_backward(const mn_f16* X, const mn_f16* gamma, const float* rstd,
                              const mn_f16* dY, mn_f16* dX, float* dgamma,
                              int64_t N, int64_t D, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ---------------------------------------------------------------------------
 * LayerNorm. [meTile] contract, layer_norm_forward (centre by the mean, then
 * the population variance of the centred values); [tensorcore] LayerNorm:
 *   mean[i] = sum_j X[i,j] / D
 *   rstd[i] = 1 / sqrt(sum_j (X[i,j] - mean[i])^2 / D + eps)
 *   Y[i,j]  = fp16((X[i,j] - mean[i]) * rstd[i] * gamma[j] + beta[j])
 * ------------------------------------------------------------------------- */
mn_status mn_layernorm_forward(const mn_f16* X, const mn_f16* gamma, const mn_f16* beta,
                               mn_f16* Y, float* mean, float* rstd,
                               int64_t N, int64_t D, float eps, void* stream);

/* LayerNorm backward ([meTile] contract: source, weight and bias gradients).
 * With xhat = (X - mean)*rstd and g = dY*gamma:
 *   dX[i,j]   = fp16(rstd[i] * (g - mean_j(g) - xhat * mean_j(g*xhat)))
 *   dgamma[j] = sum_i dY[i,j] * xhat[i,j];  dbeta[j] = sum_i dY[i,j]
 * Workspace: mn_norm_workspace_bytes(MN_LAYERNORM, N, D). */
mn_status mn_layernorm_backward(const mn_f16* X, const mn_f16* gamma, const float* mean,
                                const float* rstd, const mn_f16* dY, mn_f16* dX,
                                float* dgamma, float* dbeta, int64_t N, int64_t D,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Fused residual-add + RMSNorm. [meTile] contract, add_rms_norm_forward: the
 * sum s = X + R is formed in fp32 and normalised without rounding to fp16;
 * the sum rounded to fp16 is returned as H (the next residual stream):
 *   H[i,j]  = fp16(X[i,j] + R[i,j])        (exactly rounded binary16 sum)
 *   rstd[i] = 1 / sqrt(mean_j(s[i,j]^2) + eps)
 *   Y[i,j]  = fp16(s[i,j] * rstd[i] * gamma[j])
 * ------------------------------------------------------------------------- */
mn_status mn_add_rmsnorm_forward(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                 mn_f16* H, mn_f16* Y, float* rstd,
                                 int64_t N, int64_t D, float eps, void* stream);

/* Fused add backward with both output cotangents ([meTile] contract: the
 * residual-output cotangent is zero when absent, and its contribution goes
 * into both the source and the residual gradient). The gradient is taken at
 * the unrounded sum s = X + R, re-formed from X and R (H is not read):
 *   dX[i,j] = dR[i,j] = fp16(dH[i,j] + rstd*(g - shat * mean_j(g*shat)))
 * with shat = s*rstd, g = dY*gamma; dH == NULL means a zero cotangent. One
 * output array serves as both dX and dR.
 *   dgamma[j] = sum_i dY[i,j] * shat[i,j]
 * Workspace: mn_norm_workspace_bytes(MN_ADD_RMSNORM, N, D). */
mn_status mn_add_rmsnorm_backward(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                  const float* rstd, const mn_f16* dY, const mn_f16* dH,
                                  mn_f16* dX, float* dgamma, int64_t N, int64_t D,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Storage types beyond binary16. The [meTile] normalization contract lets
 * the source be FP16 or FP32 and lets weight, bias and cotangents each take
 * either type, with statistics, accumulation and every returned gradient in
 * FP32; this library adds bfloat16. The *_ex entry points take:
 *   act    storage of the activations X, R and of the forward outputs Y, H
 *   param  storage of gamma and beta (any of the three types)
 *   cot    storage of the cotangents dY, dH            (backward only)
 *   dxt    storage of dX (= dR)                       (backward only)
 * each MN_F16, MN_BF16 or MN_F32. Backward combinations (act, cot, dxt):
 *   act 16-bit (F16 or BF16): cot in {act, F32}, dxt in {act, F32};
 *   act F32: cot any of the three, dxt F32.
 * Anything else returns MN_ERR_DTYPE. Everything else -- formulas, saved
 * fp32 statistics, fp32 dgamma/dbeta, workspace, validation, determinism --
 * is exactly as for the binary16 calls above, which equal the *_ex calls
 * with every type MN_F16. Results in 16-bit storage are rounded to nearest,
 * ties to even; the fused add's H is the exact sum x + r rounded once to
 * `act`. Workspace sizes do not depend on the storage types. The 128-bit
 * vector kernels need D % 8 == 0 when `act` is 16-bit and D % 4 == 0 when it
 * is MN_F32 (and 16-byte aligned pointers).
 * ------------------------------------------------------------------------- */
mn_status mn_rmsnorm_forward_ex(const void* X, const void* gamma, void* Y, float* rstd,
                                int64_t N, int64_t D, float eps, mn_dtype act, mn_dtype param,
                                void* stream);
mn_status mn_rmsnorm_backward_ex(const void* X, const void* gamma, const float* rstd,
                                 const void* dY, void* dX, float* dgamma, int64_t N, int64_t D,
                                 mn_dtype act, mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                 void* workspace, size_t workspace_bytes, void* stream);
mn_status mn_layernorm_forward_ex(const void* X, const void* gamma, const void* beta, void* Y,
                                  float* mean, float* rstd, int64_t N, int64_t D, float eps,
                                  mn_dtype act, mn_dtype param, void* stream);
mn_status mn_layernorm_backward_ex(const void* X, const void* gamma, const float* mean,
                                   const float* rstd, const void* dY, void* dX, float* dgamma,
                                   float* dbeta, int64_t N, int64_t D, mn_dtype act,
                                   mn_dtype param, mn_dtype cot, mn_dtype dxt, void* workspace,
                                   size_t workspace_bytes, void* stream);
mn_status mn_add_rmsnorm_forward_ex(const void* X, const void* R, const void* gamma, void* H,
                                    void* Y, float* rstd, int64_t N, int64_t D, float eps,
                                    mn_dtype act, mn_dtype param, void* stream);
mn_status mn_add_rmsnorm_backward_ex(const void* X, const void* R, const void* gamma,
                                     const float* rstd, const void* dY, const void* dH, void* dX,
                                     float* dgamma, int64_t N, int64_t D, mn_dtype act,
                                     mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The other row-wise norms. The [meTile] coverage inventory (section
 * "Normalization", parity checklist) lists Modulated RMSNorm, PolyNorm and
 * Dynamic Tanh as missing there, naming the gradients each must return but
 * not the formulas; these calls implement the published definitions below.
 * Conventions are those of the *_ex calls above, except: the cotangent dY has
 * the activation type `act`; dX has `dxt`, which is `act` or MN_F32; every
 * parameter gradient is fp32 and is overwritten. Each backward runs its row
 * kernel and its fixed-order parameter reduction on `stream`.
 * ------------------------------------------------------------------------- */

/* Dynamic Tanh (Zhu et al., "Transformers without Normalization", 2025):
 *   Y[i,j] = gamma[j] * tanh(alpha * X[i,j]) + beta[j]
 * alpha is one fp32 scalar in device memory; gamma, beta are [D] of `param`.
 * No statistics are saved and there is no epsilon. Backward, with
 * t = tanh(alpha x):
 *   dX = dY * gamma * alpha * (1 - t^2)
 *   dalpha[0] = sum_{i,j} dY * gamma * x * (1 - t^2)
 *   dgamma[j] = sum_i dY * t,   dbeta[j] = sum_i dY
 * Workspace: mn_norm_workspace_bytes(MN_DYT, N, D). */
mn_status mn_dyt_forward_ex(const void* X, const float* alpha, const void* gamma,
                            const void* beta, void* Y, int64_t N, int64_t D, mn_dtype act,
                            mn_dtype param, void* stream);
mn_status mn_dyt_backward_ex(const void* X, const float* alpha, const void* gamma, const void* dY,
                             void* dX, float* dalpha, float* dgamma, float* dbeta, int64_t N,
                             int64_t D, mn_dtype act, mn_dtype param, mn_dtype dxt,
                             void* workspace, size_t workspace_bytes, void* stream);

/* PolyNorm (Zhuo et al., "Polynomial Composition Activations", 2024): the
 * RMS-normalised first three powers of each row, weighted, plus a bias,
 *   Y = w1 * n1 + w2 * n2 + w3 * n3 + b,   n_p = X^p * rstd_p,
 *   rstd_p = 1 / sqrt(mean_j(X^(2p)) + eps)   (per row).
 * params = {w1, w2, w3, b}: four fp32 scalars in device memory. rstd is
 * [N][3] fp32 (rstd_1, rstd_2, rstd_3 of each row), saved for the backward.
 * Backward (g = dY):
 *   dX = sum_p p * X^(p-1) * w_p * rstd_p * (g - n_p * mean_j(g * n_p))
 *   dparams = {sum g*n1, sum g*n2, sum g*n3, sum g} over all elements.
 * Workspace: mn_norm_workspace_bytes(MN_POLYNORM, N, D). */
mn_status mn_polynorm_forward_ex(const void* X, const float* params, void* Y, float* rstd,
                                 int64_t N, int64_t D, float eps, mn_dtype act, void* stream);
mn_status mn_polynorm_backward_ex(const void* X, const float* params, const float* rstd,
                                  const void* dY, void* dX, float* dparams, int64_t N, int64_t D,
                                  mn_dtype act, mn_dtype dxt, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Modulated RMSNorm: RMSNorm modulated per sample by a broadcast scale and
 * shift (the adaptive-norm modulation of conditioned transformers). The N
 * rows form B samples of S = N / B consecutive rows (B must divide N,
 * 1 <= B <= 4096); scale and shift are [B][D] of the activation type:
 *   Y[i,j] = gamma[j] * xhat[i,j] * (1 + scale[b,j]) + shift[b,j],
 *   xhat = X * rstd (RMSNorm, rstd [N] saved),  b = i / S.
 * Backward, with m = gamma * (1 + scale) the weight the row sees:
 *   dX = rstd * (dY*m - xhat * mean_j(dY*m*xhat))
 *   dgamma[j] = sum_i dY * xhat * (1 + scale[b,j])
 *   dscale[b,j] = sum_{i in b} dY * xhat * gamma[j]
 *   dshift[b,j] = sum_{i in b} dY            (dscale, dshift [B][D] fp32)
 * Workspace: mn_mod_rmsnorm_workspace_bytes(B, N, D). */
mn_status mn_mod_rmsnorm_forward_ex(const void* X, const void* gamma, const void* scale,
                                    const void* shift, void* Y, float* rstd, int64_t B,
                                    int64_t N, int64_t D, float eps, mn_dtype act, mn_dtype param,
                                    void* stream);
mn_status mn_mod_rmsnorm_backward_ex(const void* X, const void* gamma, const void* scale,
                                     const float* rstd, const void* dY, void* dX, float* dgamma,
                                     float* dscale, float* dshift, int64_t B, int64_t N,
                                     int64_t D, mn_dtype act, mn_dtype param, mn_dtype dxt,
                                     void* workspace, size_t workspace_bytes, void* stream);
size_t mn_mod_rmsnorm_workspace_bytes(int64_t B, int64_t N, int64_t D);

/* ---------------------------------------------------------------------------
 * GroupNorm. [meTile] "Normalization" lists GroupNorm among the missing
 * row-wise norms, with group/channel layouts and affine gradients; the
 * formula is the published one (Wu and He, "Group Normalization"):
 *   X, Y, dY, dX [N][C][L] (L positions per channel, contiguous), C = G * Cg;
 *   the (sample n, group g) slice is the Cg * L contiguous values of
 *   channels g*Cg .. g*Cg + Cg - 1 of sample n; mean and rstd [N][G] fp32
 *   (population variance, eps inside the square root, as LayerNorm);
 *   y = (x - mean) * rstd * gamma[c] + beta[c]  (gamma, beta [C] of `param`);
 *   dgamma[c] = sum over n, l of dY * xhat, dbeta[c] = sum of dY (fp32 [C]).
 * Storage: X, Y, dY in `act`; dX in `act` or MN_F32 (`dxt`). Any shape with
 * C % G == 0 and positive sizes is accepted (slices of up to 2^31 - 1 values,
 * L up to 2^30 - 1): a slice that fits one workgroup's registers is handled
 * by one kernel per direction; a larger one is split over many workgroups,
 * with its statistics (forward) or its channel and slice sums (backward)
 * combined in fixed order between launches. The split forward keeps its
 * per-chunk statistics in Y until it writes Y. The backward workspace
 * (mn_groupnorm_workspace_bytes(N, C, L, G) bytes, 16-byte aligned; no
 * initial contents needed) holds the per-sample fp32 partials of dgamma and
 * dbeta, added in fixed order by a second kernel, and the split path's
 * sums. Errors: MN_ERR_SHAPE for C % G != 0, zero sizes or sizes beyond
 * those bounds; otherwise as the row-wise norms.
 * ------------------------------------------------------------------------- */
mn_status mn_groupnorm_forward_ex(const void* X, const void* gamma, const void* beta, void* Y,
                                  float* mean, float* rstd, int64_t N, int64_t C, int64_t L,
                                  int64_t G, float eps, mn_dtype act, mn_dtype param,
                                  void* stream);
mn_status mn_groupnorm_backward_ex(const void* X, const void* gamma, const float* mean,
                                   const float* rstd, const void* dY, void* dX, float* dgamma,
                                   float* dbeta, int64_t N, int64_t C, int64_t L, int64_t G,
                                   mn_dtype act, mn_dtype param, mn_dtype dxt, void* workspace,
                                   size_t workspace_bytes, void* stream);
size_t mn_groupnorm_workspace_bytes(int64_t N, int64_t C, int64_t L, int64_t G);

/* ---------------------------------------------------------------------------
 * GroupNorm over channels-last activations. [meTile] "Normalization" asks
 * for GroupNorm's group and channel layouts; this is the same operation as
 * mn_groupnorm_*_ex (same groups, statistics, affine and gradients) over
 * X, Y, dY, dX [N][L][C]: the C channels of a position contiguous (the NHWC
 * layout of image activations), position l of channel c of sample n at
 * (n * L + l) * C + c. mean and rstd [N][G] fp32; gamma, beta [C] of `param`;
 * dgamma, dbeta [C] fp32; dX in `act` or MN_F32 (`dxt`).
 * Both directions take a workspace of mn_groupnorm_nlc_workspace_bytes(N, L,
 * C, G) bytes, 16-byte aligned, no initial contents needed: per-chunk
 * channel sums of the position chunks each workgroup streams, combined per
 * (sample, group) in fixed order by a second kernel (the forward's in
 * binary64, from sums shifted by each channel's value at position 0), then
 * an apply pass; the backward's per-sample dgamma and dbeta partials are
 * added in fixed order by the column-reduce kernel. X (and dY) are read
 * twice. Calls with C a multiple of 8 (binary32: 4) and every tensor
 * pointer 16-byte aligned take 16-byte chunks of channels; others go
 * channel by channel. Accepted shapes: those of mn_groupnorm_*_ex, with C
 * up to 16,776,960. Errors: as mn_groupnorm_*_ex, plus MN_ERR_WORKSPACE.
 * ------------------------------------------------------------------------- */
mn_status mn_groupnorm_nlc_forward_ex(const void* X, const void* gamma, const void* beta, void* Y,
                                      float* mean, float* rstd, int64_t N, int64_t L, int64_t C,
                                      int64_t G, float eps, mn_dtype act, mn_dtype param,
                                      void* workspace, size_t workspace_bytes, void* stream);
mn_status mn_groupnorm_nlc_backward_ex(const void* X, const void* gamma, const float* mean,
                                       const float* rstd, const void* dY, void* dX,
                                       float* dgamma, float* dbeta, int64_t N, int64_t L,
                                       int64_t C, int64_t G, mn_dtype act, mn_dtype param,
                                       mn_dtype dxt, void* workspace, size_t workspace_bytes,
                                       void* stream);
size_t mn_groupnorm_nlc_workspace_bytes(int64_t N, int64_t L, int64_t C, int64_t G);

/* ---------------------------------------------------------------------------
 * Fused normalization + GEMV for small inference batches. [tensorcore]
 * "Fused Norm + GEMV": Y = Norm(X, gamma[, beta]) @ W, the normalisation
 * applied in registers during the product instead of writing the normalised
 * rows out; the fused path returns no statistics and has no backward.
 *   X [M][K] (1 <= M <= 8), W [K][N] row-major, Y [M][N]: storage `act`
 *   (MN_F16 or MN_BF16); gamma, beta [K] of `param`; fp32 arithmetic.
 *   Norm is the RMSNorm or LayerNorm forward above over each row of X (the
 *   normalised rows are not rounded to a storage type); Y is rounded once.
 * The workspace (mn_norm_gemv_workspace_bytes(M, N, K), 16-byte aligned)
 * holds the row statistics, a fixed area of arrival counters (one per
 * column tile) and fp32 partial products over slices of K. It must be
 * zero-filled before its
 * first use and kept for this entry point (with any M, N, K): every call
 * leaves its counters at zero again, and the other words need no contents.
 * Calls that share a workspace must not overlap (one stream, or events
 * between streams). The sums over the slices run in ascending order,
 * whichever workgroup performs them, so Y is bitwise reproducible. The normalisation
 * is applied to the sums (rstd, and LayerNorm's mean through the column sums
 * of gamma*W and beta*W) rather than to each X element; the results agree
 * with the element-wise form to fp32 rounding. Validation as elsewhere (MN_ERR_SHAPE for M
 * outside [1, 8], N outside [1, 1048576] or K < 1).
 * ------------------------------------------------------------------------- */
mn_status mn_fused_rmsnorm_gemv(const mn_f16* X, const mn_f16* gamma, const mn_f16* W, mn_f16* Y,
                                int64_t M, int64_t N, int64_t K, float eps, void* workspace,
                                size_t workspace_bytes, void* stream);
mn_status mn_fused_layernorm_gemv(const mn_f16* X, const mn_f16* gamma, const mn_f16* beta,
                                  const mn_f16* W, mn_f16* Y, int64_t M, int64_t N, int64_t K,
                                  float eps, void* workspace, size_t workspace_bytes,
                                  void* stream);
mn_status mn_fused_rmsnorm_gemv_ex(const void* X, const void* gamma, const void* W, void* Y,
                                   int64_t M, int64_t N, int64_t K, float eps, mn_dtype act,
                                   mn_dtype param, void* workspace, size_t workspace_bytes,
                                   void* stream);
mn_status mn_fused_layernorm_gemv_ex(const void* X, const void* gamma, const void* beta,
                                     const void* W, void* Y, int64_t M, int64_t N, int64_t K,
                                     float eps, mn_dtype act, mn_dtype param, void* workspace,
                                     size_t workspace_bytes, void* stream);
size_t mn_norm_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* ---------------------------------------------------------------------------
 * Workspace and diagnostics.
 * ------------------------------------------------------------------------- */

/* Bytes of device workspace the backward of `kind` needs at (N, D): the
 * per-block fp32 parameter-gradient partials (two arrays for LayerNorm and
 * Dynamic Tanh, plus scalar partials for Dynamic Tanh and PolyNorm), and for
 * the one-launch backward of small RMSNorm, LayerNorm and fused-add
 * problems 528 bytes of hand-off words.
 * Depends only on (kind, N, D). Returns 0 for invalid arguments and for
 * MN_MOD_RMSNORM, whose size also depends on the sample count (see
 * mn_mod_rmsnorm_workspace_bytes). */
size_t mn_norm_workspace_bytes(mn_norm_kind kind, int64_t N, int64_t D);

/* Kernel launches of the full backward of `kind` at (N, D), for any storage
 * types and pointer alignment: 1 where the parameter-gradient reduction runs
 * inside the row launch (RMSNorm, LayerNorm and the fused add with
 * N * round_up(D, 4) <= 131,072 and D <= 5120), 2 otherwise (row kernel,
 * then the fixed-order column reduce); 0 for an invalid kind or shape. */
int mn_norm_backward_launches(mn_norm_kind kind, int64_t N, int64_t D);

/* Static description of a status code. */
const char* mn_status_string(mn_status s);

/* Text of the last HIP runtime error seen by this thread's MN_ERR_DEVICE
 * return ("" if none). */
const char* mn_last_device_error(void);

/* ---------------------------------------------------------------------------
 * The two stages of the training-pair backward calls, exported for callers
 * that schedule them separately (for instance to time the row kernel on its
 * own, or to overlap the parameter reduction with other work). Calling stage 1 then stage 2 on
 * the same stream with the same workspace is exactly the corresponding
 * mn_*_backward call.
 *
 * Stage 1 (row kernel): writes dX and the per-block fp32 partials of dgamma
 * (and dbeta) into `workspace`. Arguments and validation as the full call,
 * minus the gradient vectors. */
mn_status mn_rmsnorm_backward_rows(const mn_f16* X, const mn_f16* gamma, const float* rstd,
                                   const mn_f16* dY, mn_f16* dX, int64_t N, int64_t D,
                                   void* workspace, size_t workspace_bytes, void* stream);
mn_status mn_layernorm_backward_rows(const mn_f16* X, const mn_f16* gamma, const float* mean,
                                     const float* rstd, const mn_f16* dY, mn_f16* dX,
                                     int64_t N, int64_t D, void* workspace,
                                     size_t workspace_bytes, void* stream);
mn_status mn_add_rmsnorm_backward_rows(const mn_f16* X, const mn_f16* R, const mn_f16* gamma,
                                       const float* rstd, const mn_f16* dY, const mn_f16* dH,
                                       mn_f16* dX, int64_t N, int64_t D, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Stage 1 with explicit storage types (see the *_ex calls above). */
mn_status mn_rmsnorm_backward_rows_ex(const void* X, const void* gamma, const float* rstd,
                                      const void* dY, void* dX, int64_t N, int64_t D,
                                      mn_dtype act, mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                      void* workspace, size_t workspace_bytes, void* stream);
mn_status mn_layernorm_backward_rows_ex(const void* X, const void* gamma, const float* mean,
                                        const float* rstd, const void* dY, void* dX, int64_t N,
                                        int64_t D, mn_dtype act, mn_dtype param, mn_dtype cot,
                                        mn_dtype dxt, void* workspace, size_t workspace_bytes,
                                        void* stream);
mn_status mn_add_rmsnorm_backward_rows_ex(const void* X, const void* R, const void* gamma,
                                          const float* rstd, const void* dY, const void* dH,
                                          void* dX, int64_t N, int64_t D, mn_dtype act,
                                          mn_dtype param, mn_dtype cot, mn_dtype dxt,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2 (column reduce): dgamma[j] = sum over partial rows p of
 * partial[p][j] in a fixed order (dbeta likewise for LayerNorm; pass
 * dbeta = NULL otherwise). Overwrites dgamma/dbeta. `kind`, N and D must be
 * those of the stage-1 call that filled `workspace`. */
mn_status mn_norm_reduce_partials(mn_norm_kind kind, int64_t N, int64_t D,
                                  const void* workspace, size_t workspace_bytes,
                                  float* dgamma, float* dbeta, void* stream);

/* ---------------------------------------------------------------------------
 * RMSNorm backward without a caller workspace, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, validation, kernels and
 * results as mn_rmsnorm_backward (bitwise), minus `workspace`: the dgamma
 * partial rows (and, for small problems, the one-launch hand-off words) go
 * to a fixed array of mn_noalloc_scratch_bytes() bytes
 * (8 MiB, enough for every valid N, D) that the library holds on each
 * device it runs on until the process ends; a shape needing more would
 * return MN_ERR_WORKSPACE. The call allocates nothing. Its first call on a
 * device looks up that device's copy of the array (the device of `stream`,
 * or the current one for the null stream); a failure there returns
 * MN_ERR_DEVICE. All calls on one device share its array, so two such calls
 * that may run at the same time on one device (different streams without
 * ordering between them) race and give wrong dgamma: order them, or use the
 * workspace entry point. Nothing in the array needs clearing between calls.
 * ------------------------------------------------------------------------- */
mn_status mn_rmsnorm_backward_noalloc(const mn_f16* X, const mn_f16* gamma, const float* rstd,
                                      const mn_f16* dY, mn_f16* dX, float* dgamma,
                                      int64_t N, int64_t D, void* stream);
size_t mn_noalloc_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* MN_NORM_H */
