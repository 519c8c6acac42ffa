/*
 * abi_check.c -- compiles against include/mn_norm.h as plain C (no HIP
 * headers), links libmn_norm.so and exercises the host-side validation paths,
 * which return before anything touches a GPU. Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mn_norm.h"

static int failures = 0;

#define EXPECT(expr, want)                                                        \
    do {                                                                          \
        mn_status got_ = (expr);                                                  \
        if (got_ != (want)) {                                                     \
            fprintf(stderr, "%s:%d: %s -> %d (%s), want %d\n", __FILE__, __LINE__, \
                    #expr, (int)got_, mn_status_string(got_), (int)(want));        \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

int main(void)
{
    /* placeholder device addresses, far apart; validation never dereferences */
    mn_f16* X = (mn_f16*)(uintptr_t)0x100000;
    mn_f16* G = (mn_f16*)(uintptr_t)0x20000000;
    mn_f16* Y = (mn_f16*)(uintptr_t)0x40000000;
    float* r = (float*)(uintptr_t)0x60000000;
    mn_f16* dY = (mn_f16*)(uintptr_t)0x80000000;
    mn_f16* dX = (mn_f16*)(uintptr_t)0xA0000000;
    float* dg = (float*)(uintptr_t)0xC0000000;
    void* ws = (void*)(uintptr_t)0xE0000000;
    const int64_t N = 64, D = 512;

    size_t need = mn_norm_workspace_bytes(MN_RMSNORM, N, D);
    if (need == 0 || need % 16 != 0) {
        fprintf(stderr, "workspace bytes %zu\n", need);
        ++failures;
    }
    /* a small problem: 8 partial rows (one per eight rows) of 512 floats,
       a second array for LayerNorm (the hand-off words come once) */
    if (mn_norm_workspace_bytes(MN_LAYERNORM, N, D) != need + 8 * 512 * 4) {
        fprintf(stderr, "LayerNorm workspace is not one more partial array\n");
        ++failures;
    }
    EXPECT(mn_rmsnorm_forward(NULL, G, Y, r, N, D, 1e-5f, NULL), MN_ERR_NULL);
    EXPECT(mn_rmsnorm_forward(X, G, Y, r, 0, D, 1e-5f, NULL), MN_ERR_SHAPE);
    EXPECT(mn_rmsnorm_forward(X, G, Y, r, N, MN_MAX_COLS + 1, 1e-5f, NULL), MN_ERR_SHAPE);
    EXPECT(mn_rmsnorm_forward(X, G, Y, r, N, D, -1.0f, NULL), MN_ERR_EPS);
    EXPECT(mn_rmsnorm_forward(X, G, X, r, N, D, 1e-5f, NULL), MN_ERR_ALIAS);
    EXPECT(mn_rmsnorm_backward(X, G, r, dY, dX, dg, N, D, ws, need - 16, NULL), MN_ERR_WORKSPACE);
    EXPECT(mn_rmsnorm_backward(X, G, r, dY, dY, dg, N, D, ws, need, NULL), MN_ERR_ALIAS);
    EXPECT(mn_layernorm_forward(X, G, NULL, Y, r, r + 4096, N, D, 1e-5f, NULL), MN_ERR_NULL);
    EXPECT(mn_add_rmsnorm_backward(X, NULL, G, r, dY, NULL, dX, dg, N, D, ws, need, NULL),
           MN_ERR_NULL);
    EXPECT(mn_norm_reduce_partials(MN_LAYERNORM, N, D, ws, 2 * need, dg, NULL, NULL), MN_ERR_NULL);
    /* explicit storage types */
    EXPECT(mn_rmsnorm_forward_ex(X, G, Y, r, N, D, 1e-5f, (mn_dtype)7, MN_F16, NULL),
           MN_ERR_DTYPE);
    EXPECT(mn_layernorm_backward_ex(X, G, r, r + 4096, dY, dX, dg, dg + 8192, N, D, MN_BF16,
                                    MN_F32, MN_F16, MN_BF16, ws, 2 * need, NULL),
           MN_ERR_DTYPE);
    EXPECT(mn_add_rmsnorm_forward_ex(X, dY, G, X, Y, r, N, D, 1e-5f, MN_F16, MN_F16, NULL),
           MN_ERR_ALIAS);
    /* the other norms, GroupNorm, the fused GEMV */
    EXPECT(mn_dyt_forward_ex(X, NULL, G, G, Y, N, D, MN_F16, MN_F16, NULL), MN_ERR_NULL);
    EXPECT(mn_polynorm_forward_ex(X, r, Y, r + 4096, N, D, 0.0f, MN_F16, NULL), MN_ERR_EPS);
    EXPECT(mn_mod_rmsnorm_forward_ex(X, G, dY, dX, Y, r, 3, N, D, 1e-5f, MN_F16, MN_F16, NULL),
           MN_ERR_SHAPE);
    EXPECT(mn_groupnorm_forward_ex(X, G, G + 4096, Y, r, r + 4096, 2, 64, 256, 7, 1e-5f, MN_F16,
                                   MN_F16, NULL),
           MN_ERR_SHAPE);
    if (mn_groupnorm_workspace_bytes(2, 64, 256, 8) == 0) ++failures;
    /* channels-last GroupNorm: groups must divide C; the workspace is checked */
    {
        const size_t gw = mn_groupnorm_nlc_workspace_bytes(2, 256, 64, 8);
        if (gw == 0 || gw % 16 != 0 || mn_groupnorm_nlc_workspace_bytes(2, 256, 64, 7) != 0)
            ++failures;
        EXPECT(mn_groupnorm_nlc_forward_ex(X, G, G + 4096, Y, r, r + 4096, 2, 256, 64, 7, 1e-5f,
                                           MN_F16, MN_F16, ws, gw, NULL),
               MN_ERR_SHAPE);
        EXPECT(mn_groupnorm_nlc_forward_ex(X, G, G + 4096, Y, r, r + 4096, 2, 256, 64, 8, 1e-5f,
                                           MN_F16, MN_F16, ws, gw - 16, NULL),
               MN_ERR_WORKSPACE);
        EXPECT(mn_groupnorm_nlc_backward_ex(X, G, r, r + 4096, dY, dY, dg, dg + 8192, 2, 256, 64,
                                            8, MN_F16, MN_F16, MN_F16, ws, gw, NULL),
               MN_ERR_ALIAS);
    }
    if (mn_norm_gemv_workspace_bytes(4, 4096, 4096) == 0) ++failures;
    EXPECT(mn_fused_rmsnorm_gemv(X, G, dY, Y, 9, 4096, 4096, 1e-5f, ws,
                                 mn_norm_gemv_workspace_bytes(4, 4096, 4096), NULL),
           MN_ERR_SHAPE);
    /* the no-allocation backward: argument errors before any device call */
    EXPECT(mn_rmsnorm_backward_noalloc(X, G, r, dY, dX, NULL, N, D, NULL), MN_ERR_NULL);
    EXPECT(mn_rmsnorm_backward_noalloc(X, G, r, dY, dX, dg, N, 0, NULL), MN_ERR_SHAPE);
    if (mn_noalloc_scratch_bytes() < mn_norm_workspace_bytes(MN_RMSNORM, 1 << 20, 4096))
        ++failures;
    if (mn_norm_backward_launches(MN_LAYERNORM, 128, 1024) != 1) ++failures;
    if (mn_norm_backward_launches(MN_RMSNORM, N, D) != 1) ++failures;
    if (mn_norm_backward_launches(MN_RMSNORM, 16384, 4096) != 2) ++failures;
    if (strlen(mn_status_string(MN_ERR_DEVICE)) == 0) ++failures;
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
