"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/mn_norm.h declares, and rejects bad arguments
before touching the device (validation never dereferences the pointers, so
placeholder addresses are enough)."""
import ctypes
import os
import re
import subprocess

import pytest

import row_wise_normalization_amd as mn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mn_norm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mn.LIB_PATH),
                                reason="libmn_norm.so not built (run __graft_entry__.build())")


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(mn_\w+)\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("mn_rmsnorm_forward", "mn_rmsnorm_backward", "mn_layernorm_forward",
              "mn_layernorm_backward", "mn_add_rmsnorm_forward", "mn_add_rmsnorm_backward",
              "mn_norm_workspace_bytes", "mn_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", mn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s(mn_\w+)$", out, re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    L = mn.lib()
    for n in declared_functions():
        getattr(L, n)


def test_status_strings():
    L = mn.lib()
    for code in range(8):
        assert len(L.mn_status_string(code)) > 0
    assert L.mn_last_device_error() == b""


P = ctypes.c_void_p
A = P(0x100000)   # placeholder addresses far apart (never dereferenced)
B = P(0x20000000)
C = P(0x40000000)
Dp = P(0x60000000)
E = P(0x80000000)
F = P(0xA0000000)
G = P(0xC0000000)
NULL = None
S = None  # stream
C_ = P(0x50000000)
G_ = P(0x58000000)


def rms_fwd(X=A, g=B, Y=C, r=Dp, N=16, D=64, eps=1e-5):
    return mn.lib().mn_rmsnorm_forward(X, g, Y, r, N, D, ctypes.c_float(eps), S)


def test_forward_validation():
    assert rms_fwd(X=NULL) == 1
    assert rms_fwd(Y=NULL) == 1
    assert rms_fwd(r=NULL) == 1
    assert rms_fwd(N=0) == 2
    assert rms_fwd(N=-3) == 2
    assert rms_fwd(D=0) == 2
    assert rms_fwd(D=8193) == 2
    for eps in (0.0, -1e-5, float("nan"), float("inf")):
        assert rms_fwd(eps=eps) == 3, eps
    assert rms_fwd(Y=A) == 4                      # Y is X
    assert rms_fwd(Y=P(0x100000 + 16 * 64 * 2 - 2)) == 4   # Y overlaps X's last element
    assert rms_fwd(r=P(0x100000 + 64)) == 4       # rstd inside X
    assert rms_fwd(r=C) == 4                      # rstd overlaps Y
    L = mn.lib()
    f = ctypes.c_float(1e-5)
    assert L.mn_layernorm_forward(A, B, NULL, C, Dp, E, 4, 64, f, S) == 1
    assert L.mn_layernorm_forward(A, B, C, Dp, NULL, E, 4, 64, f, S) == 1
    assert L.mn_add_rmsnorm_forward(A, NULL, B, C, Dp, E, 4, 64, f, S) == 1
    assert L.mn_add_rmsnorm_forward(A, B, C, NULL, Dp, E, 4, 64, f, S) == 1
    assert L.mn_add_rmsnorm_forward(A, B, C, Dp, Dp, E, 4, 64, f, S) == 4  # H is Y


def test_backward_validation():
    L = mn.lib()
    N, D = 16, 64
    ws = mn.workspace_bytes(mn.MN_RMSNORM, N, D)
    W = P(0xE0000000)
    assert ws > 0
    call = lambda **k: L.mn_rmsnorm_backward(
        k.get("X", A), k.get("g", B), k.get("r", C), k.get("dY", Dp), k.get("dX", E),
        k.get("dg", F), k.get("N", N), k.get("D", D), k.get("W", W), k.get("ws", ws), S)
    assert call(dg=NULL) == 1
    assert call(r=NULL) == 1
    assert call(N=0) == 2
    assert call(D=9000) == 2
    assert call(W=NULL) == 5
    assert call(ws=ws - 1) == 5
    assert call(W=P(0xE0000004)) == 5             # not 16-byte aligned
    assert call(dX=A) == 4                        # dX is X
    assert call(dX=Dp) == 4                       # dX is dY
    assert call(dg=W) == 4                        # dgamma inside the workspace
    assert call(W=P(0x100000)) == 5 or call(W=P(0x100000)) == 4
    assert L.mn_layernorm_backward(A, B, NULL, C, Dp, E, F, G, N, D, W,
                                   mn.workspace_bytes(mn.MN_LAYERNORM, N, D), S) == 1
    assert L.mn_layernorm_backward(A, B, P(0x30000000), C, Dp, E, F, NULL, N, D, W,
                                   mn.workspace_bytes(mn.MN_LAYERNORM, N, D), S) == 1
    assert L.mn_add_rmsnorm_backward(A, NULL, B, C, Dp, NULL, E, F, N, D, W, ws, S) == 1
    assert L.mn_norm_reduce_partials(1, N, D, W, ws, F, NULL, S) == 1


def test_typed_entry_points_validate_storage_types():
    L = mn.lib()
    f = ctypes.c_float(1e-5)
    fwd = lambda act, par, **k: L.mn_rmsnorm_forward_ex(
        k.get("X", A), B, k.get("Y", C), Dp, k.get("N", 16), k.get("D", 64), f, act, par, S)
    for act in (mn.MN_F16, mn.MN_BF16, mn.MN_F32):
        for par in (mn.MN_F16, mn.MN_BF16, mn.MN_F32):
            assert fwd(act, par, N=0) == 2          # valid types reach the shape check
    for bad in (-1, 3, 7):
        assert fwd(bad, mn.MN_F16) == 7
        assert fwd(mn.MN_F16, bad) == 7
    # spans scale with the storage type: 16 x 64 float32 elements occupy 4096 bytes
    assert fwd(mn.MN_F32, mn.MN_F32, Y=P(0x100000 + 16 * 64 * 4 - 4)) == 4
    N, D = 16, 64
    W = P(0xE0000000)
    ws = mn.workspace_bytes(mn.MN_LAYERNORM, N, D)
    F16, BF16, F32 = mn.MN_F16, mn.MN_BF16, mn.MN_F32
    lnb = lambda act, par, cot, dxt, ws=ws: L.mn_layernorm_backward_ex(
        A, B, P(0x30000000), C, Dp, E, F, G, N, D, act, par, cot, dxt, W, ws, S)
    assert lnb(9, F16, F16, F16) == 7
    assert lnb(F16, 9, F16, F16) == 7
    assert lnb(F16, F16, -1, F16) == 7
    assert lnb(F16, F16, F16, 3) == 7
    # the backward storage combinations provided (act, cot, dxt); a valid
    # combination gets as far as the workspace check
    provided = {(a, c, o) for a in (F16, BF16) for c in (a, F32) for o in (a, F32)}
    provided |= {(F32, c, F32) for c in (F16, BF16, F32)}
    for act in (F16, BF16, F32):
        for cot in (F16, BF16, F32):
            for dxt in (F16, BF16, F32):
                want = 5 if (act, cot, dxt) in provided else 7
                assert lnb(act, BF16, cot, dxt, ws=0) == want, (act, cot, dxt)
    assert L.mn_add_rmsnorm_backward_ex(A, B, C, Dp, E, NULL, F, G, N, D, 1, 4, 1, 1, W, ws,
                                        S) == 7
    assert L.mn_add_rmsnorm_backward_rows_ex(A, B, C, Dp, E, NULL, F, N, D, 2, 2, 2, 2, W, 0,
                                             S) == 5
    assert L.mn_rmsnorm_backward_rows_ex(A, B, C, Dp, E, N, D, F16, F16, BF16, F16, W, 0, S) == 7
    assert L.mn_layernorm_forward_ex(A, B, NULL, C, Dp, E, N, D, f, 1, 1, S) == 1
    # dX spans scale with its own storage type: a float32 dX of 16 x 64 covers
    # 4096 bytes, so one starting 2 KiB before dY overlaps it
    assert L.mn_rmsnorm_backward_rows_ex(A, B, C, P(0x60000000), P(0x60000000 - 2048), N, D,
                                         F16, F16, F16, F32, W,
                                         mn.workspace_bytes(mn.MN_RMSNORM, N, D), S) == 4


def test_workspace_bytes():
    for kind in (mn.MN_RMSNORM, mn.MN_LAYERNORM, mn.MN_ADD_RMSNORM):
        assert mn.workspace_bytes(kind, 0, 64) == 0
        assert mn.workspace_bytes(kind, 4, 0) == 0
        assert mn.workspace_bytes(kind, 4, 8193) == 0
        for N, D in ((1, 1), (17, 257), (16384, 4096), (1048576, 128), (32768, 8192)):
            b = mn.workspace_bytes(kind, N, D)
            assert b > 0 and b % 16 == 0
            # at most 256 partial rows of round_up(D, 4) floats (two arrays for
            # LayerNorm), 512 for RMSNorm rows of up to 3072 columns; small
            # problems (N * Dp <= 131072) one partial row per eight rows (at
            # most 64) and the one-launch hand-off words (an epoch and 64
            # flags, 528 bytes)
            Dp = (D + 3) // 4 * 4
            small = N * Dp <= 131072
            P = min(1 << ((N + 7) // 8 - 1).bit_length(), 64) if small else min(
                N, 512 if kind == mn.MN_RMSNORM and D <= 3072 else 256)
            planes = 2 if kind == mn.MN_LAYERNORM else 1
            assert b == P * Dp * 4 * planes + (528 if small else 0)
    assert mn.workspace_bytes(6, 16, 64) == 0
    # the other norms: Dynamic Tanh keeps two partial arrays plus scalars,
    # PolyNorm only scalars, the Modulated RMSNorm sizes by its sample count
    for N, D in ((1, 1), (17, 257), (16384, 4096), (16384, 8192)):
        P = min(N, 256)
        Dp = (D + 3) // 4 * 4
        assert mn.workspace_bytes(mn.MN_DYT, N, D) == 2 * P * Dp * 4 + P * 16
        assert mn.workspace_bytes(mn.MN_POLYNORM, N, D) == min(N, 512 if D <= 4096 else 256) * 16
    assert mn.workspace_bytes(mn.MN_MOD_RMSNORM, 16, 64) == 0
    assert mn.mod_rmsnorm_workspace_bytes(4, 16, 64) == 4 * 4 * 64 * 4 * 3  # 4 per sample (S = 4)
    assert mn.mod_rmsnorm_workspace_bytes(8, 8192, 1024) == 8 * 32 * 1024 * 4 * 3
    assert mn.mod_rmsnorm_workspace_bytes(3, 16, 64) == 0      # 3 does not divide 16
    assert mn.mod_rmsnorm_workspace_bytes(0, 16, 64) == 0
    assert mn.mod_rmsnorm_workspace_bytes(4097, 4097, 64) == 0


def test_backward_launches():
    """One launch for small RMSNorm, LayerNorm and fused-add problems (at most
    131,072 partial values, rows of at most 5120 columns), else the row kernel
    and the column reduce."""
    pair = (mn.MN_RMSNORM, mn.MN_LAYERNORM, mn.MN_ADD_RMSNORM)
    for kind in pair:
        assert mn.backward_launches(kind, 17, 257) == 1
        assert mn.backward_launches(kind, 128, 1024) == 1       # exactly 131,072
        assert mn.backward_launches(kind, 129, 1024) == 2
        assert mn.backward_launches(kind, 25, 5120) == 1
        assert mn.backward_launches(kind, 16, 5121) == 2        # wider than 5120
        assert mn.backward_launches(kind, 1, 8192) == 2
        assert mn.backward_launches(kind, 16384, 4096) == 2
        assert mn.backward_launches(kind, 0, 64) == 0
        assert mn.backward_launches(kind, 4, 8193) == 0
    for kind in (mn.MN_DYT, mn.MN_POLYNORM, mn.MN_MOD_RMSNORM):
        assert mn.backward_launches(kind, 17, 257) == 2
    assert mn.backward_launches(6, 16, 64) == 0
    assert mn.backward_launches(-1, 16, 64) == 0


def test_other_norms_validation():
    L = mn.lib()
    f = ctypes.c_float(1e-5)
    F16, BF16, F32 = mn.MN_F16, mn.MN_BF16, mn.MN_F32
    N, D = 16, 64
    W = P(0xE0000000)
    a_ = P(0x30000000)
    # Dynamic Tanh: no epsilon; alpha, gamma, beta required
    assert L.mn_dyt_forward_ex(A, NULL, B, C, Dp, N, D, F16, F16, S) == 1
    assert L.mn_dyt_forward_ex(A, a_, B, NULL, Dp, N, D, F16, F16, S) == 1
    assert L.mn_dyt_forward_ex(A, a_, B, C, A, N, D, F16, F16, S) == 4          # Y is X
    assert L.mn_dyt_forward_ex(A, a_, B, C, Dp, N, D, F16, 5, S) == 7
    ws = mn.workspace_bytes(mn.MN_DYT, N, D)
    dyt_b = lambda act, dxt, ws=ws, da=G: L.mn_dyt_backward_ex(
        A, a_, B, C, Dp, da, E, F, N, D, act, F16, dxt, W, ws, S)
    assert dyt_b(F16, F16, da=NULL) == 1
    assert dyt_b(F16, BF16) == 7                     # dX must be act or binary32
    assert dyt_b(F32, F16) == 7
    assert dyt_b(F16, F32, ws=ws - 1) == 5
    assert dyt_b(BF16, BF16, ws=0) == 5
    assert dyt_b(F16, F16, da=E) == 4                # dalpha inside dgamma
    # PolyNorm: params and rstd required; eps checked
    assert L.mn_polynorm_forward_ex(A, NULL, B, C, N, D, f, F16, S) == 1
    assert L.mn_polynorm_forward_ex(A, a_, B, C, N, D, ctypes.c_float(0.0), F16, S) == 3
    assert L.mn_polynorm_forward_ex(A, a_, B, P(0x20000000 + N * D * 2 - 4), N, D, f, F16,
                                    S) == 4          # rstd [N][3] overlaps Y
    wsp = mn.workspace_bytes(mn.MN_POLYNORM, N, D)
    assert L.mn_polynorm_backward_ex(A, a_, C, Dp, E, NULL, N, D, F16, F16, W, wsp, S) == 1
    assert L.mn_polynorm_backward_ex(A, a_, C, Dp, E, F, N, D, F16, F16, W, wsp - 1, S) == 5
    # Modulated RMSNorm: B must divide N
    assert L.mn_mod_rmsnorm_forward_ex(A, B, C, NULL, Dp, E, 4, N, D, f, F16, F16, S) == 1
    assert L.mn_mod_rmsnorm_forward_ex(A, B, C, G, Dp, E, 3, N, D, f, F16, F16, S) == 2
    assert L.mn_mod_rmsnorm_forward_ex(A, B, C, G, Dp, E, 0, N, D, f, F16, F16, S) == 2
    wsm = mn.mod_rmsnorm_workspace_bytes(4, N, D)
    mod_b = lambda **k: L.mn_mod_rmsnorm_backward_ex(
        A, B, C, Dp, E, F, G, P(0x50000000), P(0x58000000), k.get("B", 4), N, D, F16, F16,
        k.get("dxt", F16), W, k.get("ws", wsm), S)
    assert mod_b(B=5) == 2
    assert mod_b(ws=wsm - 16) == 5
    assert mod_b(dxt=BF16) == 7


def test_groupnorm_validation_and_workspace():
    L_ = mn.lib()
    f = ctypes.c_float(1e-5)
    F16, BF16, F32 = mn.MN_F16, mn.MN_BF16, mn.MN_F32
    # per-sample partial rows of dgamma and dbeta (C rounded up to 4), the
    # split path's per-unit channel sums (units of at least 8192 values) and
    # its slice sums
    ws = lambda N, C, L, G: 2 * 4 * N * ((C + 3) // 4 * 4 + C * -(-L // 8192) + G)
    assert mn.groupnorm_workspace_bytes(32, 320, 4096, 32) == ws(32, 320, 4096, 32)
    assert mn.groupnorm_workspace_bytes(3, 10, 7, 5) == 2 * 4 * 3 * (12 + 10 + 5)
    assert mn.groupnorm_workspace_bytes(1, 128, 262144, 32) == 2 * 4 * (128 + 128 * 32 + 32)
    for bad in ((0, 8, 8, 1), (2, 0, 8, 1), (2, 8, 0, 1), (2, 8, 8, 0), (2, 8, 8, 3)):
        assert mn.groupnorm_workspace_bytes(*bad) == 0
    N, C, L, G = 2, 8, 64, 2
    mean, rstd = P(0x30000000), P(0x38000000)
    fwd = lambda X=A, g=B, b=C_, Y=Dp, N=N, C=C, L=L, G=G, eps=f, act=F16, par=F16: \
        L_.mn_groupnorm_forward_ex(X, g, b, Y, mean, rstd, N, C, L, G, eps, act, par, S)
    assert fwd(b=NULL) == 1 and fwd(Y=NULL) == 1
    assert fwd(G=3) == 2                        # 3 does not divide 8
    assert fwd(G=0) == 2 and fwd(N=0) == 2 and fwd(L=0) == 2
    assert fwd(L=1 << 30) == 2                  # rows of 2^30 values or more
    assert fwd(C=4096, L=1 << 20, G=1) == 2     # a slice of 2^32 values
    assert fwd(eps=ctypes.c_float(-1.0)) == 3
    assert fwd(Y=A) == 4                        # Y is X
    assert fwd(act=7) == 7 and fwd(par=9) == 7
    ws = mn.groupnorm_workspace_bytes(N, C, L, G)
    W = P(0xE0000000)
    bwd = lambda dxt=F16, act=F16, nb=ws, ws_=W, dX=E: L_.mn_groupnorm_backward_ex(
        A, B, mean, rstd, Dp, dX, F, G_, N, C, L, G, act, F16, dxt, ws_, nb, S)
    assert bwd(dxt=BF16) == 7                   # dX is the activation type or binary32
    assert bwd(act=F32, dxt=F16) == 7
    assert bwd(nb=ws - 4) == 5 and bwd(ws_=NULL) == 5
    assert bwd(dX=Dp) == 4                      # dX is dY


def test_fused_gemv_validation_and_workspace():
    L = mn.lib()
    f = ctypes.c_float(1e-5)
    F16, BF16, F32 = mn.MN_F16, mn.MN_BF16, mn.MN_F32
    # 64 floats of row statistics, 16384 arrival counters (one per column
    # tile, tiles at least 64 columns wide), then S slices of M + 2 fp32
    # partial rows; one tile per workgroup, K slices halve from 512 rows
    # until there are 256 tiles (192 for the wide 512-column tiles of one or
    # two X rows) or the slices reach 64 rows; S is the larger of the 16-byte
    # path (128-column or wide tiles) and the element-wise path (64-column
    # tiles)
    ws = lambda S, M, N: 4 * (64 + 16384 + S * (M + 2) * N)
    assert mn.norm_gemv_workspace_bytes(4, 4096, 4096) == ws(8, 4, 4096)
    assert mn.norm_gemv_workspace_bytes(4, 1024, 4096) == ws(32, 4, 1024)
    assert mn.norm_gemv_workspace_bytes(1, 14336, 4096) == ws(8, 1, 14336)
    assert mn.norm_gemv_workspace_bytes(4, 12288, 4096) == ws(8, 4, 12288)
    assert mn.norm_gemv_workspace_bytes(2, 7, 100) == ws(2, 2, 7)
    for bad in ((0, 8, 8), (9, 8, 8), (1, 0, 8), (1, 8, 0), (1, 64 * 16384 + 1, 8)):
        assert mn.norm_gemv_workspace_bytes(*bad) == 0
    assert mn.norm_gemv_workspace_bytes(1, 64 * 16384, 8) > 0
    M, N, K = 4, 64, 128
    ws = mn.norm_gemv_workspace_bytes(M, N, K)
    W = P(0xE0000000)
    rms = lambda X=A, g=B, Wt=C, Y=Dp, M=M, act=F16, par=F16, ws_=W, nb=ws, eps=f: \
        L.mn_fused_rmsnorm_gemv_ex(X, g, Wt, Y, M, N, K, eps, act, par, ws_, nb, S)
    assert rms(X=NULL) == 1 and rms(Wt=NULL) == 1 and rms(ws_=NULL) == 5
    assert rms(M=0) == 2 and rms(M=9) == 2
    assert rms(eps=ctypes.c_float(0.0)) == 3
    assert rms(Y=A) == 4                                   # Y is X
    assert rms(Y=P(0x40000000 + K * N * 2 - 2)) == 4        # Y overlaps W's last element
    assert rms(nb=ws - 4) == 5
    assert rms(act=F32) == 7 and rms(par=5) == 7
    assert L.mn_fused_layernorm_gemv_ex(A, B, NULL, C, Dp, M, N, K, f, F16, F16, W, ws, S) == 1
    assert L.mn_fused_layernorm_gemv(A, B, E, C, Dp, M, N, K, f, W, ws - 1, S) == 5
    assert L.mn_fused_rmsnorm_gemv(A, B, C, Dp, M, N, K, f, W, 0, S) == 5


def test_product_and_oracle_are_independent():
    """Neither side imports, includes or links the other."""
    pkg = os.path.join(ROOT, "row_wise_normalization_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    src = f.read()
                assert not re.search(r"\boracle\b|mn_oracle|mno_", src), f"{fn} refers to the oracle"
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith((".py", ".c", ".h")):
            with open(os.path.join(ROOT, "oracle", fn)) as f:
                src = f.read()
            assert "row_wise_normalization_amd" not in src and "mn_norm.h" not in src, fn


def test_noalloc_validation_and_scratch_size():
    """The no-allocation RMSNorm backward validates before touching a device,
    and its fixed scratch array holds the partial rows of every valid shape."""
    L = mn.lib()
    cap = mn.noalloc_scratch_bytes()
    assert cap == 8 << 20
    call = lambda **k: L.mn_rmsnorm_backward_noalloc(
        k.get("X", A), k.get("g", B), k.get("r", C), k.get("dY", Dp), k.get("dX", E),
        k.get("dg", F), k.get("N", 16), k.get("D", 64), S)
    assert call(X=NULL) == 1
    assert call(dg=NULL) == 1
    assert call(N=0) == 2
    assert call(D=0) == 2
    assert call(D=8193) == 2
    worst = 0
    for D in range(1, 8193):
        for N in (1, 255, 256, 511, 512, 513, 1 << 20):
            worst = max(worst, mn.workspace_bytes(mn.MN_RMSNORM, N, D))
    assert 0 < worst <= cap
