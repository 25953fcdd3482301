"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/sq.h, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest

import w8a8_int8_post_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(sq_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sq.LIB_PATH)
    names = _declared()
    assert {"sq_calibrate_absmax", "sq_smooth_fold", "sq_quant_weight_perchannel",
            "sq_quant_act_pertoken", "sq_w8a8_gemm_dequant"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), n


def test_version():
    assert "gfx950" in sq.version()


A = 4096  # a 16-byte aligned fake address: validation never dereferences


@pytest.fixture(scope="module")
def lib():
    return sq.load_library()


def test_null_pointers(lib):
    assert lib.sq_calibrate_absmax(None, 0, 4, 4, A, 0, None) == 1
    assert lib.sq_smooth_fold(A, A, 0, 4, 4, 0.5, None, A, None, None, None) == 1
    assert lib.sq_quant_weight_perchannel(A, 1, 4, 4, None, A, None) == 1
    assert lib.sq_quant_act_pertoken(A, 1, 4, 4, None, A, None, None) == 1
    assert lib.sq_w8a8_gemm_dequant(A, A, None, A, 4, 4, 16, A, 1, None) == 1
    assert lib.sq_w8a8_gemm_i32(A, A, 4, 4, 16, None, None) == 1
    assert lib.sq_smooth_activation(A, 1, 4, 4, None, A, None) == 1


@pytest.mark.parametrize("dims", [(0, 4), (4, 0), (-1, 4), (4, 4194305)])
def test_bad_shapes(lib, dims):
    a, b = dims
    assert lib.sq_calibrate_absmax(A, 0, a, b, A, 0, None) == 2
    assert lib.sq_quant_act_pertoken(A, 1, a, b, None, A, A, None) == 2
    assert lib.sq_quant_weight_perchannel(A, 1, a, b, A, A, None) == 2
    assert lib.sq_smooth_fold(A, A, 1, a, b, 0.5, A, A, None, None, None) == 2
    assert lib.sq_w8a8_gemm_dequant(A, A, A, A, a, b, 16, A, 1, None) == 2
    assert lib.sq_smooth_activation(A, 1, a, b, A, A, None) == 2


def test_k_overflow(lib):
    assert lib.sq_w8a8_gemm_i32(A, A, 4, 4, 133145, A, None) == 4
    assert lib.sq_w8a8_gemm_dequant(A, A, A, A, 4, 4, 133145, A, 1, None) == 4
    assert lib.sq_w8a8_gemm_i32(A, A, 4, 4, 0, A, None) == 2


def test_bad_dtype(lib):
    assert lib.sq_calibrate_absmax(A, 7, 4, 4, A, 0, None) == 3
    assert lib.sq_quant_act_pertoken(A, -1, 4, 4, None, A, A, None) == 3
    assert lib.sq_w8a8_gemm_dequant(A, A, A, A, 4, 4, 16, A, 3, None) == 3


def test_misaligned(lib):
    assert lib.sq_calibrate_absmax(A + 2, 1, 4, 4, A, 0, None) == 5
    assert lib.sq_w8a8_gemm_i32(A, A + 8, 4, 4, 16, A, None) == 5
    assert lib.sq_quant_act_pertoken(A, 1, 4, 4, A + 4, A, A, None) == 5


@pytest.mark.parametrize("alpha", [-0.1, 1.5, float("nan"), float("inf")])
def test_bad_alpha(lib, alpha):
    assert lib.sq_smooth_fold(A, A, 0, 4, 4, alpha, A, A, None, None, None) == 6


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 4, dtype=torch.float16)
    with pytest.raises(TypeError):
        sq.quant_act_pertoken(x)


def test_pertensor_entry_points_validate(lib):
    # argument order: x, xdt, M, K, smooth, step_in, xq, x_scale, stream
    assert lib.sq_quant_act_pertensor(None, 1, 4, 4, None, None, A, A, None) == 1
    assert lib.sq_quant_act_pertensor(A, 1, 0, 4, None, None, A, A, None) == 2
    assert lib.sq_quant_act_pertensor(A, 5, 4, 4, None, None, A, A, None) == 3
    assert lib.sq_quant_act_pertensor(A, 1, 4, 4, A + 4, None, A, A, None) == 5
    # a static step inside x_scale (x_scale = 8192, M = 4 floats) is refused
    assert lib.sq_quant_act_pertensor(A, 1, 4, 4, None, 8192 + 12, A, 8192, None) == 8
    assert lib.sq_static_act_step(A, None, 4, A, None) == 1
    assert lib.sq_static_act_step(A, A, 0, A, None) == 2
    assert lib.sq_quant_weight_pertensor(A, 1, 4, 4, None, A, None) == 1
    assert lib.sq_quant_weight_pertensor(A, 1, 4, -3, A, A, None) == 2
    assert lib.sq_quant_weight_pertensor(A, 9, 4, 4, A, A, None) == 3
    assert lib.sq_quant_weight_pertensor(A, 1, 4, 4, A, A + 2, None) == 5


def test_epilogue_entry_points_validate(lib):
    # sq_w8a8_gemm_dequant_ex(xq, sx, wq, sw, bias, act, M, N, K, y, ydt, stream)
    assert lib.sq_w8a8_gemm_dequant_ex(A, A, A, A, None, 2, 4, 4, 16, A, 1, None) == 9
    assert lib.sq_w8a8_gemm_dequant_ex(A, A, A, A, None, -1, 4, 4, 16, A, 1, None) == 9
    assert lib.sq_w8a8_gemm_dequant_ex(A, A, None, A, None, 0, 4, 4, 16, A, 1, None) == 1
    assert lib.sq_w8a8_gemm_dequant_ex(A, A, A, A, A + 4, 1, 4, 4, 16, A, 1, None) == 5
    assert lib.sq_w8a8_gemm_dequant_ex(A, A, A, A, None, 1, 4, 4, 16, A, 7, None) == 3
    assert lib.sq_w8a8_gemm_dequant_packed_ex(A, A, A, A, None, 1, 4, 4, 64, A, 1, None) == 2
    assert lib.sq_w8a8_gemm_dequant_packed_ex(A, A, A, A, None, 3, 4, 4, 128, A, 1, None) == 9
    # sq_fold_prev_linear(s, w_prev, wdt, Kp, K, w_out, bias, stream)
    assert lib.sq_fold_prev_linear(None, A, 0, 4, 4, A, None, None) == 1
    assert lib.sq_fold_prev_linear(A, A, 0, 0, 4, A, None, None) == 2
    assert lib.sq_fold_prev_linear(A, A, 4, 4, 4, A, None, None) == 3
    assert lib.sq_fold_prev_linear(A, A, 0, 4, 4, A, A + 8, None) == 5


def test_layernorm_quant_entry_point_validates(lib):
    import ctypes
    f = lib.sq_layernorm_quant_pertoken
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    B = 1 << 30  # fake, far-apart, aligned addresses: validation never dereferences
    ok = (B, 1, 4, 16, 2 * B, 3 * B, 1e-5, 4 * B, 5 * B, None, None)
    assert f(*ok[:4], None, *ok[5:]) == 1                       # null gamma
    assert f(ok[0], 1, 4, 70000, *ok[4:]) == 2                   # K beyond the register budget
    assert f(ok[0], 0, 4, 16385, *ok[4:]) == 2                   # fp32, K not a multiple of 4
    assert f(ok[0], 7, *ok[2:]) == 3
    assert f(*ok[:6], -1.0, *ok[7:]) == 10
    assert f(*ok[:6], float("nan"), *ok[7:]) == 10
    assert f(*ok[:6], float("inf"), *ok[7:]) == 10
    assert f(ok[0] + 2, *ok[1:]) == 5
    assert f(*ok[:7], ok[0], *ok[8:]) == 8                      # xq on top of x
    assert f(*ok[:9], 4 * B + 32, None) == 8                    # x_hat inside xq


def test_batched_entry_points_validate(lib):
    # sq_w8a8_bmm_dequant(xq, sx, wq, sw, batch, M, N, K, y, ydt, stream)
    assert lib.sq_w8a8_bmm_dequant(A, A, A, A, 0, 4, 4, 16, A, 1, None) == 2
    assert lib.sq_w8a8_bmm_dequant(A, A, A, A, 65536, 4, 4, 16, A, 1, None) == 2
    assert lib.sq_w8a8_bmm_dequant(A, A, A, A, 2, 4, 4, 200000, A, 1, None) == 4
    assert lib.sq_w8a8_bmm_dequant(A, None, A, A, 2, 4, 4, 16, A, 1, None) == 1
    assert lib.sq_w8a8_bmm_dequant(A, A, A, A, 2, 4, 4, 16, A, 9, None) == 3
    assert lib.sq_w8a8_bmm_dequant(A, A, A + 1, A, 2, 4, 4, 16, A, 1, None) == 5
    assert lib.sq_w8a8_bmm_i32(A, A, -1, 4, 4, 16, A, None) == 2
    assert lib.sq_w8a8_bmm_i32(A, A, 2, 4, 4, 16, A + 4, None) == 5
    # sq_quant_weight_perchannel_batched(w, wdt, batch, K, N, wq, sw, stream)
    assert lib.sq_quant_weight_perchannel_batched(A, 1, 0, 4, 4, A, A, None) == 2
    assert lib.sq_quant_weight_perchannel_batched(A, 5, 2, 4, 4, A, A, None) == 3
    assert lib.sq_quant_weight_perchannel_batched(None, 1, 2, 4, 4, A, A, None) == 1


def test_splitk_workspace_query_and_validation(lib):
    # no split for few tokens (the few-token kernels) or a wide layer at many tokens
    assert sq.sq_gemm_workspace_bytes(16, 4096, 16384) == 0
    assert sq.sq_gemm_workspace_bytes(4096, 16384, 4096) == 0
    # 128 tokens through a 16384 x 4096 layer: K split (64 tiles of 128 x 64,
    # 4 splits), int32 slices plus counters; 512 tokens (one tile per CU): the
    # plain kernel keeps up there, no split; 256 tokens on K = 28672: 2 splits
    need = sq.sq_gemm_workspace_bytes(128, 4096, 16384)
    assert need == 4 * 4096 + 4 * 4 * 128 * 4096
    assert sq.sq_gemm_workspace_bytes(512, 4096, 16384) == 0
    assert sq.sq_gemm_workspace_bytes(512, 4096, 28672) == 0
    assert sq.sq_gemm_workspace_bytes(256, 4096, 28672) == 4 * 4096 + 4 * 2 * 256 * 4096
    assert sq.sq_gemm_workspace_bytes(128, 4096, 8320) == 0    # K % 256 != 0
    assert sq.sq_gemm_workspace_bytes(128, 4096, 4096) == 0    # K < 8192
    assert lib.sq_gemm_workspace_bytes(0, 4, 4) == -1
    B = 1 << 32  # fake, far-apart, aligned addresses: validation never dereferences
    args = (B, 2 * B, 3 * B, 4 * B, 128, 4096, 16384, 5 * B, 1)
    f = lib.sq_w8a8_gemm_dequant_packed_ws
    assert f(*args, None, need, None) == 11           # workspace needed, none given
    assert f(*args, 6 * B + 8, need, None) == 11      # misaligned
    assert f(*args, 6 * B, need - 16, None) == 11     # too small
    assert f(*args, 5 * B + 4096, need, None) == 8    # overlaps y
    assert f(B, 2 * B, 3 * B, 4 * B, 128, 4096, 16064, 5 * B, 1, 6 * B, need, None) == 2
    g = lib.sq_w8a8_gemm_dequant_ws
    assert g(*args, None, need, None) == 11
    assert g(None, *args[1:], 6 * B, need, None) == 1


@pytest.mark.parametrize("M,N,K,splits", [
    (65, 4096, 16384, 4), (128, 1000, 8192, 4), (128, 1000, 12288, 4), (300, 4100, 8192, 1),
    (100, 4100, 12288, 2), (300, 1000, 28672, 4), (512, 4096, 16384, 1), (128, 4096, 16384, 4),
    (512, 4096, 28672, 1), (100, 8192, 28672, 2), (129, 2048, 9216, 4), (120, 2048, 13824, 2),
    (128, 1024, 16384, 8), (70, 300, 24576, 8), (128, 1000, 8320, 1), (100, 12288, 4096, 1),
    (16, 4096, 16384, 1), (200, 1002, 16384, 1), (65, 12288, 49152, 1), (256, 4096, 28672, 2),
    (65, 8192, 49152, 2), (65, 2048, 12288, 4)])
def test_splitk_split_counts(lib, M, N, K, splits):
    """The split the library takes on a 256-CU device (the count a host
    without a GPU assumes): the workspace holds the tile counters and
    `splits` int32 slices of M x N."""
    want = 0 if splits == 1 else 4 * 4096 + (4 * splits * M * N + 255) // 256 * 256
    assert sq.sq_gemm_workspace_bytes(M, N, K) == want


def test_noalloc_validation_and_scratch_bound(lib):
    """The allocation-free split-K entry point validates like the workspace
    form, and its static scratch holds the workspace of every split the
    library takes (tiles x splits <= the workgroup slots of a 256-CU GPU)."""
    B = 1 << 32
    f = lib.sq_w8a8_gemm_dequant_packed_noalloc
    assert f(None, 2 * B, 3 * B, 4 * B, 128, 4096, 16384, 5 * B, 1, None) == 1
    assert f(B, 2 * B, 3 * B, 4 * B, 128, 4096, 16064, 5 * B, 1, None) == 2   # K % 128
    assert f(B, 2 * B, 3 * B, 4 * B, 0, 4096, 16384, 5 * B, 1, None) == 2
    assert f(B, 2 * B, 3 * B, 4 * B, 128, 4096, 133248, 5 * B, 1, None) == 4
    assert f(B, 2 * B, 3 * B, 4 * B, 128, 4096, 16384, 5 * B, 7, None) == 3
    assert f(B, 2 * B, 3 * B + 8, 4 * B, 128, 4096, 16384, 5 * B, 1, None) == 5
    cap = sq.sq_noalloc_scratch_bytes()
    assert cap == 4 * 4096 + (8 << 20)
    worst = 0
    for M in list(range(65, 1025, 7)) + [128, 256, 512, 1024]:
        for N in (128, 1000, 2048, 4096, 4100, 5120, 8192, 12288, 16384, 28672):
            for K in (12288, 16384, 24576, 28672, 49152, 131072):
                worst = max(worst, sq.sq_gemm_workspace_bytes(M, N, K))
    assert 0 < worst <= cap, (worst, cap)


def test_linear_ws_query_and_validation(lib):
    """sq_w8a8_linear_packed_ws: the workspace need by shape, and every
    rejection before any HIP call (fake, aligned, distinct addresses)."""
    F16, F32 = 1, 0
    q = lib.sq_linear_workspace_bytes
    assert q(F16, 16, 8192, 28672) == 16 * 28672      # 13-16 tokens, >= 512 channel blocks
    assert q(F16, 13, 28672, 8192) == 16 * 8192
    assert q(F32, 16, 8192, 28672) == 16 * 28672
    assert q(F16, 12, 8192, 28672) == 0                # fewer tokens: the plain layer
    assert q(F16, 17, 8192, 28672) == 0
    assert q(F16, 16, 8176, 4096) == 0                 # 511 channel blocks
    assert q(F16, 16, 8177, 4096) == 16 * 4096
    assert q(F16, 16, 4096, 16384) == 16 * 16384       # narrower, but K >= 16384
    assert q(F16, 13, 16, 16384) == 16 * 16384
    assert q(F16, 16, 4096, 16256) == 0                # narrower and K < 16384
    assert q(F16, 12, 4096, 16384) == 0
    assert q(F32, 16, 8192, 131072) == 0               # row beyond the register-resident quantiser
    assert q(F16, 16, 8192, 4000) == -1 and q(F16, 0, 8192, 4096) == -1 and q(5, 16, 8192, 4096) == -1
    x, wp, sw, xq, sx, y, ws = (1 << 20) * 16, (2 << 20) * 16, (3 << 20) * 16, (4 << 20) * 16, \
        (5 << 20) * 16, (6 << 20) * 16, (7 << 20) * 16
    f = lib.sq_w8a8_linear_packed_ws
    need = 16 * 4096
    args = lambda **k: [k.get("x", x), 1, 16, 4096, wp, sw, 8192, k.get("xq", xq), sx,
                        k.get("y", y), 1, k.get("ws", ws), k.get("wb", need), None]
    assert f(*args(ws=None)) == 11
    assert f(*args(wb=need - 1)) == 11
    assert f(*args(ws=ws + 8)) == 11
    assert f(*args(x=None)) == 1
    assert f(*args(ws=xq + 1024)) == 8            # workspace inside xq
    assert f(*args(xq=x + 4096)) == 8             # codes over the activations
    assert f(*args(y=wp + 65536)) == 8            # output over the weights
    assert f(*args(ws=sx)) == 8
