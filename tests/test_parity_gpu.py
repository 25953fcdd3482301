"""GPU parity: every C-ABI entry point against the CPU oracle.

Inputs are seeded and synthetic; GPU and oracle receive the same bits.  The
bar: codes, steps, accumulators, calibration maxima and folded weights are
bit-exact; the smoothing factor may differ by one fp32 ulp only where the
device and host double pow straddle an fp32 rounding boundary; 16-bit outputs
are within 1e-3 relative or one output ulp of the oracle's double value.
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_int8_post_amd as sq
from sqtest_util import assert_equal, assert_y_close, f32_ulp_diff, log, to_np

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _gpu(t, dev):
    return t.contiguous().to(dev)


# --------------------------------------------------------------- calibration

@pytest.mark.parametrize("T,K,dt", [(64, 512, "f32"), (37, 1000, "f16"), (33, 1001, "f16"),
                                    (512, 4096, "f16"), (100, 12288, "bf16"), (3, 7, "bf16"),
                                    (1, 1, "f32"), (2000, 96, "f32")])
def test_calibrate_absmax(ref, dev, T, K, dt):
    log("calibrate", T, K, dt)
    x1 = synth.random_matrix(T * 7 + K, T, K, dt, outlier_cols=[0, K // 2], factor=40.0)
    x2 = synth.random_matrix(T * 7 + K + 1, T, K, dt, outlier_cols=[K - 1], factor=90.0)
    a = sq.calibrate_absmax(_gpu(x1, dev))
    a = sq.calibrate_absmax(_gpu(x2, dev), a)  # running max over two batches
    torch.cuda.synchronize()
    r = ref.calibrate_absmax(x2, ref.calibrate_absmax(x1))
    assert_equal(a, r, "calibration absmax")


# --------------------------------------------------------------- smooth/fold

@pytest.mark.parametrize("K,N,dt", [(512, 512, "f32"), (300, 1000, "f16"), (77, 333, "bf16"),
                                    (1024, 4104, "bf16"), (5, 1, "f16")])
@pytest.mark.parametrize("alpha", [0.0, 0.4, 0.5, 0.6, 0.75, 1.0])
def test_smooth_fold(ref, dev, K, N, dt, alpha):
    log("smooth_fold", K, N, dt, alpha)
    xc = synth.random_matrix(K + 5, 64, K, "f32", outlier_cols=[1, K // 3], factor=60.0)
    a_np = ref.calibrate_absmax(xc)
    a_np[K // 2] = 0.0  # a silent channel takes s = 1
    w = synth.random_matrix(K * 3 + N, K, N, dt, scale=0.02)
    gamma, beta = synth.layernorm_params(synth.CONFIGS[1], "toy")
    gamma = torch.cat([gamma] * (K // 512 + 1))[:K].contiguous()
    beta = torch.cat([beta] * (K // 512 + 1))[:K].contiguous()
    g_gpu, b_gpu = _gpu(gamma, dev), _gpu(beta, dev)
    s, w_hat = sq.smooth_fold(_gpu(torch.from_numpy(a_np), dev), _gpu(w, dev), alpha, g_gpu, b_gpu)
    torch.cuda.synchronize()
    s_ref, w_hat_ref, g_ref, b_ref = ref.smooth_fold(a_np, w, alpha, gamma, beta)
    s_g = to_np(s)
    d = f32_ulp_diff(s_g, s_ref)
    assert d.max() <= 1, "s differs by %d ulp" % d.max()
    same = d == 0
    log("  s bit-equal fraction", same.mean())
    assert_equal(to_np(w_hat)[same], w_hat_ref[same], "W_hat rows with equal s")
    assert_equal(to_np(g_gpu)[same], g_ref[same], "gamma'")
    assert_equal(to_np(b_gpu)[same], b_ref[same], "beta'")
    if (~same).any():
        # an ulp-different s_j (the two double pow results straddle an fp32
        # rounding boundary) is the other admissible factor: the row is then
        # the oracle's fold with the GPU's s_j, bit for bit
        w_hat_alt = ref.fold_weight(w, s_g)
        g_alt, b_alt = ref.fold_norm(s_g, gamma, beta)
        assert_equal(to_np(w_hat)[~same], w_hat_alt[~same], "W_hat rows with the other s")
        assert_equal(to_np(g_gpu)[~same], g_alt[~same], "gamma' with the other s")
        assert_equal(to_np(b_gpu)[~same], b_alt[~same], "beta' with the other s")


# --------------------------------------------------------------- weight quant

@pytest.mark.parametrize("K,N,dt", [
    # one-pass kernel (K % 16 == 0, K <= 8192, N a multiple of 8 fp32 / 16 16-bit columns)
    (512, 512, "f32"), (4096, 1000, "f32"), (16, 16, "f16"), (528, 24, "f32"),
    (2064, 32, "f16"), (8192, 48, "bf16"), (4096, 4096, "f16"),
    # column maxima, then a transposing quantiser
    (77, 333, "f32"), (1000, 4096, "f16"), (130, 70, "bf16"), (1, 3, "f32"), (63, 65, "f16"),
    (8208, 16, "f16"), (512, 40, "f16")])
def test_quant_weight_perchannel(ref, dev, K, N, dt):
    log("quant_weight", K, N, dt)
    w = synth.random_matrix(K * 11 + N, K, N, dt, scale=0.02)
    w[:, N // 2] = 0  # an all-zero output channel: step 0, codes 0
    wq, sw = sq.quant_weight_perchannel(_gpu(w, dev))
    torch.cuda.synchronize()
    wq_r, sw_r = ref.quant_weight_perchannel(w)
    assert_equal(sw, sw_r, "w_scale")
    assert_equal(wq, wq_r, "wq")


# --------------------------------------------------------------- act quant

@pytest.mark.parametrize("M,K,dt", [(16, 512, "f32"), (2048, 4096, "f16"), (5, 16384, "f16"),
                                    # many short rows: 8, 16 or 32 lanes per row
                                    (1024, 64, "f16"), (700, 128, "f16"), (2048, 256, "bf16"),
                                    (512, 32, "f32"), (515, 16, "f16"), (4096, 128, "f16"),
                                    # one wave per row, 1, 2 or 4 pieces per lane
                                    (513, 512, "f16"), (600, 1024, "f32"), (1000, 2048, "f16"),
                                    (3, 49152, "bf16"), (4, 50000, "f16"), (9, 1001, "f16"),
                                    (300, 28672, "f16"), (1, 8, "bf16"), (7, 13, "f32"),
                                    (2, 24576, "f32"), (3, 24580, "f32"),
                                    # many rows: two waves of 4 pieces; 8 waves of 3
                                    # or 4; 16 waves of 6 or 8 (full and partial rows)
                                    (600, 4096, "bf16"), (513, 4000, "f16"),
                                    (520, 12288, "bf16"), (512, 12000, "f16"),
                                    (513, 16384, "f16"), (516, 12296, "bf16"),
                                    (512, 49152, "bf16"), (514, 50000, "f16"),
                                    (512, 6144, "f32"), (530, 24576, "f32")])
@pytest.mark.parametrize("smooth", [False, True])
def test_quant_act_pertoken(ref, dev, M, K, dt, smooth):
    log("act_quant", M, K, dt, smooth)
    x = synth.random_matrix(M * 13 + K, M, K, dt, outlier_cols=[0, K - 1, K // 2], factor=50.0)
    if M > 2:
        x[1] = 0  # an all-zero token: step 0, codes 0
    s_np = None
    s_gpu = None
    if smooth:
        s_np = np.exp(np.random.default_rng([3, K]).standard_normal(K)).astype(np.float32)
        s_gpu = _gpu(torch.from_numpy(s_np), dev)
    xq, sx = sq.quant_act_pertoken(_gpu(x, dev), s_gpu)
    torch.cuda.synchronize()
    xf = x.float().numpy()
    if smooth:
        xf = ref.smooth_activation(xf, s_np)
    xq_r, sx_r = ref.quant_act_pertoken(xf)
    assert_equal(sx, sx_r, "x_scale")
    assert_equal(xq, xq_r, "xq")


def test_quant_act_tiny_values(ref, dev):
    # steps in the subnormal range keep the same IEEE division semantics
    x = torch.from_numpy((np.random.default_rng(4).standard_normal((4, 64)) *
                          np.array([[1e-36], [1e-40], [3e-39], [1.0]])).astype(np.float32))
    xq, sx = sq.quant_act_pertoken(_gpu(x, dev))
    torch.cuda.synchronize()
    xq_r, sx_r = ref.quant_act_pertoken(x.numpy())
    assert_equal(sx, sx_r, "x_scale (tiny)")
    assert_equal(xq, xq_r, "xq (tiny)")


@pytest.mark.parametrize("M,K,dt", [(16, 512, "f32"), (33, 4096, "f16"), (5, 1001, "bf16"),
                                    (64, 12288, "bf16")])
def test_smooth_activation(ref, dev, M, K, dt):
    log("smooth_activation", M, K, dt)
    x = synth.random_matrix(M + K, M, K, dt, outlier_cols=[3], factor=40.0)
    s_np = np.exp(np.random.default_rng([5, K]).standard_normal(K)).astype(np.float32)
    xh = sq.smooth_activation(_gpu(x, dev), _gpu(torch.from_numpy(s_np), dev))
    torch.cuda.synchronize()
    r = torch.from_numpy(ref.smooth_activation(x, s_np)).to(DT[dt])  # round to the dtype
    assert_equal(xh.cpu().view(torch.int16 if dt != "f32" else torch.int32),
                 r.view(torch.int16 if dt != "f32" else torch.int32).numpy(), "x_hat bits")


# --------------------------------------------------------------- INT8 GEMM

GEMM_SHAPES = [
    (1, 1, 16), (1, 12288, 4096), (16, 512, 512), (3, 37, 77), (17, 4099, 4096),
    (64, 1000, 2000), (48, 64, 512), (33, 200, 1040),            # skinny kernel
    (65, 300, 1040), (300, 513, 2064), (70, 100, 100),
    (1000, 1000, 1008), (129, 255, 48),                          # register-staged tiles
    (512, 2048, 4096), (257, 256, 4096),                         # 128 x 128 DMA tiles
    (2048, 4096, 256),
    (2048, 12288, 256), (1999, 4100, 384),                       # 256 x 192 DMA tiles
    (2047, 16380, 640),                                          # 256 x 256 DMA tiles
    (300, 130, 128), (2000, 12300, 128), (65, 64, 128),          # K = 128: one operand stage
    (100, 4100, 4096), (128, 1000, 384), (65, 63, 16384),        # <= 128 rows: 128 x 64 tiles, BK 64
    (200, 1000, 2048), (256, 4100, 640), (129, 64, 256),         # <= 256 rows: 128 x 64 tiles, BK 128
    (40, 12288, 256), (33, 16384, 384), (64, 12300, 128),        # 17-64 rows on wide layers: tiles
    (32, 12288, 512), (17, 28672, 256), (31, 12288, 256),        # the edge of that rule (31: few-token)
    (70, 200, 16384), (130, 260, 16384),                         # deep: 64-deep k-tiles, four stages
    (200, 8010, 8192), (256, 4100, 16384),                       # few tiles, K >= 8192: two wave
    (512, 8192, 8192), (300, 8192, 8192),                        # groups over K (128 x 64; 128 x 128)
    (400, 12100, 4096), (100, 4100, 2048),                       # (128 x 192 in one round; K = 2048)
    (200, 4100, 8320), (65, 300, 2176),                          # few tiles, K % 256 != 0: 64-deep groups
    (130, 16400, 8192), (200, 20000, 8192), (160, 33000, 8192),  # 129-256 rows, wide and deep:
                                                                 # 256 x 128 ring, 256 x 128 (8 waves), 128 x 192
    (500, 12200, 384), (512, 12288, 256),                        # 128 x 192 tiles (one round)
    (500, 16300, 256), (2048, 4096, 512),                        # 256 x 128 tiles, eight waves
]


def _codes(M, N, K, seed):
    xq = synth.random_int8(seed, M, K)
    wq = synth.random_int8(seed + 1, N, K)
    xq[0, :] = 127
    wq[0, :] = 127
    if N > 1:
        wq[N - 1, :] = -127
    return xq, wq


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32(ref, dev, M, N, K):
    log("gemm_i32", M, N, K)
    xq, wq = _codes(M, N, K, M * 31 + N * 7 + K)
    acc = sq.w8a8_gemm_i32(_gpu(torch.from_numpy(xq), dev), _gpu(torch.from_numpy(wq), dev))
    torch.cuda.synchronize()
    assert_equal(acc, ref.gemm_i32(xq, wq), "acc")


def test_gemm_i32_worst_case(ref, dev):
    K = 133136  # largest multiple of 16 below the bound: all-extreme codes
    xq = np.full((2, K), 127, np.int8)
    xq[1] = -127
    wq = np.full((3, K), 127, np.int8)
    wq[1] = -127
    acc = sq.w8a8_gemm_i32(_gpu(torch.from_numpy(xq), dev), _gpu(torch.from_numpy(wq), dev))
    torch.cuda.synchronize()
    assert_equal(acc, ref.gemm_i32(xq, wq), "worst-case acc")
    assert int(to_np(acc)[0, 0]) == K * 127 * 127


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("ydt", ["f16", "bf16", "f32"])
def test_gemm_dequant(ref, dev, M, N, K, ydt):
    log("gemm_dequant", M, N, K, ydt)
    xq, wq = _codes(M, N, K, M * 17 + N * 5 + K)
    r = np.random.default_rng([M, N, K])
    sx = (r.uniform(0.01, 2.0, M) / 127).astype(np.float32)
    sw = (r.uniform(1e-4, 0.05, N) / 127).astype(np.float32)
    y = sq.w8a8_gemm_dequant(_gpu(torch.from_numpy(xq), dev), _gpu(torch.from_numpy(sx), dev),
                             _gpu(torch.from_numpy(wq), dev), _gpu(torch.from_numpy(sw), dev),
                             DT[ydt])
    torch.cuda.synchronize()
    acc_r = ref.gemm_i32(xq, wq)
    same = assert_y_close(y, ref.dequant(acc_r, sx, sw))
    log("  bit-equal to RNE(oracle):", same)
    _assert_fp32_order(y, ref, acc_r, sx, sw)


def _assert_fp32_order(y, ref, acc, sx, sw):
    """The scale back is RN(RN(fp32(acc) * sx) * sw) in fp32, then one rounding
    to y's dtype: bit-equal to the oracle's fp32 evaluation of that order."""
    y32 = torch.from_numpy(ref.dequant_bias_act_f32(acc, sx, sw)).to(y.dtype)
    bits = torch.int16 if y.dtype != torch.float32 else torch.int32
    assert_equal(y.cpu().view(bits), y32.view(bits).numpy(), "y (fp32 order, bits)")


# --------------------------------------------------------------- packed weights

def _pack_ref(wq):
    """The documented packed layout, re-laid out with numpy (no arithmetic)."""
    N, K = wq.shape
    NB, KG = (N + 15) // 16, K // 64
    pad = np.zeros((NB * 16, K), np.int8)
    pad[:N] = wq
    # [NB, 16 rows, KG, 4 subgroups, 16 bytes] -> [NB, KG, 4 subgroups, 16 rows, 16 bytes]
    t = pad.reshape(NB, 16, KG, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


@pytest.mark.parametrize("N,K", [(16, 128), (37, 256), (4099, 4096), (300, 1280)])
def test_pack_weight_layout(dev, N, K):
    wq = synth.random_int8(N + K, N, K)
    wp = sq.pack_weight(_gpu(torch.from_numpy(wq), dev))
    torch.cuda.synchronize()
    assert wp.numel() == sq.sq_packed_weight_bytes(N, K)
    assert_equal(wp, _pack_ref(wq), "packed weight bytes")


PACKED_SHAPES = [s for s in GEMM_SHAPES if s[2] % 128 == 0] + [
    (1, 4096, 16384), (16, 300, 128),
    # 4 to 16 tokens over 2 or 4 16-channel blocks per workgroup (ragged N too)
    (4, 8192, 256), (16, 12288, 512), (8, 12300, 1024), (5, 8200, 384), (16, 16384, 128),
    # 9 to 16 tokens on layers of more than 1024 blocks: 4 blocks per 4-wave workgroup
    (12, 20000, 1024), (16, 28672, 512), (9, 16400, 2048)]


@pytest.mark.parametrize("M,N,K", PACKED_SHAPES)
def test_gemm_packed(ref, dev, M, N, K):
    log("gemm_packed", M, N, K)
    xq, wq = _codes(M, N, K, M * 13 + N * 3 + K)
    r = np.random.default_rng([M, N, K, 1])
    sx = (r.uniform(0.01, 2.0, M) / 127).astype(np.float32)
    sw = (r.uniform(1e-4, 0.05, N) / 127).astype(np.float32)
    xq_d = _gpu(torch.from_numpy(xq), dev)
    wp = sq.pack_weight(_gpu(torch.from_numpy(wq), dev))
    sw_d = _gpu(torch.from_numpy(sw), dev)
    acc = sq.w8a8_gemm_i32_packed(xq_d, wp, N)
    y = sq.w8a8_gemm_dequant_packed(xq_d, _gpu(torch.from_numpy(sx), dev), wp, sw_d, torch.float16)
    torch.cuda.synchronize()
    acc_r = ref.gemm_i32(xq, wq)
    assert_equal(acc, acc_r, "acc (packed)")
    assert_y_close(y, ref.dequant(acc_r, sx, sw), "y (packed)")
    _assert_fp32_order(y, ref, acc_r, sx, sw)


# ------------------------------------------- whole run-time layer (packed)

LINEAR_CASES = [
    # M <= 2 and M * K <= 16384: one fused kernel (persistent over 16-channel blocks)
    (1, 37, 128, "f16", "f16"), (2, 4099, 4096, "bf16", "bf16"), (2, 300, 1024, "f32", "f32"),
    (1, 12288, 4096, "f16", "f16"), (1, 4096, 16384, "f16", "f32"), (2, 700, 8192, "bf16", "f16"),
    (1, 28672, 8192, "f16", "f16"), (2, 16400, 8192, "f32", "f32"),  # 4-wave workgroups
    # two launches: quantiser then the packed GEMM
    (1, 512, 28672, "bf16", "f16"), (2, 700, 16384, "f16", "f32"), (3, 300, 1024, "f32", "f32"),
    (4, 12288, 4096, "f16", "f16"), (5, 300, 1024, "f16", "f16"), (8, 300, 2048, "bf16", "f32"),
    (16, 4099, 2048, "f16", "f16"), (13, 1000, 2048, "f32", "bf16"),
    (4, 1000, 16384, "f16", "f32"), (4, 200, 16512, "f16", "f16"), (16, 200, 4096, "f16", "f16"),
    (17, 300, 1024, "f16", "f16"), (64, 600, 2048, "f16", "bf16"), (300, 513, 2048, "bf16", "f16"),
]


def _linear_check(ref, dev, x, wq, ydt):
    """sq_w8a8_linear_packed against the oracle and against the two-call path."""
    M, K = x.shape
    N = wq.shape[0]
    sw = (np.random.default_rng([M, N, K, 2]).uniform(1e-4, 0.05, N) / 127).astype(np.float32)
    x_d = _gpu(x, dev)
    wp = sq.pack_weight(_gpu(torch.from_numpy(wq), dev))
    sw_d = _gpu(torch.from_numpy(sw), dev)
    y, xq, sx = sq.linear_w8a8_packed(x_d, wp, sw_d, DT[ydt])
    xq2, sx2 = sq.quant_act_pertoken(x_d)
    y2 = sq.w8a8_gemm_dequant_packed(xq2, sx2, wp, sw_d, DT[ydt])
    torch.cuda.synchronize()
    xq_r, sx_r = ref.quant_act_pertoken(x if x.dtype != torch.float32 else x.numpy())
    assert_equal(xq, xq_r, "xq")
    assert_equal(sx, sx_r, "x_scale")
    acc_r = ref.gemm_i32(xq_r, wq)
    assert_y_close(y, ref.dequant(acc_r, sx_r, sw), "y")
    assert_equal(y.cpu().view(torch.int16 if ydt != "f32" else torch.int32),
                 y2.cpu().view(torch.int16 if ydt != "f32" else torch.int32).numpy(),
                 "y vs two-call path")


@pytest.mark.parametrize("M,N,K,xdt,ydt", LINEAR_CASES)
def test_linear_packed(ref, dev, M, N, K, xdt, ydt):
    log("linear_packed", M, N, K, xdt, ydt)
    x = synth.random_matrix(7 * M + K + N, M, K, xdt, outlier_cols=[1, K - 3], factor=30.0)
    _, wq = _codes(M, N, K, M * 5 + N * 7 + K)
    _linear_check(ref, dev, x, wq, ydt)


@pytest.mark.parametrize("M,pattern", [(2, (0.0, 1e-40)), (2, (1e31, 1.0)), (1, (1e-40,)),
                                       (4, (0.0, 1e-40, 1e31, 1.0)),
                                       (12, (0.0, 1e-40, 1e31, 1.0) * 3)])
def test_linear_packed_special_rows(ref, dev, M, pattern):
    # zero rows (step 0), subnormal steps, steps above 2^96 (IEEE division
    # path) and ordinary rows, through the fused kernel (M <= 2) and the
    # two-launch path.  1e31 puts the step above 2^96 while fp32(acc) * step
    # stays finite (the scale-back multiplies in fp32, the oracle in double).
    K = 256
    scale = np.array(pattern)[:, None]
    x = torch.from_numpy((np.random.default_rng(6 + M).standard_normal((M, K)) * scale)
                         .astype(np.float32))
    _, wq = _codes(M, 100, K, 11)
    _linear_check(ref, dev, x, wq, "f32")


# --------------------------------------------------------------- whole chain

@pytest.mark.parametrize("ydt", ["f16", "f32"])
def test_config_toy_chain(ref, dev, ydt):
    """Toy SmoothQuant linear (512 x 512, 16 tokens, 64 calibration tokens, 5
    outlier channels x40, alpha 0.5): every stage and the output."""
    cfg = synth.CONFIGS[1]
    xc = synth.activations(cfg, "toy", cfg.T, calibration=True)
    x = synth.activations(cfg, "toy", cfg.M[0])
    w = synth.weight(cfg, "toy")
    a = sq.calibrate_absmax(_gpu(xc, dev))
    s, w_hat = sq.smooth_fold(a, _gpu(w, dev), 0.5)
    wq, sw = sq.quant_weight_perchannel(w_hat)
    x_hat = sq.smooth_activation(_gpu(x, dev), s)
    y = sq.linear_w8a8(x_hat, wq, sw, DT[ydt])
    xq, sx = sq.quant_act_pertoken(x_hat)
    acc = sq.w8a8_gemm_i32(xq, wq)
    torch.cuda.synchronize()

    a_r = ref.calibrate_absmax(xc)
    assert_equal(a, a_r, "a")
    s_r, w_hat_r, _, _ = ref.smooth_fold(a_r, w, 0.5)
    assert_equal(s, s_r, "s")
    assert_equal(w_hat, w_hat_r, "W_hat")
    wq_r, sw_r = ref.quant_weight_perchannel(w_hat_r)
    assert_equal(wq, wq_r, "Wq")
    assert_equal(sw, sw_r, "sw")
    x_hat_r = ref.smooth_activation(x, s_r)
    assert_equal(x_hat, x_hat_r, "X_hat")
    xq_r, sx_r = ref.quant_act_pertoken(x_hat_r)
    assert_equal(xq, xq_r, "Xq")
    assert_equal(sx, sx_r, "sx")
    acc_r = ref.gemm_i32(xq_r, wq_r)
    assert_equal(acc, acc_r, "acc")
    y_r = ref.dequant(acc_r, sx_r, sw_r)
    assert_y_close(y, y_r)
    # SmoothQuant keeps the layer close to the float one on outlier inputs
    exact = x.double().numpy() @ w.double().numpy()
    rel = np.linalg.norm(to_np(y).astype(np.float64) - exact) / np.linalg.norm(exact)
    log("  relative error vs float XW:", rel)
    assert rel < 0.05
