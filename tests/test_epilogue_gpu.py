"""GPU parity for the rest of a linear layer: the scale back extended by a bias
and a ReLU (sq_w8a8_gemm_dequant_ex, sq_w8a8_gemm_dequant_packed_ex), and the
fold of a layer's smoothing factors into the linear layer before it
(sq_fold_prev_linear).

The extended scale back is RN(RN(fp32(acc) * sx) * sw + bias) with one rounding
for the multiply-add, then ReLU; the oracle evaluates the same fp32 operations
(dequant_bias_act_f32), so after the round to the output dtype the results are
compared bit for bit.  They are also checked against the oracle's double value:
within 1e-3 relative or one output ulp, plus 2^-22 |acc sx sw| for the two fp32
roundings ahead of the bias add (a bias can cancel most of the product).
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_int8_post_amd as sq
from sqtest_util import assert_equal, log, out_ulp, to_np

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
MODES = {"bias": (True, False), "relu": (False, True), "bias+relu": (True, True)}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _gpu(t, dev):
    if isinstance(t, np.ndarray):
        t = torch.from_numpy(t)
    return t.contiguous().to(dev)


def _case(M, N, K, seed):
    xq = synth.random_int8(seed, M, K)
    wq = synth.random_int8(seed + 1, N, K)
    r = np.random.default_rng([M, N, K, seed])
    sx = (r.uniform(0.01, 2.0, M) / 127).astype(np.float32)
    sw = (r.uniform(1e-4, 0.05, N) / 127).astype(np.float32)
    # a bias of the size of the products, so that ReLU cuts about half
    bias = (r.standard_normal(N) * 0.05 * np.sqrt(K)).astype(np.float32)
    return xq, wq, sx, sw, bias


def _check(y, ref, acc, sx, sw, bias, relu, what):
    """Bit-exact against the fp32 oracle rounded to y's dtype, and within the
    stated bound of the oracle's double value."""
    y32 = torch.from_numpy(ref.dequant_bias_act_f32(acc, sx, sw, bias, relu)).to(y.dtype)
    bits = torch.int16 if y.dtype != torch.float32 else torch.int32
    assert_equal(y.cpu().view(bits), y32.view(bits).numpy(), what + " (bits)")
    yd = ref.dequant_bias_act(acc, sx, sw, bias, relu)
    p = np.abs(ref.dequant(acc, sx, sw))
    g = to_np(y).astype(np.float64)
    rel = 1e-6 if y.dtype == torch.float32 else 1e-3
    diff = np.abs(g - yd)
    ok = (diff <= rel * np.abs(yd) + 2.0 ** -22 * p) | (diff <= out_ulp(yd, y.dtype) + 2.0 ** -22 * p)
    assert ok.all(), "%s: %d outside the bound" % (what, int((~ok).sum()))
    if relu:
        assert (g >= 0).all() and not np.signbit(g).any()


EX_SHAPES = [
    (1, 12288, 4096), (3, 37, 77), (48, 64, 512), (64, 1000, 2000),   # few-token kernels
    (65, 300, 1040), (1000, 1000, 1008), (129, 255, 48),             # register-staged tiles
    (512, 2048, 4096), (300, 130, 128),                              # 128 x 128 DMA tiles
    (2048, 12288, 256), (1999, 4100, 384),                           # 256 x 192 DMA tiles
    (2000, 12300, 128), (2047, 16380, 640),                          # 256 x 256
    (100, 300, 16384), (40, 12288, 256),                             # few-tile four-stage; wide 17-64
    (130, 16400, 8192), (200, 20000, 8192), (160, 33000, 8192),      # 129-256 rows, wide and deep
    (500, 12200, 384), (500, 16300, 256),                            # 128 x 192; 256 x 128 (8 waves)
    (200, 8010, 8192), (300, 8192, 8192), (400, 12100, 4096),        # two wave groups over K
    (200, 4100, 8320),                                               # the same, K % 256 != 0
]


@pytest.mark.parametrize("M,N,K", EX_SHAPES)
@pytest.mark.parametrize("ydt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mode", list(MODES))
def test_gemm_dequant_ex(ref, dev, M, N, K, ydt, mode):
    log("gemm_dequant_ex", M, N, K, ydt, mode)
    use_bias, relu = MODES[mode]
    xq, wq, sx, sw, bias = _case(M, N, K, M * 11 + N * 3 + K)
    b = bias if use_bias else None
    y = sq.w8a8_gemm_dequant_ex(_gpu(xq, dev), _gpu(sx, dev), _gpu(wq, dev), _gpu(sw, dev),
                                None if b is None else _gpu(b, dev),
                                sq.SQ_ACT_RELU if relu else sq.SQ_ACT_NONE, DT[ydt])
    torch.cuda.synchronize()
    _check(y, ref, ref.gemm_i32(xq, wq), sx, sw, b, relu, "y_ex")


PACKED_EX_SHAPES = [(1, 4096, 16384), (16, 300, 128), (33, 200, 1280), (64, 1000, 2048),
                    (300, 130, 128), (512, 2048, 4096), (2048, 12288, 256), (2000, 12300, 128),
                    (40, 12288, 256), (100, 300, 16384), (129, 8320, 16384),  # wide 17-64; deep
                    (130, 16400, 8192),  # 129-256 rows, wide and deep: 256 x 128 tiles
                    (16, 20000, 512)]    # 9-16 tokens, > 1024 blocks: 4-block 4-wave workgroups


@pytest.mark.parametrize("M,N,K", PACKED_EX_SHAPES)
@pytest.mark.parametrize("ydt", ["f16", "bf16"])
@pytest.mark.parametrize("mode", ["bias", "bias+relu"])
def test_gemm_dequant_packed_ex(ref, dev, M, N, K, ydt, mode):
    log("gemm_dequant_packed_ex", M, N, K, ydt, mode)
    use_bias, relu = MODES[mode]
    xq, wq, sx, sw, bias = _case(M, N, K, M * 7 + N + K)
    wp = sq.pack_weight(_gpu(wq, dev))
    act = sq.SQ_ACT_RELU if relu else sq.SQ_ACT_NONE
    y = sq.w8a8_gemm_dequant_packed_ex(_gpu(xq, dev), _gpu(sx, dev), wp, _gpu(sw, dev),
                                       _gpu(bias, dev), act, DT[ydt])
    y_rm = sq.w8a8_gemm_dequant_ex(_gpu(xq, dev), _gpu(sx, dev), _gpu(wq, dev), _gpu(sw, dev),
                                   _gpu(bias, dev), act, DT[ydt])
    torch.cuda.synchronize()
    _check(y, ref, ref.gemm_i32(xq, wq), sx, sw, bias, relu, "y_packed_ex")
    assert_equal(y.cpu().view(torch.int16), y_rm.cpu().view(torch.int16).numpy(),
                 "packed vs row-major")


@pytest.mark.parametrize("M,N,K", [(5, 300, 512), (700, 513, 2048)])
def test_gemm_dequant_ex_without_extras_is_plain_scale_back(dev, M, N, K):
    xq, wq, sx, sw, _ = _case(M, N, K, 3)
    args = [_gpu(a, dev) for a in (xq, sx, wq, sw)]
    y0 = sq.w8a8_gemm_dequant(*args, torch.float16)
    y1 = sq.w8a8_gemm_dequant_ex(*args, None, sq.SQ_ACT_NONE, torch.float16)
    torch.cuda.synchronize()
    assert_equal(y1.cpu().view(torch.int16), y0.cpu().view(torch.int16).numpy(), "ex vs plain")


# ------------------------------------------------------ fold into a linear layer

@pytest.mark.parametrize("Kp,K,dt", [(64, 512, "f32"), (333, 1000, "f16"), (100, 77, "bf16"),
                                     (4096, 16384, "f16"), (7, 5, "f32"), (1, 1, "bf16")])
@pytest.mark.parametrize("with_bias", [False, True])
def test_fold_prev_linear(ref, dev, Kp, K, dt, with_bias):
    log("fold_prev_linear", Kp, K, dt, with_bias)
    w = synth.random_matrix(Kp + 3 * K, Kp, K, dt, scale=0.02)
    s = np.exp(np.random.default_rng([Kp, K]).standard_normal(K)).astype(np.float32)
    bias = (np.random.default_rng([K, Kp]).standard_normal(K) * 0.1).astype(np.float32)
    b_d = _gpu(bias, dev) if with_bias else None
    w_out = sq.fold_prev_linear(_gpu(s, dev), _gpu(w, dev), b_d)
    torch.cuda.synchronize()
    w_r, b_r = ref.fold_prev_linear(s, w, bias if with_bias else None)
    assert_equal(w_out, w_r, "folded weight")
    if with_bias:
        assert_equal(b_d, b_r, "folded bias")


@pytest.mark.parametrize("M,Kp,K,N", [(16, 512, 2048, 512), (300, 1024, 4096, 1024)])
def test_folded_layer_pair_chain(ref, dev, M, Kp, K, N):
    """FC1 -> ReLU -> FC2 with FC2's smoothing folded into FC1 (weight columns
    and bias), both layers W8A8: every intermediate bit-exact, the output within
    the bar.  FC2's calibration input is the float ReLU output of FC1 on a
    separate draw (computed here in double, an input to both sides)."""
    log("folded pair", M, Kp, K, N)
    rng = np.random.default_rng([M, Kp, K, N])
    out_cols = rng.choice(Kp, 4, replace=False).tolist()
    x = synth.random_matrix(M + Kp, M, Kp, "f16", outlier_cols=out_cols, factor=30.0)
    x_cal = synth.random_matrix(M + Kp + 1, 128, Kp, "f16", outlier_cols=out_cols, factor=30.0)
    w1 = synth.random_matrix(Kp * 5 + K, Kp, K, "f16", scale=0.02)
    w2 = synth.random_matrix(K * 5 + N, K, N, "f16", scale=0.02)
    b1 = (rng.standard_normal(K) * 0.1).astype(np.float32)
    h_cal = torch.from_numpy(np.maximum(x_cal.double().numpy() @ w1.double().numpy() + b1, 0.0)
                             .astype(np.float32)).half()

    # GPU: offline (calibrate, smooth FC2, fold into FC1, quantise both), run time
    a = sq.calibrate_absmax(_gpu(h_cal, dev))
    s, w2_hat = sq.smooth_fold(a, _gpu(w2, dev), 0.5)
    b1_d = _gpu(b1, dev)
    w1_f = sq.fold_prev_linear(s, _gpu(w1, dev), b1_d)
    wq1, sw1 = sq.quant_weight_perchannel(w1_f)
    wq2, sw2 = sq.quant_weight_perchannel(w2_hat)
    xq0, sx0 = sq.quant_act_pertoken(_gpu(x, dev))
    h = sq.w8a8_gemm_dequant_ex(xq0, sx0, wq1, sw1, b1_d, sq.SQ_ACT_RELU, torch.float16)
    xq1, sx1 = sq.quant_act_pertoken(h)
    y = sq.w8a8_gemm_dequant(xq1, sx1, wq2, sw2, torch.float16)
    torch.cuda.synchronize()

    a_r = ref.calibrate_absmax(h_cal)
    s_r, w2_hat_r, _, _ = ref.smooth_fold(a_r, w2, 0.5)
    assert_equal(s, s_r, "s")
    w1_f_r, b1_r = ref.fold_prev_linear(s_r, w1, b1)
    assert_equal(w1_f, w1_f_r, "folded FC1 weight")
    assert_equal(b1_d, b1_r, "folded FC1 bias")
    wq1_r, sw1_r = ref.quant_weight_perchannel(w1_f_r)
    wq2_r, sw2_r = ref.quant_weight_perchannel(w2_hat_r)
    assert_equal(wq1, wq1_r, "Wq1")
    assert_equal(wq2, wq2_r, "Wq2")
    xq0_r, sx0_r = ref.quant_act_pertoken(x)
    assert_equal(xq0, xq0_r, "Xq0")
    acc1_r = ref.gemm_i32(xq0_r, wq1_r)
    h_r = torch.from_numpy(ref.dequant_bias_act_f32(acc1_r, sx0_r, sw1_r, b1_r, True)).half()
    assert_equal(h.cpu().view(torch.int16), h_r.view(torch.int16).numpy(), "FC1 output (smoothed)")
    xq1_r, sx1_r = ref.quant_act_pertoken(h_r)
    assert_equal(xq1, xq1_r, "Xq1")
    assert_equal(sx1, sx1_r, "sx1")
    acc2_r = ref.gemm_i32(xq1_r, wq2_r)
    y_r = ref.dequant(acc2_r, sx1_r, sw2_r)
    g = to_np(y).astype(np.float64)
    diff = np.abs(g - y_r)
    assert ((diff <= 1e-3 * np.abs(y_r)) | (diff <= out_ulp(y_r, torch.float16))).all()
    # the folded pair stays close to the float pair relu(x W1 + b1) W2: two
    # stacked W8A8 layers measure 3-6% here; a fold on the wrong axis or with
    # the factors inverted is off by far more than 10%
    exact = np.maximum(x.double().numpy() @ w1.double().numpy() + b1, 0.0) @ w2.double().numpy()
    rel = np.linalg.norm(g - exact) / np.linalg.norm(exact)
    log("  relative error vs float pair:", rel)
    assert rel < 0.1
