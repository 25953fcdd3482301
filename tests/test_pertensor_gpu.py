"""GPU parity of the per-tensor paths [P1 推論方法: O2 per-tensor dynamic
activations, O3 per-tensor static activations from calibration, per-tensor
weights] against the CPU oracle: codes and steps bit-exact, 16-bit outputs of
the chained GEMM within 1e-3 relative or one output ulp."""
import numpy as np
import pytest
import torch

import synth
import w8a8_int8_post_amd as sq
from sqtest_util import assert_equal, assert_y_close, log, to_np

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _gpu(t, dev):
    return t.contiguous().to(dev)


def _smooth(K):
    return np.exp(np.random.default_rng([5, K]).standard_normal(K)).astype(np.float32)


ACT_SHAPES = [(16, 512, "f32"), (2048, 4096, "f16"), (1, 4096, "f16"), (5, 16384, "bf16"),
              (9, 1001, "f16"), (7, 13, "f32"), (1, 1, "bf16"), (300, 28672, "f16"),
              (3, 24580, "f32"), (4097, 12288, "bf16")]


@pytest.mark.parametrize("K,N,dt", [(512, 512, "f32"), (4096, 1000, "f32"), (77, 333, "f32"),
                                    (1000, 4096, "f16"), (130, 70, "bf16"), (1, 3, "f32"),
                                    (4096, 12288, "bf16")])
def test_quant_weight_pertensor(ref, dev, K, N, dt):
    log("quant_weight_pertensor", K, N, dt)
    w = synth.random_matrix(K * 17 + N, K, N, dt, scale=0.02)
    wq, sw = sq.quant_weight_pertensor(_gpu(w, dev))
    torch.cuda.synchronize()
    wq_r, sw_r = ref.quant_weight_pertensor(w)
    assert_equal(sw, sw_r, "w_scale (per tensor)")
    assert_equal(wq, wq_r, "wq (per tensor)")


def test_quant_weight_pertensor_zero(ref, dev):
    w = torch.zeros(64, 48, dtype=torch.float16)
    wq, sw = sq.quant_weight_pertensor(_gpu(w, dev))
    torch.cuda.synchronize()
    assert (to_np(sw) == 0).all() and (to_np(wq) == 0).all()


@pytest.mark.parametrize("M,K,dt", ACT_SHAPES)
@pytest.mark.parametrize("smooth", [False, True])
def test_quant_act_pertensor_dynamic(ref, dev, M, K, dt, smooth):
    log("act_pertensor O2", M, K, dt, smooth)
    x = synth.random_matrix(M * 19 + K, M, K, dt, outlier_cols=[0, K // 2], factor=50.0)
    s_np = _smooth(K) if smooth else None
    s_gpu = _gpu(torch.from_numpy(s_np), dev) if smooth else None
    xq, sx = sq.quant_act_pertensor(_gpu(x, dev), s_gpu)
    torch.cuda.synchronize()
    xf = x.float().numpy()
    if smooth:
        xf = ref.smooth_activation(xf, s_np)
    xq_r, sx_r = ref.quant_act_pertensor(xf)
    assert_equal(sx, sx_r, "x_scale (O2)")
    assert_equal(xq, xq_r, "xq (O2)")


@pytest.mark.parametrize("M,K,dt", ACT_SHAPES)
@pytest.mark.parametrize("smooth", [False, True])
def test_quant_act_pertensor_static(ref, dev, M, K, dt, smooth):
    """O3: the step comes from a calibration batch; the quantised batch has
    larger outliers, and twice the calibration maximum in the channel that
    sets the step, so the clamp at +-127 is exercised."""
    log("act_pertensor O3", M, K, dt, smooth)
    calib = synth.random_matrix(M * 23 + K, max(M, 8), K, dt, outlier_cols=[0], factor=20.0)
    x = synth.random_matrix(M * 29 + K, M, K, dt, outlier_cols=[0, K - 1], factor=60.0)
    s_np = _smooth(K) if smooth else np.ones(K, np.float32)
    j = int(np.argmax(ref.calibrate_absmax(calib).astype(np.float64) / s_np))
    x[M // 2, j] = -2.0 * calib[:, j].float().abs().max()
    s_gpu = _gpu(torch.from_numpy(s_np), dev)
    a = sq.calibrate_absmax(_gpu(calib, dev))
    step = sq.static_act_step(a, s_gpu)
    xq, sx = sq.quant_act_pertensor(_gpu(x, dev), s_gpu if smooth else None, step)
    torch.cuda.synchronize()
    a_r = ref.calibrate_absmax(calib)
    step_r = ref.static_act_step(a_r, s_np)
    assert_equal(step, np.array([step_r], np.float32), "static step")
    xf = x.float().numpy()
    if smooth:
        xf = ref.smooth_activation(xf, s_np)
    xq_r, sx_r = ref.quant_act_pertensor(xf, step_r)
    assert_equal(sx, sx_r, "x_scale (O3)")
    assert_equal(xq, xq_r, "xq (O3)")
    assert xq_r[M // 2, j] == -127, "the planted value should saturate"
    log("  saturated fraction", (np.abs(xq_r) == 127).mean())


@pytest.mark.parametrize("step_val", [0.0, 1e-40, 3e-30, 0.5, 1.0 / 127, 7.5e28, 1e31])
def test_quant_act_static_steps(ref, dev, step_val):
    """Given steps across the fp32 range: zero (codes 0), subnormal, the edges
    of the reciprocal fast path, and huge."""
    rng = np.random.default_rng(int(step_val * 0) + 11)
    x = (rng.standard_normal((6, 1024)) * np.float64(step_val or 1.0) * 90.0).astype(np.float32)
    x[2] *= 4.0  # a row beyond 127 steps saturates
    x[3] = 0.0
    st = torch.tensor([step_val], dtype=torch.float32, device=dev)
    xq, sx = sq.quant_act_pertensor(_gpu(torch.from_numpy(x), dev), None, st)
    torch.cuda.synchronize()
    xq_r, sx_r = ref.quant_act_pertensor(x, np.float32(step_val))
    assert_equal(sx, sx_r, "x_scale (given step %g)" % step_val)
    assert_equal(xq, xq_r, "xq (given step %g)" % step_val)


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (16, 4096, 4096), (300, 1000, 1024),
                                   (2048, 12288, 4096)])
@pytest.mark.parametrize("ydt", ["f16", "bf16"])
def test_o3_chain(ref, dev, M, N, K, ydt):
    """O3 end to end: calibration -> smoothing factors -> fold -> per-tensor
    weights -> static step -> codes -> INT8 GEMM with scale back, both the
    row-major and the fragment-packed GEMM."""
    log("O3 chain", M, N, K, ydt)
    calib = synth.random_matrix(M + 7 * K, 64, K, "f16", outlier_cols=[3, K // 3], factor=40.0)
    x = synth.random_matrix(M + 11 * K, M, K, "f16", outlier_cols=[3, K // 3], factor=45.0)
    w = synth.random_matrix(N + 13 * K, K, N, "f16", scale=0.02)
    a = sq.calibrate_absmax(_gpu(calib, dev))
    s, w_hat = sq.smooth_fold(a, _gpu(w, dev), 0.5)
    wq, sw = sq.quant_weight_pertensor(w_hat)
    step = sq.static_act_step(a, s)
    x_hat = sq.smooth_activation(_gpu(x, dev), s)
    xq, sx = sq.quant_act_pertensor(x_hat, None, step)
    y = sq.w8a8_gemm_dequant(xq, sx, wq, sw, DT[ydt])
    y_p = sq.w8a8_gemm_dequant_packed(xq, sx, sq.pack_weight(wq), sw, DT[ydt]) \
        if K % 128 == 0 else None
    torch.cuda.synchronize()
    # the oracle follows the same steps from the same inputs
    a_r = ref.calibrate_absmax(calib)
    s_r, w_hat_r, _, _ = ref.smooth_fold(a_r, w, 0.5)
    same_s = (to_np(s) == s_r).all()
    if not same_s:  # one-ulp pow differences: continue from the GPU's factors
        s_r = to_np(s)
        w_hat_r = ref.fold_weight(w.float().numpy(), s_r)
    wq_r, sw_r = ref.quant_weight_pertensor(w_hat_r)
    step_r = ref.static_act_step(a_r, s_r)
    x_hat_r = ref.smooth_activation(x.float().numpy(), s_r).astype(np.float16)
    xq_r, sx_r = ref.quant_act_pertensor(x_hat_r, step_r)
    assert_equal(wq, wq_r, "wq")
    assert_equal(sx, sx_r, "x_scale")
    assert_equal(xq, xq_r, "xq")
    if M * N * K <= 2 ** 31:
        y_r = ref.dequant(ref.gemm_i32(xq_r, wq_r), sx_r, sw_r)
        assert_y_close(y, y_r, "y (O3)")
    else:  # full-size layer: every (sampled token, sampled channel) output
        rng = np.random.default_rng([M, N, K])
        rows = np.unique(np.r_[0, M - 1, rng.integers(0, M, 61)])
        cols = np.unique(np.r_[0, N - 1, rng.integers(0, N, 251)])
        acc_r = ref.gemm_i32_sampled(xq_r, wq_r, rows, cols)
        y_r = ref.dequant(acc_r, sx_r[rows], sw_r[cols])
        y_s = y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)]
        assert_y_close(y_s, y_r, "y (O3, sampled)")
    if y_p is not None:
        assert torch.equal(y_p, y), "packed and row-major GEMMs differ"


def _y_check(ref, dev, y, xq_r, sx_r, wq_r, sw_r, what):
    M, N = y.shape
    K = xq_r.shape[1]
    if M * N * K <= 2 ** 31:
        assert_y_close(y, ref.dequant(ref.gemm_i32(xq_r, wq_r), sx_r, sw_r), what)
        return
    rng = np.random.default_rng([M, N, K, 1])
    rows = np.unique(np.r_[0, M - 1, rng.integers(0, M, 61)])
    cols = np.unique(np.r_[0, N - 1, rng.integers(0, N, 251)])
    y_r = ref.dequant(ref.gemm_i32_sampled(xq_r, wq_r, rows, cols), sx_r[rows], sw_r[cols])
    y_s = y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)]
    assert_y_close(y_s, y_r, what + " (sampled)")


# (M, N, K, x dtype, y dtype): one kernel while M <= 2 and M * K <= 16384,
# else the per-tensor codes kernel and the packed GEMM
STATIC_LINEAR = [(1, 4096, 4096, "f16", "f16"), (4, 12288, 4096, "f16", "f16"),
                 (2, 28672, 8192, "f16", "bf16"), (16, 1000, 2048, "bf16", "f16"),
                 (3, 4100, 8192, "f32", "f32"), (1, 8, 128, "f16", "f16"),
                 (16, 4096, 4096, "f16", "f16"), (64, 16384, 4096, "f16", "bf16"),
                 (300, 1000, 1024, "bf16", "f32"), (2048, 12288, 4096, "f16", "f16"),
                 (1, 28672, 16384, "f16", "f16"), (2, 700, 4096, "bf16", "f32")]


@pytest.mark.parametrize("M,N,K,xdt,ydt", STATIC_LINEAR)
def test_linear_packed_static(ref, dev, M, N, K, xdt, ydt):
    log("linear_packed_static", M, N, K, xdt, ydt)
    calib = synth.random_matrix(M + 31 * K, 64, K, xdt, outlier_cols=[1, K // 5], factor=30.0)
    x = synth.random_matrix(M + 37 * K, M, K, xdt, outlier_cols=[1, K // 5], factor=45.0)
    a_r = ref.calibrate_absmax(calib)
    j = int(np.argmax(a_r))
    x[M - 1, j] = 3.0 * calib[:, j].float().abs().max()  # saturates at +127
    w = synth.random_matrix(N + 41 * K, K, N, "f32", scale=0.02)
    ones = np.ones(K, np.float32)
    step = sq.static_act_step(_gpu(torch.from_numpy(a_r), dev), _gpu(torch.from_numpy(ones), dev))
    wq, sw = sq.quant_weight_pertensor(_gpu(w, dev))
    wp = sq.pack_weight(wq)
    x_d = _gpu(x, dev)
    y, xq, sx = sq.linear_w8a8_packed_static(x_d, wp, sw, step, DT[ydt])
    # the same layer as two calls
    xq2, sx2 = sq.quant_act_pertensor(x_d, None, step)
    y2 = sq.w8a8_gemm_dequant_packed(xq2, sx2, wp, sw, DT[ydt])
    torch.cuda.synchronize()
    step_r = ref.static_act_step(a_r, ones)
    wq_r, sw_r = ref.quant_weight_pertensor(w)
    xq_r, sx_r = ref.quant_act_pertensor(x.float().numpy(), step_r)
    assert xq_r[M - 1, j] == 127
    assert_equal(step, np.array([step_r], np.float32), "static step")
    assert_equal(xq, xq_r, "xq (one-call O3)")
    assert_equal(sx, sx_r, "x_scale (one-call O3)")
    assert torch.equal(y, y2), "one-call and two-call O3 layers differ"
    _y_check(ref, dev, y, xq_r, sx_r, wq_r, sw_r, "y (one-call O3)")


def test_linear_packed_static_alias(dev):
    x = torch.zeros(2, 128, dtype=torch.float16, device=dev)
    wp = torch.zeros(sq.sq_packed_weight_bytes(16, 128), dtype=torch.int8, device=dev)
    sw = torch.ones(16, device=dev)
    xq = torch.empty(2, 128, dtype=torch.int8, device=dev)
    sx = torch.empty(2, device=dev)
    y = torch.empty(2, 16, dtype=torch.float16, device=dev)
    with pytest.raises(sq.SQError) as ei:
        sq.sq_w8a8_linear_packed_static(x, wp, sw, sx[1:], xq, sx, y)
    assert ei.value.code == 8


# Values whose quotient v / step overflows fp32 under steps inside the
# reciprocal fast path [2^-96, 2^96]: they must saturate to +-127 with their
# own sign (P1 推論方法 O3: a static step clamps values past the calibrated
# range).  fp16 cannot reach such quotients (|v| <= 65504).
OVERFLOW_STEPS = [2.0 ** -96, 1e-20, 0.05]


def _overflow_input(rng, M, K, step, dt):
    x = (rng.standard_normal((M, K)) * 90.0 * step).astype(np.float32)
    big = np.array([1e10, 1e19, 3e37, 3.3e38], np.float32)
    idx = rng.integers(0, M * K, 64)
    x.ravel()[idx] = big[rng.integers(0, 4, 64)] * np.where(rng.random(64) < 0.5, -1.0, 1.0)
    planted = rng.choice(M * K, 2, replace=False)  # two distinct elements
    x.ravel()[planted] = [3e37, -3e37]
    t = torch.from_numpy(x)
    if dt == "bf16":
        t = t.to(torch.bfloat16)
    return t, planted


@pytest.mark.parametrize("step_val", OVERFLOW_STEPS)
@pytest.mark.parametrize("M,K,dt", [(6, 1024, "f32"), (5, 1001, "f32"), (7, 13, "f32"),
                                    (6, 1024, "bf16"), (3, 4104, "bf16"), (1, 9, "bf16")])
def test_quant_act_static_overflow(ref, dev, M, K, dt, step_val):
    rng = np.random.default_rng([17, M, K])
    x, planted = _overflow_input(rng, M, K, step_val, dt)
    st = torch.tensor([step_val], dtype=torch.float32, device=dev)
    xq, sx = sq.quant_act_pertensor(_gpu(x, dev), None, st)
    torch.cuda.synchronize()
    xq_r, sx_r = ref.quant_act_pertensor(x.float().numpy(), np.float32(step_val))
    assert list(xq_r.ravel()[planted]) == [127, -127]
    assert_equal(sx, sx_r, "x_scale (given step %g)" % step_val)
    assert_equal(xq, xq_r, "xq (given step %g, quotients past fp32)" % step_val)


# one kernel (M <= 2, M * K <= 16384) and the codes kernel + packed GEMM
@pytest.mark.parametrize("M,N,K,xdt", [(1, 4096, 4096, "bf16"), (2, 700, 8192, "f32"),
                                       (16, 1000, 2048, "f32"), (300, 1000, 1024, "bf16")])
def test_linear_packed_static_overflow(ref, dev, M, N, K, xdt):
    rng = np.random.default_rng([19, M, N, K])
    # calibration maxima that give the step 2^-90 (inside the fast path)
    a_r = np.full(K, np.float32(127.0 * 2.0 ** -90), np.float32)
    ones = np.ones(K, np.float32)
    step_r = ref.static_act_step(a_r, ones)
    x, planted = _overflow_input(rng, M, K, float(step_r), xdt)
    w = synth.random_matrix(N + 43 * K, K, N, "f32", scale=0.02)
    step = sq.static_act_step(_gpu(torch.from_numpy(a_r), dev), _gpu(torch.from_numpy(ones), dev))
    wq, sw = sq.quant_weight_pertensor(_gpu(w, dev))
    y, xq, sx = sq.linear_w8a8_packed_static(_gpu(x, dev), sq.pack_weight(wq), sw, step,
                                              torch.float32)
    torch.cuda.synchronize()
    wq_r, sw_r = ref.quant_weight_pertensor(w)
    xq_r, sx_r = ref.quant_act_pertensor(x.float().numpy(), step_r)
    assert list(xq_r.ravel()[planted]) == [127, -127]
    assert_equal(step, np.array([step_r], np.float32), "static step")
    assert_equal(xq, xq_r, "xq (one-call O3, quotients past fp32)")
    assert_equal(sx, sx_r, "x_scale (one-call O3)")
    _y_check(ref, dev, y, xq_r, sx_r, wq_r, sw_r, "y (one-call O3, quotients past fp32)")
