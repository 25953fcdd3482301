"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
value the pages print, a hand derivation, a closed form of the method, a
library routine on a reduction of the method, or a pure-Python brute force.

P1 = abeam.tech SmoothQuant explainer; P4 = blogs.itmedia.co.jp 量子化 blog.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Quantiser: P4 section 3 worked example, ties, bounds

def test_p4_worked_example(ref):
    g = _golden("p4_worked_example.json")
    q = ref.quantize_value(g["value"], g["step"])
    assert q == g["code"]
    assert q * g["step"] == g["dequantized"]
    assert g["value"] - q * g["step"] == g["error"]


@pytest.mark.parametrize("v,expect", [(62.5, 63), (-62.5, -63), (0.5, 1), (-0.5, -1),
                                      (0.49999997, 0), (-0.49999997, 0), (126.5, 127),
                                      (127.0, 127), (-127.0, -127), (1.5, 2), (2.5, 3),
                                      (0.0, 0)])
def test_ties_round_away_from_zero(ref, v, expect):
    # step 1 exactly (absmax 127): v / step == v, so only the rounding rule acts.
    assert ref.step(127.0) == 1.0
    assert ref.quantize_value(v, 1.0) == expect


def test_clamp_to_127(ref):
    # A value beyond the range (static steps) clamps to the symmetric code range.
    assert ref.quantize_value(500.0, 1.0) == 127
    assert ref.quantize_value(-500.0, 1.0) == -127


def test_zero_vector_has_zero_step_and_codes(ref):
    q, st = ref.quantize_vector(np.zeros(33, np.float32))
    assert st == 0.0 and not q.any()


@pytest.mark.parametrize("seed", range(6))
def test_quantizer_matches_bruteforce(ref, seed):
    r = np.random.default_rng([7, seed])
    v = (r.standard_normal(97) * r.choice([1e-3, 1.0, 37.0])).astype(np.float32)
    v[r.integers(0, 97)] *= 40  # an outlier sets the range
    q, st = ref.quantize_vector(v)
    qb, stb = brute.quantize_vector(v)
    assert st == stb
    assert q.tolist() == qb


@pytest.mark.parametrize("seed", range(4))
def test_quantizer_error_bound_and_full_range(ref, seed):
    r = np.random.default_rng([8, seed])
    x = r.standard_normal((64, 301)).astype(np.float32) * 3
    xq, sx = ref.quant_act_pertoken(x)
    # every non-zero row uses the extreme code (the range is set by the absmax)
    assert (np.abs(xq.astype(np.int32)).max(axis=1) == 127).all()
    assert xq.min() >= -127
    # |v - q*step| <= step * (1/2 + 2^-17) elementwise, evaluated in fp64
    err = np.abs(x.astype(np.float64) - xq.astype(np.float64) * sx[:, None].astype(np.float64))
    assert (err <= sx[:, None].astype(np.float64) * (0.5 + 2.0 ** -17)).all()
    # the step is absmax/127 of each row (library reduction of the same data)
    np.testing.assert_array_equal(sx, (np.abs(x).max(axis=1) / np.float32(127)).astype(np.float32))


def test_weight_quant_is_per_output_channel_and_transposed(ref):
    r = np.random.default_rng(11)
    w = (r.standard_normal((37, 5)) * 0.02).astype(np.float32)
    w[:, 3] *= 50  # one loud output channel must not coarsen the others
    wq, sw = ref.quant_weight_perchannel(w)
    assert wq.shape == (5, 37) and sw.shape == (5,)
    for n in range(5):
        codes, st = brute.quantize_vector(w[:, n])
        assert sw[n] == st
        assert wq[n].tolist() == codes


# --------------------------------------------------------------------------
# INT8 GEMM: brute force over Python integers

@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (17, 9, 64), (8, 33, 129), (5, 4, 300)])
def test_gemm_matches_python_ints(ref, shape):
    M, N, K = shape
    xq = synth.random_int8(M * 1000 + K, M, K)
    wq = synth.random_int8(N * 1000 + K + 1, N, K)
    xq[0, :] = 127
    wq[0, :] = -127  # extremes included
    acc = ref.gemm_i32(xq, wq)
    assert acc.tolist() == brute.gemm_int(xq, wq)


def test_gemm_sampled_equals_full(ref):
    xq = synth.random_int8(1, 40, 200)
    wq = synth.random_int8(2, 30, 200)
    rows = np.array([0, 7, 39, 7])
    cols = np.array([29, 0, 3])
    sub = ref.gemm_i32_sampled(xq, wq, rows, cols)
    assert sub.tolist() == [[r[c] for c in cols] for r in np.array(brute.gemm_int(xq[rows], wq)).tolist()]


def test_gemm_int32_worst_case_fits():
    # |acc| <= K * 127^2 < 2^31 at the largest accepted K.
    assert 133144 * 127 * 127 == 2147479576 < 2 ** 31
    assert 133145 * 127 * 127 >= 2 ** 31


def test_gemm_worst_case_value(ref):
    K = 133144
    xq = np.full((1, K), 127, np.int8)
    wq = np.full((2, K), 127, np.int8)
    wq[1] = -127
    acc = ref.gemm_i32_sampled(xq, wq, np.array([0]), np.array([0, 1]))
    assert acc.tolist() == [[2147479576, -2147479576]]
    with pytest.raises(ValueError):
        ref.gemm_i32(np.zeros((1, K + 1), np.int8), np.zeros((1, K + 1), np.int8))


def test_int8_numpy_wrap_pitfall_is_avoided(ref):
    a = np.array([[127, 127]], np.int8)
    assert int(np.dot(a[0], a[0])) != 2 * 127 * 127  # numpy int8 dot wraps
    assert ref.gemm_i32(a, a)[0, 0] == 2 * 127 * 127


# --------------------------------------------------------------------------
# Calibration and smoothing factor (P1 smoothing factor section, identity)

def test_calibration_is_columnwise_absmax_and_running(ref):
    r = np.random.default_rng(3)
    x = r.standard_normal((50, 70)).astype(np.float32)
    a = ref.calibrate_absmax(x)
    np.testing.assert_array_equal(a, np.abs(x).max(axis=0))
    a2 = ref.calibrate_absmax(x[30:], ref.calibrate_absmax(x[:30]))
    np.testing.assert_array_equal(a, a2)


def test_hand_chain_golden(ref):
    g = _golden("hand_chain_2x2.json")
    a = ref.calibrate_absmax(np.array(g["X_cal"], np.float32))
    assert a.tolist() == g["a"]
    W = np.array(g["W"], np.float32)
    assert ref.weight_row_absmax(W).tolist() == g["b"]
    s, w_hat, _, _ = ref.smooth_fold(a, W, g["alpha"])
    assert s.tolist() == g["s"]
    assert w_hat.tolist() == g["W_hat"]
    wq, sw = ref.quant_weight_perchannel(w_hat)
    assert wq.tolist() == g["Wq"]
    np.testing.assert_array_equal(sw, np.array(g["sw_absmax"], np.float32) / np.float32(127))
    x_hat = ref.smooth_activation(np.array(g["X"], np.float32), s)
    np.testing.assert_array_equal(x_hat, np.array(g["X_hat"], np.float32))
    xq, sx = ref.quant_act_pertoken(x_hat)
    assert xq.tolist() == g["Xq"]
    acc = ref.gemm_i32(xq, wq)
    assert acc.tolist() == g["acc"]
    y = ref.dequant(acc, sx, sw)
    np.testing.assert_allclose(y, np.array(g["y"]), rtol=1e-6)
    np.testing.assert_allclose(y, np.array(g["XW"]), rtol=2e-3)
    np.testing.assert_array_equal(ref.linear_w8a8(x_hat, wq, sw), y)


def _outlier_problem(seed, K=96, N=40, T=128, M=24, factor=40.0):
    r = np.random.default_rng([5, seed])
    cols = r.choice(K, 4, replace=False)
    xc = r.standard_normal((T, K)).astype(np.float32)
    xc[:, cols] *= factor
    x = r.standard_normal((M, K)).astype(np.float32)
    x[:, cols] *= factor
    w = (r.standard_normal((K, N)) * 0.02).astype(np.float32)
    return xc, x, w


@pytest.mark.parametrize("alpha", [0.4, 0.5, 0.6, 0.75])
def test_identity_holds_fp64(ref, alpha):
    # (X diag(s)^-1)(diag(s) W) == X W  [P1 数学的に何をしているのか]
    xc, x, w = _outlier_problem(1)
    s, w_hat, _, _ = ref.smooth_fold(ref.calibrate_absmax(xc), w, alpha)
    s64 = s.astype(np.float64)
    lhs = (x.astype(np.float64) / s64) @ (s64[:, None] * w.astype(np.float64))
    rhs = x.astype(np.float64) @ w.astype(np.float64)
    assert np.abs(lhs - rhs).max() / np.abs(rhs).max() <= 1e-12
    # and the oracle's fp32 fold realises it up to fp32 rounding
    lhs32 = ref.smooth_activation(x, s).astype(np.float64) @ w_hat.astype(np.float64)
    assert np.abs(lhs32 - rhs).max() / np.abs(rhs).max() <= 1e-6


def test_alpha_half_balances_maxima(ref):
    # At alpha = 0.5: max|X_hat_j| = max|W_hat_j| = sqrt(max|X_j| max|W_j|)
    xc, _, w = _outlier_problem(2)
    a = ref.calibrate_absmax(xc)
    b = np.abs(w).max(axis=1)
    s, w_hat, _, _ = ref.smooth_fold(a, w, 0.5)
    xm = np.abs(ref.smooth_activation(xc, s)).max(axis=0).astype(np.float64)
    wm = np.abs(w_hat).max(axis=1).astype(np.float64)
    target = np.sqrt(a.astype(np.float64) * b.astype(np.float64))
    ulp = np.spacing(target.astype(np.float32)).astype(np.float64)
    assert (np.abs(xm - target) <= 4 * ulp).all()
    assert (np.abs(wm - target) <= 4 * ulp).all()


@pytest.mark.parametrize("alpha", [0.4, 0.6, 0.75])
def test_alpha_closed_form(ref, alpha):
    # s = a^alpha / b^(1-alpha) gives max|X_hat_j| = a/s = (a b)^(1-alpha) and
    # max|W_hat_j| = s b = (a b)^alpha; their product is a_j b_j for every alpha.
    xc, _, w = _outlier_problem(3)
    a = ref.calibrate_absmax(xc).astype(np.float64)
    b = np.abs(w).max(axis=1).astype(np.float64)
    s, w_hat, _, _ = ref.smooth_fold(a.astype(np.float32), w, alpha)
    xm = np.abs(ref.smooth_activation(xc, s)).max(axis=0).astype(np.float64)
    wm = np.abs(w_hat).max(axis=1).astype(np.float64)
    np.testing.assert_allclose(xm, (a * b) ** (1 - alpha), rtol=4e-7)
    np.testing.assert_allclose(wm, (a * b) ** alpha, rtol=4e-7)
    np.testing.assert_allclose(xm * wm, a * b, rtol=8e-7)


def test_alpha_one_flattens_activations_exactly(ref):
    # alpha = 1: s_j = max|X_j| exactly, so every calibration channel's max is 1.0
    xc, _, w = _outlier_problem(4)
    a = ref.calibrate_absmax(xc)
    s, _, _, _ = ref.smooth_fold(a, w, 1.0)
    np.testing.assert_array_equal(s, a)
    np.testing.assert_array_equal(np.abs(ref.smooth_activation(xc, s)).max(axis=0), 1.0)


def test_alpha_zero_normalises_weights(ref):
    xc, _, w = _outlier_problem(5)
    a = ref.calibrate_absmax(xc)
    s, w_hat, _, _ = ref.smooth_fold(a, w, 0.0)
    b = np.abs(w).max(axis=1)
    np.testing.assert_array_equal(s, (np.float32(1) / b).astype(np.float32))
    wm = np.abs(w_hat).max(axis=1)
    assert (np.abs(wm - 1.0) <= 2.0 ** -23).all()


def test_zero_channel_gets_unit_factor(ref):
    a = np.array([0.0, 2.0, 3.0], np.float32)
    w = np.array([[1.0, 2.0], [0.0, 0.0], [0.5, -4.0]], np.float32)
    s, _, _, _ = ref.smooth_fold(a, w, 0.5)
    assert s[0] == 1.0 and s[1] == 1.0
    assert s[2] == np.float32(math.sqrt(3.0) / math.sqrt(4.0))


def test_layernorm_fold(ref):
    # LN(x)/s = (gamma/s) n + beta/s: folding diag(s)^-1 into LN gives the
    # same smoothed activations as dividing the LN output by s.
    r = np.random.default_rng(9)
    K = 64
    s = (np.exp(r.standard_normal(K))).astype(np.float32)
    gamma = (1 + 0.1 * r.standard_normal(K)).astype(np.float32)
    beta = (0.1 * r.standard_normal(K)).astype(np.float32)
    g2, b2 = ref.fold_norm(s, gamma, beta)
    n = r.standard_normal((8, K))
    lhs = n * g2.astype(np.float64) + b2.astype(np.float64)
    rhs = (n * gamma.astype(np.float64) + beta.astype(np.float64)) / s.astype(np.float64)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-6, atol=1e-7)


# --------------------------------------------------------------------------
# Whole chain

@pytest.mark.parametrize("alpha", [0.5, 0.75])
def test_chain_error_bound(ref, alpha):
    # |Y_q - X_hat W_hat| <= sum_k (|x|dw/2 + |w|dx/2 + dx dw/4) (+ tiny fp slack)
    xc, x, w = _outlier_problem(6)
    s, w_hat, _, _ = ref.smooth_fold(ref.calibrate_absmax(xc), w, alpha)
    x_hat = ref.smooth_activation(x, s)
    wq, sw = ref.quant_weight_perchannel(w_hat)
    xq, sx = ref.quant_act_pertoken(x_hat)
    y = ref.dequant(ref.gemm_i32(xq, wq), sx, sw)
    exact = x_hat.astype(np.float64) @ w_hat.astype(np.float64)
    dx = sx.astype(np.float64)[:, None]
    dw = sw.astype(np.float64)[None, :]
    ax = np.abs(x_hat.astype(np.float64)).sum(axis=1)[:, None]
    aw = np.abs(w_hat.astype(np.float64)).sum(axis=0)[None, :]
    K = x.shape[1]
    bound = (ax * dw + aw * dx) * (0.5 + 2.0 ** -17) + K * dx * dw / 4
    assert (np.abs(y - exact) <= bound * (1 + 1e-9) + 1e-12).all()


def test_smoothing_beats_naive_w8a8_on_outliers(ref):
    # P1 結果 / 精度: naive W8A8 (no smoothing) degrades on outlier activations,
    # SmoothQuant (alpha = 0.5) stays close to the float result.
    xc, x, w = _outlier_problem(7, K=256, N=64, factor=60.0)
    exact = x.astype(np.float64) @ w.astype(np.float64)

    def err(alpha):
        if alpha is None:
            x_hat, w_hat = x, w
        else:
            s, w_hat, _, _ = ref.smooth_fold(ref.calibrate_absmax(xc), w, alpha)
            x_hat = ref.smooth_activation(x, s)
        wq, sw = ref.quant_weight_perchannel(w_hat)
        y = ref.linear_w8a8(x_hat, wq, sw)
        return np.linalg.norm(y - exact) / np.linalg.norm(exact)

    assert err(0.5) < 0.5 * err(None)


def test_synth_outliers_persist():
    cfg = synth.CONFIGS[1]
    idx = synth.outlier_channels(cfg, "toy")
    assert len(idx) == 5
    xc = synth.activations(cfg, "toy", 64, calibration=True).numpy()
    xe = synth.activations(cfg, "toy", 16).numpy()
    for x in (xc, xe):
        col = np.abs(x).max(axis=0)
        assert set(np.argsort(col)[-5:]) == set(idx.tolist())
    assert not np.array_equal(xc[:16], xe)


# --------------------------------------------------------------------------
# Per-tensor variants (P1 推論方法: O2 per-tensor dynamic, O3 per-tensor static)

@pytest.mark.parametrize("seed", range(3))
def test_pertensor_dynamic_is_one_range_for_the_tensor(ref, seed):
    r = np.random.default_rng([11, seed])
    x = (r.standard_normal((5, 37)) * np.array([[0.1], [1.0], [3.0], [0.01], [7.0]])).astype(np.float32)
    xq, sx = ref.quant_act_pertensor(x)
    qb, stb = brute.quantize_vector(x.ravel())
    assert (sx == stb).all()
    assert xq.ravel().tolist() == qb


def test_pertensor_dynamic_single_row_is_pertoken(ref):
    x = np.random.default_rng(12).standard_normal((1, 300)).astype(np.float32)
    xq, sx = ref.quant_act_pertensor(x)
    xq_t, sx_t = ref.quant_act_pertoken(x)
    assert (xq == xq_t).all() and (sx == sx_t).all()


def test_pertensor_static_step_clamps(ref):
    # step 1: the code is the value rounded half away from zero, clamped to +-127
    v = np.array([[-200.0, -127.5, -126.5, -0.5, 0.49999997, 0.5, 126.49998, 126.5, 127.4, 300.0]],
                 np.float32)
    xq, sx = ref.quant_act_pertensor(v, 1.0)
    assert xq.tolist() == [[-127, -127, -127, -1, 0, 1, 126, 127, 127, 127]]
    assert sx.tolist() == [1.0]
    # step 0.5: 63.25 -> 126.5 -> 127; 64 -> 128 -> clamped
    xq, _ = ref.quant_act_pertensor(np.array([[63.25, 64.0, -64.0, 10.0]], np.float32), 0.5)
    assert xq.tolist() == [[127, 127, -127, 20]]


@pytest.mark.parametrize("seed", range(3))
def test_pertensor_static_matches_bruteforce(ref, seed):
    r = np.random.default_rng([13, seed])
    x = (r.standard_normal((4, 29)) * 3).astype(np.float32)
    step = np.float32(r.uniform(0.005, 0.05))
    xq, sx = ref.quant_act_pertensor(x, step)
    assert xq.ravel().tolist() == brute.quantize_with_step(x.ravel(), step)
    assert (sx == step).all()


def test_static_step_is_largest_smoothed_calibration_value(ref):
    # O3's step: the largest |x_hat| over the calibration set (x_hat = x / s,
    # one fp32 division per element, numpy here), over 127
    cfg = synth.CONFIGS[1]
    xc = synth.activations(cfg, "toy", cfg.T, calibration=True).float().numpy()
    w = synth.weight(cfg, "toy").float().numpy()
    a = np.abs(xc).max(axis=0)
    s = ref.smoothing_factors(a, np.abs(w).max(axis=1), 0.5)
    x_hat = xc / s[None, :]
    assert x_hat.dtype == np.float32
    assert ref.static_act_step(a, s) == np.float32(np.abs(x_hat).max()) / np.float32(127)


def test_static_step_alpha_one_is_one_over_127(ref):
    # alpha = 1: s_j = a_j, so every calibration channel is flattened to max 1
    a = np.abs(np.random.default_rng(14).standard_normal(64)).astype(np.float32) + 0.1
    s = ref.smoothing_factors(a, np.ones(64, np.float32), 1.0)
    assert ref.static_act_step(a, s) == np.float32(1) / np.float32(127)


def test_pertensor_weight_is_one_range_transposed(ref):
    w = (np.random.default_rng(15).standard_normal((23, 5)) * 0.02).astype(np.float32)
    w[3, 2] = 0.9  # one large weight sets the tensor's range
    wq, sw = ref.quant_weight_pertensor(w)
    codes, st = brute.quantize_vector(w.ravel())
    assert (sw == st).all()
    assert wq.tolist() == np.array(codes).reshape(23, 5).T.tolist()


def test_pertensor_weight_single_column_is_perchannel(ref):
    w = np.random.default_rng(16).standard_normal((40, 1)).astype(np.float32)
    assert all((p == q).all() for p, q in zip(ref.quant_weight_pertensor(w),
                                                ref.quant_weight_perchannel(w)))



# --------------------------------------------------------------------------
# Bias / ReLU epilogue and the fold into a preceding linear layer

def test_dequant_bias_relu_hand_example(ref):
    # token 0: 100*0.5*0.25 - 20 = -7.5 and -40*0.5*2 + 10 = -30;
    # token 1 (step 2): 100*2*0.25 - 20 = 30 and -40*2*2 + 10 = -150
    acc = np.array([[100, -40], [100, -40]], np.int32)
    sx = np.array([0.5, 2.0], np.float32)
    sw = np.array([0.25, 2.0], np.float32)
    bias = np.array([-20.0, 10.0], np.float32)
    assert ref.dequant_bias_act(acc, sx, sw, bias).tolist() == [[-7.5, -30.0], [30.0, -150.0]]
    assert ref.dequant_bias_act(acc, sx, sw, bias, relu=True).tolist() == [[0.0, 0.0], [30.0, 0.0]]
    assert ref.dequant_bias_act(acc, sx, sw).tolist() == [[12.5, -40.0], [50.0, -160.0]]
    assert ref.dequant_bias_act(acc, sx, sw, None, relu=True).tolist() == [[12.5, 0.0], [50.0, 0.0]]


def test_dequant_bias_act_reduces_to_dequant(ref):
    r = np.random.default_rng(21)
    acc = r.integers(-2 ** 20, 2 ** 20, (5, 7)).astype(np.int32)
    sx = r.random(5).astype(np.float32)
    sw = r.random(7).astype(np.float32)
    y0 = ref.dequant(acc, sx, sw)
    assert np.array_equal(ref.dequant_bias_act(acc, sx, sw), y0)
    assert np.array_equal(ref.dequant_bias_act(acc, sx, sw, relu=True), np.maximum(y0, 0.0))
    b = r.standard_normal(7).astype(np.float32)
    np.testing.assert_allclose(ref.dequant_bias_act(acc, sx, sw, b), y0 + b.astype(np.float64),
                               rtol=1e-15, atol=1e-15)


def test_fold_into_preceding_linear_through_relu(ref):
    # relu(x W1' + b1') (diag(s) W2) = relu(x W1 + b1) W2 when W1', b1' are
    # W1, b1 divided by s per output column (ReLU is positively homogeneous)
    r = np.random.default_rng(23)
    T, Kp, K, N = 6, 24, 40, 12
    x = r.standard_normal((T, Kp))
    w1 = (0.2 * r.standard_normal((Kp, K))).astype(np.float32)
    b1 = (0.1 * r.standard_normal(K)).astype(np.float32)
    w2 = (0.2 * r.standard_normal((K, N))).astype(np.float32)
    s = np.exp(r.standard_normal(K)).astype(np.float32)
    w1f, b1f = ref.fold_prev_linear(s, w1, b1)
    w2f = ref.fold_weight(w2, s)
    h = np.maximum(x @ w1f.astype(np.float64) + b1f.astype(np.float64), 0.0)
    lhs = h @ w2f.astype(np.float64)
    rhs = np.maximum(x @ w1.astype(np.float64) + b1.astype(np.float64), 0.0) @ w2.astype(np.float64)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-5, atol=1e-6)
    # the folded layer's output is the smoothed activation X diag(s)^-1
    h0 = np.maximum(x @ w1.astype(np.float64) + b1.astype(np.float64), 0.0)
    np.testing.assert_allclose(h, h0 / s.astype(np.float64), rtol=1e-5, atol=1e-7)
    # columns, not rows, are divided: the transposed fold breaks the identity
    # (a planted mistake the test must be able to see)
    assert not np.allclose(w1f, w1 / s[:Kp, None] if Kp <= K else w1, rtol=1e-3)


def test_fold_prev_linear_without_bias_and_unit_factors(ref):
    r = np.random.default_rng(24)
    w = r.standard_normal((9, 5)).astype(np.float32)
    out, b = ref.fold_prev_linear(np.ones(5, np.float32), w)
    assert b is None and np.array_equal(out, w)
    out, b = ref.fold_prev_linear(np.full(5, 2.0, np.float32), w, np.ones(5, np.float32))
    assert np.array_equal(out, w * np.float32(0.5)) and np.array_equal(b, np.full(5, 0.5, np.float32))


def test_dequant_bias_act_f32_hand_and_single_rounding(ref):
    acc = np.array([[100, -40], [100, -40]], np.int32)
    sx = np.array([0.5, 2.0], np.float32)
    sw = np.array([0.25, 2.0], np.float32)
    bias = np.array([-20.0, 10.0], np.float32)
    y = ref.dequant_bias_act_f32(acc, sx, sw, bias, relu=True)
    assert y.dtype == np.float32 and y.tolist() == [[0.0, 0.0], [30.0, 0.0]]
    assert ref.dequant_bias_act_f32(acc, sx, sw, bias).tolist() == [[-7.5, -30.0], [30.0, -150.0]]
    # f = 1 + 2^-12, sw = 1 + 2^-12: f*sw = 1 + 2^-11 + 2^-24 exactly; with
    # bias -1 one rounding keeps 2^-11 + 2^-24, while a rounded product (a tie,
    # to even: 1 + 2^-11) minus 1 would give 2^-11
    e = np.float32(1 + 2.0 ** -12)
    y = ref.dequant_bias_act_f32(np.array([[1]], np.int32), np.array([e]), np.array([e]),
                                 np.array([-1.0], np.float32))
    assert float(y[0, 0]) == 2.0 ** -11 + 2.0 ** -24
    # relu returns +0 for negative and zero values
    y = ref.dequant_bias_act_f32(np.array([[-3, 0]], np.int32), np.array([1.0], np.float32),
                                 np.array([1.0, 1.0], np.float32), None, relu=True)
    assert y.tolist() == [[0.0, 0.0]] and not np.signbit(y).any()


def test_dequant_bias_act_f32_within_fp32_bound_of_exact(ref):
    # |y32 - y| <= 2^-24 (|acc sx sw| + |y|) (one rounding for acc*sx, one for
    # the multiply-add; |acc| < 2^24 converts exactly), checked against the
    # double version
    r = np.random.default_rng(25)
    acc = r.integers(-2 ** 23, 2 ** 23, (32, 48)).astype(np.int32)
    sx = (r.random(32) * 1e-3).astype(np.float32)
    sw = (r.random(48) * 1e-3).astype(np.float32)
    b = (r.standard_normal(48) * 3).astype(np.float32)
    for relu in (False, True):
        y = ref.dequant_bias_act(acc, sx, sw, b, relu)
        p = np.abs(ref.dequant(acc, sx, sw))
        y32 = ref.dequant_bias_act_f32(acc, sx, sw, b, relu).astype(np.float64)
        assert (np.abs(y32 - y) <= 2.0 ** -24 * (p + np.abs(y)) * (1 + 1e-9)).all()


# --------------------------------------------------------------------------
# LayerNorm carrying the folded smoothing, fused with per-token quantisation

def test_layernorm_hand_example():
    from oracle import layernorm as ln
    x = np.array([[1.0, 2.0, 3.0, 4.0]], np.float32)
    y = ln.layernorm_f32(x, np.ones(4, np.float32), np.zeros(4, np.float32), 0.0)
    # mean 2.5, variance 1.25: (x - 2.5) / sqrt(1.25) = -3/sqrt5, -1/sqrt5, 1/sqrt5, 3/sqrt5
    r5 = 1.0 / np.sqrt(5.0)
    np.testing.assert_allclose(y[0], [-3 * r5, -r5, r5, 3 * r5], rtol=2 ** -22, atol=0)
    xq, sx, _ = ln.layernorm_quant_pertoken(x, np.ones(4, np.float32), np.zeros(4, np.float32),
                                            0.0, "f32")
    # step = max/127; 1/sqrt5 over step = 127/3 = 42.33 -> 42
    assert xq.tolist() == [[-127, -42, 42, 127]]
    assert sx[0] == np.float32(y[0, 3]) / np.float32(127.0)


def test_layernorm_statistics_are_rounded_once_from_exact_values():
    from decimal import Decimal, getcontext
    from oracle import layernorm as ln
    getcontext().prec = 60
    x = np.array([[1.0, 2.0, 4.0, 8.0]], np.float32)
    mu, rstd = ln.layernorm_stats(x, 0.0)
    assert mu[0] == np.float32(3.75)  # exact mean
    var = Decimal("7.1875")  # (2.75^2 + 1.75^2 + 0.25^2 + 4.25^2) / 4, exact
    exact = 1 / var.sqrt()
    # fp32 neighbours of the exact 1/sqrt(7.1875): the oracle returns the nearer
    f = np.float32(float(exact))
    cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(1))]
    best = min(cands, key=lambda c: abs(Decimal(float(c)) - exact))
    assert rstd[0] == best


def test_layernorm_matches_double_layer_norm():
    # a library routine in double: pins the formula (biased variance, eps
    # inside the root, gamma scaling and beta shift); K = 8 makes a (K - 1)
    # variance or eps outside the root visible
    import torch
    from oracle import layernorm as ln
    r = np.random.default_rng(31)
    for K, eps in ((8, 1e-5), (300, 1e-5), (4096, 1e-6)):
        x = (r.standard_normal((7, K)) * 3 + 1).astype(np.float32)
        g = (1 + 0.1 * r.standard_normal(K)).astype(np.float32)
        b = (0.1 * r.standard_normal(K)).astype(np.float32)
        y = ln.layernorm_f32(x, g, b, eps).astype(np.float64)
        t = torch.nn.functional.layer_norm(torch.from_numpy(x).double(), (K,),
                                           torch.from_numpy(g).double(),
                                           torch.from_numpy(b).double(), eps).numpy()
        np.testing.assert_allclose(y, t, rtol=3e-6, atol=3e-6)


def test_layernorm_with_folded_factors_emits_smoothed_activation():
    # LN with (gamma / s, beta / s) equals LN with (gamma, beta) divided by s
    from oracle import layernorm as ln
    import oracle as ref
    r = np.random.default_rng(32)
    K = 512
    x = r.standard_normal((5, K)).astype(np.float32)
    g = (1 + 0.1 * r.standard_normal(K)).astype(np.float32)
    b = (0.1 * r.standard_normal(K)).astype(np.float32)
    s = np.exp(r.standard_normal(K)).astype(np.float32)
    gf, bf = ref.fold_norm(s, g, b)
    y_fold = ln.layernorm_f32(x, gf, bf, 1e-5).astype(np.float64)
    y = ln.layernorm_f32(x, g, b, 1e-5).astype(np.float64) / s.astype(np.float64)
    np.testing.assert_allclose(y_fold, y, rtol=2e-6, atol=1e-6)


def test_layernorm_ambiguity_flag():
    from oracle import layernorm as ln
    one = np.float32(1.0)
    big = np.float32(2.0 ** 40)
    x = np.array([
        # mean 0.5 + 2^-25, an fp32 midpoint, from a sum that depends on the order
        [one, np.nextafter(one, np.float32(2)), big, -big],
        # mean 0.75, far from a midpoint; the sum is exact in any order
        [one, np.float32(2.0), big, -big],
        # mean 1 + 2^-24, a midpoint, but the sum is exact in any order: decided
        [one, np.nextafter(one, np.float32(2)), one, one]], np.float32)
    assert ln.ambiguous_rows(x, 1e-5) == [0]


def test_sum_exact_in_any_order_against_brute_force():
    # where the criterion holds, every summation order (sequential double adds
    # over random permutations) gives the correctly rounded sum; the first
    # row's sum does depend on the order
    import math
    from oracle import layernorm as ln
    import torch
    r = np.random.default_rng(34)
    a = np.array([1.0, 1.0 + 2.0 ** -23, 2.0 ** 40, -2.0 ** 40])
    assert not ln.sum_exact_in_any_order(a)
    sums = {float(np.cumsum(a[r.permutation(4)])[-1]) for _ in range(200)}
    assert len(sums) > 1
    rows = [torch.from_numpy(r.standard_normal(4096).astype(np.float32) * 20).half()
            .double().numpy(),
            torch.from_numpy(r.standard_normal(12288).astype(np.float32)).bfloat16()
            .double().numpy(),
            np.array([1.0, 2.0, 2.0 ** 40, -2.0 ** 40]), np.zeros(5)]
    for row in rows:
        assert ln.sum_exact_in_any_order(row)
        want = math.fsum(row.tolist())
        for _ in range(20):
            assert float(np.cumsum(row[r.permutation(row.size)])[-1]) == want


def test_layernorm_store_and_quantise_in_the_activation_dtype():
    import torch
    from oracle import layernorm as ln
    import oracle as ref
    r = np.random.default_rng(33)
    x = torch.from_numpy(r.standard_normal((6, 256)).astype(np.float32)).half()
    g = np.ones(256, np.float32)
    b = np.zeros(256, np.float32)
    xq, sx, y = ln.layernorm_quant_pertoken(x.float().numpy(), g, b, 1e-5, "f16")
    y32 = ln.layernorm_f32(x.float().numpy(), g, b, 1e-5)
    assert np.array_equal(y, torch.from_numpy(y32).half().float().numpy())
    xq2, sx2 = ref.quant_act_pertoken(y)
    assert np.array_equal(xq, xq2) and np.array_equal(sx, sx2)


# --------------------------------------------------------------------------
# Attention products: per-entry application of the pinned steps

def test_bmm_entries_are_independent_products(ref):
    from oracle.brute import gemm_int as brute_gemm
    r = np.random.default_rng(41)
    xq = r.integers(-127, 128, (3, 5, 9)).astype(np.int8)
    wq = r.integers(-127, 128, (3, 4, 9)).astype(np.int8)
    xq[1] = 127
    wq[2] = -127
    acc = ref.bmm_i32(xq, wq)
    for b in range(3):
        assert acc[b].tolist() == brute_gemm(xq[b].tolist(), wq[b].tolist())
    sx = r.random((3, 5)).astype(np.float32)
    sw = r.random((3, 4)).astype(np.float32)
    y = ref.bmm_dequant(acc, sx, sw)
    for b in range(3):
        assert np.array_equal(y[b], ref.dequant(acc[b], sx[b], sw[b]))


def test_batched_weight_quant_is_per_entry(ref):
    r = np.random.default_rng(42)
    w = r.standard_normal((4, 33, 7)).astype(np.float32)
    w[2, :, 3] = 0.0  # a zero channel in one entry only
    wq, sw = ref.quant_weight_perchannel_batched(w)
    for b in range(4):
        q1, s1 = ref.quant_weight_perchannel(w[b])
        assert np.array_equal(wq[b], q1) and np.array_equal(sw[b], s1)
    assert sw[2, 3] == 0.0 and not wq[2, 3].any()


def test_layernorm_admissible_stats_cover_every_summation_order():
    """The admissible (mu, rstd) of a row are the fp32 roundings reachable by
    double sums in any order: brute force over random permutations of rows
    whose sums depend on the order (sequential double adds, the mean and the
    centred sum of squares as the oracle forms them) lands in the set; an
    unflagged row has only its standard pair; a flagged one has more."""
    import math
    from oracle import layernorm as ln
    r = np.random.default_rng(35)
    eps = 1e-5
    rows = [np.array([2.0 ** 30, -2.0 ** 30, 1.0, 1.0 + 2.0 ** -23], np.float32),
            (r.standard_normal(64) * np.exp2(r.integers(-20, 24, 64))).astype(np.float32)]
    for row in rows:
        pairs = ln.admissible_stats(row, eps)
        assert pairs[0] == tuple(np.float32(v[0]) for v in ln.layernorm_stats(row[None], eps))
        v = row.astype(np.float64)
        K = v.size
        for _ in range(300):
            p = v[r.permutation(K)]
            mu_d = float(np.cumsum(p)[-1]) / K
            d = p - mu_d
            var_d = float(np.cumsum(d * d)[-1]) / K
            got = (np.float32(mu_d), np.float32(1.0 / math.sqrt(var_d + eps)))
            assert got in pairs, (got, pairs[:3])
    assert len(ln.admissible_stats(rows[0], eps)) > 1
    plain = r.standard_normal(256).astype(np.float16).astype(np.float32)
    assert ln.ambiguous_rows(plain[None], eps) == []
    assert ln.admissible_stats(plain, eps) == [tuple(np.float32(v[0]) for v in
                                                     ln.layernorm_stats(plain[None], eps))]
