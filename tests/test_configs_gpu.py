"""Full-size parity on the five workload configurations.

Every stage runs on the GPU at the real layer shapes and token counts (the
same entry points and launch configurations the benchmark times).  The CPU
oracle then recomputes, from the same seeded inputs, what it can afford one
by one: the full calibration vector and smoothing factors, sampled rows of the
folded weight, sampled output channels of the quantised weight (whole
columns), sampled tokens of the smoothed and quantised activations, and the
accumulators and outputs at every (sampled token, sampled channel) pair.
Configurations:

  1 toy 512x512, 16 tokens (fully compared in test_parity_gpu.py)
  2 OPT-6.7B-like QKV/FC1/FC2, fp16, tokens 1, 16, 512, 2048
  3 OPT-13B-like QKV/FC1/FC2, fp16, 4096 tokens, alpha 0.4/0.5/0.6/0.75
  4 OPT-175B-like QKV/FC1/FC2, bf16, tokens 2048, 8192
  5 Llama-70B-like up/down, fp16, tokens 1, 4, 8, 16
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_int8_post_amd as sq
from sqtest_util import assert_equal, assert_y_close, f32_ulp_diff, log, to_np

pytestmark = pytest.mark.gpu

CASES = [(c, ly.name) for c in (2, 3, 4, 5) for ly in synth.CONFIGS[c].layers]
NSAMPLE = 48


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _sample(n, k, seed):
    if n <= k:
        return np.arange(n)
    idx = np.random.default_rng(seed).choice(n - 2, k - 2, replace=False) + 1
    return np.sort(np.concatenate([[0, n - 1], idx]))


@pytest.mark.parametrize("cid,layer", CASES)
def test_config_layer(ref, dev, cid, layer):
    cfg = synth.CONFIGS[cid]
    ly = cfg.layer(layer)
    K, N = ly.K, ly.N
    ydt = synth.DTYPES[cfg.ydt]
    log("config %d %s: K=%d N=%d tokens=%s alphas=%s" % (cid, layer, K, N, cfg.M, cfg.alphas))

    w = synth.weight(cfg, layer)
    xc = synth.activations(cfg, layer, cfg.T, calibration=True)
    xe = synth.activations(cfg, layer, max(cfg.M))
    w_d, xc_d, xe_d = w.to(dev), xc.to(dev), xe.to(dev)

    # oracle pieces that are cheap at full size
    a_r = ref.calibrate_absmax(xc)
    w32 = w.float().numpy()
    b_r = ref.weight_row_absmax(w32)
    cols = _sample(N, NSAMPLE, 1000 * cid + N)
    wrows = _sample(K, NSAMPLE, 2000 * cid + K)

    a = sq.calibrate_absmax(xc_d)
    torch.cuda.synchronize()
    assert_equal(a, a_r, "calibration absmax")

    for alpha in cfg.alphas:
        s, w_hat = sq.smooth_fold(a, w_d, alpha)
        wq, sw = sq.quant_weight_perchannel(w_hat)
        torch.cuda.synchronize()
        s_r = ref.smoothing_factors(a_r, b_r, alpha)
        d = f32_ulp_diff(to_np(s), s_r)
        assert d.max() <= 1, "s differs by %d ulp" % d.max()
        # the downstream comparisons below assume the two s vectors agree
        assert (d == 0).all(), "s differs by one ulp in %d channels" % int((d != 0).sum())
        assert_equal(w_hat[torch.from_numpy(wrows).to(dev)],
                     ref.fold_weight(w32[wrows], s_r[wrows]), "W_hat rows")
        # whole columns of W_hat for the sampled output channels
        wq_r, sw_r = ref.quant_weight_perchannel(ref.fold_weight(w32[:, cols], s_r))
        cols_d = torch.from_numpy(cols).to(dev)
        assert_equal(wq[cols_d], wq_r, "Wq (sampled channels)")
        assert_equal(sw[cols_d], sw_r, "w_scale (sampled channels)")
        wp = sq.pack_weight(wq)

        for M in cfg.M:
            x_hat = sq.smooth_activation(xe_d[:M].contiguous(), s)
            xq, sx = sq.quant_act_pertoken(x_hat)
            y = torch.empty(M, N, dtype=ydt, device=dev)
            sq.sq_w8a8_gemm_dequant(xq, sx, wq, sw, y)
            acc = sq.w8a8_gemm_i32(xq, wq)
            y_p = torch.empty(M, N, dtype=ydt, device=dev)
            sq.sq_w8a8_gemm_dequant_packed(xq, sx, wp, sw, N, y_p)
            acc_p = sq.w8a8_gemm_i32_packed(xq, wp, N)
            # the one-call layer (a single fused kernel at M <= 2 and M * K <= 16384)
            y_f, xq_f, sx_f = sq.linear_w8a8_packed(x_hat, wp, sw, ydt)
            torch.cuda.synchronize()
            rows = _sample(M, NSAMPLE, 3000 * cid + M)
            rows_d = torch.from_numpy(rows).to(dev)
            xh_r = ref.smooth_activation(xe[torch.from_numpy(rows)], s_r)
            xh_r16 = torch.from_numpy(xh_r).to(synth.DTYPES[cfg.act])
            assert_equal(x_hat[rows_d].cpu().view(torch.int16), xh_r16.view(torch.int16).numpy(),
                         "X_hat bits (sampled tokens)")
            xq_r, sx_r = ref.quant_act_pertoken(xh_r16)
            assert_equal(xq[rows_d], xq_r, "Xq (sampled tokens)")
            assert_equal(sx[rows_d], sx_r, "x_scale (sampled tokens)")
            acc_r = ref.gemm_i32(xq_r, wq_r)
            assert_equal(acc[rows_d][:, cols_d], acc_r, "acc (sampled)")
            assert_equal(acc_p[rows_d][:, cols_d], acc_r, "acc, packed weights (sampled)")
            y_r = ref.dequant(acc_r, sx_r, sw_r)
            same = assert_y_close(y[rows_d][:, cols_d], y_r, "y")
            assert_y_close(y_p[rows_d][:, cols_d], y_r, "y, packed weights")
            assert_equal(xq_f[rows_d], xq_r, "Xq (one-call layer)")
            assert_equal(sx_f[rows_d], sx_r, "x_scale (one-call layer)")
            assert_y_close(y_f[rows_d][:, cols_d], y_r, "y (one-call layer)")
            # every path rounds RN(RN(fp32(acc) * sx) * sw) once to the output dtype
            y32 = torch.from_numpy(ref.dequant_bias_act_f32(acc_r, sx_r, sw_r)).to(ydt)
            for yy, nm in ((y, "y"), (y_p, "y, packed"), (y_f, "y, one-call")):
                assert_equal(yy[rows_d][:, cols_d].cpu().view(torch.int16),
                             y32.view(torch.int16).numpy(), nm + " (fp32 order, bits)")
            log("  alpha %.2f M %5d: ok (y bit-equal to RNE(oracle) %.4f)" % (alpha, M, same))
            del x_hat, xq, sx, y, acc, y_p, acc_p, y_f, xq_f, sx_f
        del s, w_hat, wq, sw, wp
        torch.cuda.empty_cache()
