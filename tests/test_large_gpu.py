"""Tensors past 2^31 elements: every offset into them must be 64-bit.

The GEMM's outputs (M x N), the per-token quantiser's and the fused
LayerNorm quantiser's inputs and codes (M x K), the calibration maxima over
T x K, and both weight quantisers (the transposing one for K > 8192, the
one-pass one for K <= 8192) each on more than 2^31 elements.  Inputs are drawn
on the device from a seeded generator (a host draw of 2^31 values would take
minutes); the rows or columns the oracle checks, always including the last
ones, are copied back and compared bit for bit: codes, steps, and 16-bit
outputs rounded from the oracle's fp32 evaluation of the scale back.
"""
import numpy as np
import pytest
import torch

import synth
import oracle as ref
from oracle import layernorm as lnref
import w8a8_int8_post_amd as sq
from sqtest_util import assert_equal, log, to_np

pytestmark = pytest.mark.gpu

TWO31 = 1 << 31


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _pick(n, k, seed):
    r = np.random.default_rng([n, seed])
    edge = [0, 1, n // 2, n - 2, n - 1]
    return np.unique(np.concatenate([edge, r.choice(n, k, replace=False)])).astype(np.int64)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("K", [128, 256])
@pytest.mark.parametrize("packed", [True, False])
def test_gemm_outputs_past_2g(dev, K, packed):
    M, N = 65600, 32800
    assert M * N > TWO31
    log("gemm past 2^31 outputs", M, N, K, "packed" if packed else "row-major")
    xq = synth.device_int8(1, M, K, dev)
    wq = synth.device_int8(2, N, K, dev)
    r = np.random.default_rng([M, N, K])
    sx_h = (r.uniform(0.01, 2.0, M) / 127).astype(np.float32)
    sw_h = (r.uniform(1e-4, 0.05, N) / 127).astype(np.float32)
    sx, sw = torch.from_numpy(sx_h).to(dev), torch.from_numpy(sw_h).to(dev)
    y = torch.empty(M, N, dtype=torch.float16, device=dev)
    if packed:
        sq.sq_w8a8_gemm_dequant_packed(xq, sx, sq.pack_weight(wq), sw, N, y)
    else:
        sq.sq_w8a8_gemm_dequant(xq, sx, wq, sw, y)
    torch.cuda.synchronize()
    xq_h, wq_h = xq.cpu().numpy(), wq.cpu().numpy()
    # a grid of sampled rows x columns, and the last two rows whole
    for rows, cols in ((_pick(M, 24, 1), _pick(N, 40, 2)),
                       (np.array([M - 2, M - 1]), np.arange(N))):
        acc = ref.gemm_i32_sampled(xq_h, wq_h, rows, cols)
        want = torch.from_numpy(ref.dequant_bias_act_f32(acc, sx_h[rows], sw_h[cols])).half()
        got = y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)].cpu()
        assert_equal(got.view(torch.int16), want.view(torch.int16).numpy(), "y bits")
    del xq, wq, y
    _free()


def test_quant_act_and_calibration_past_2g(dev):
    M, K = 65600, 32800
    assert M * K > TWO31
    log("per-token quantiser and calibration past 2^31 inputs", M, K)
    x = synth.device_matrix(3, M, K, "f16", dev, outlier_cols=[0, 7, K // 3, K - 1], factor=50.0)
    x[M - 3].zero_()  # an all-zero token near the end: step 0, codes 0
    xq, sx = sq.quant_act_pertoken(x)
    a = sq.calibrate_absmax(x)
    torch.cuda.synchronize()
    rows = _pick(M, 24, 3)
    rows = np.unique(np.concatenate([rows, [M - 3]]))
    rt = torch.from_numpy(rows).to(dev)
    xq_r, sx_r = ref.quant_act_pertoken(x[rt].float().cpu().numpy())
    assert_equal(sx[rt], sx_r, "x_scale")
    assert_equal(xq[rt], xq_r, "xq")
    # the column maxima: a max is exact in any order, so torch's reduction of
    # the same fp16 values is an independent check at this size
    assert_equal(a, x.abs().amax(dim=0).float().cpu().numpy(), "calibration maxima")
    del x, xq, sx
    _free()


def test_layernorm_quant_past_2g(dev):
    M, K = 131100, 16400
    assert M * K > TWO31
    log("fused LayerNorm quantiser past 2^31 inputs", M, K)
    x = synth.device_matrix(4, M, K, "f16", dev, outlier_cols=[5, K // 2, K - 2], factor=20.0)
    r = np.random.default_rng([M, K])
    g = (1 + 0.1 * r.standard_normal(K)).astype(np.float32)
    b = (0.1 * r.standard_normal(K)).astype(np.float32)
    xq, sx, xh = sq.layernorm_quant_pertoken(x, torch.from_numpy(g).to(dev),
                                             torch.from_numpy(b).to(dev), 1e-5, want_x_hat=True)
    torch.cuda.synchronize()
    rows = _pick(M, 24, 4)
    rt = torch.from_numpy(rows).to(dev)
    x32 = x[rt].float().cpu().numpy()
    xq_r, sx_r, xh_r = lnref.layernorm_quant_pertoken(x32, g, b, 1e-5, "f16")
    ok = np.ones(len(rows), bool)
    ok[lnref.ambiguous_rows(x32, 1e-5)] = False
    log("  rows flagged ambiguous:", int((~ok).sum()))
    assert ok.sum() >= len(rows) - 2
    assert_equal(to_np(xh[rt])[ok], xh_r[ok], "stored LayerNorm output")
    assert_equal(to_np(xq[rt])[ok], xq_r[ok], "codes")
    assert_equal(to_np(sx[rt])[ok], sx_r[ok], "steps")
    del x, xq, sx, xh
    _free()


@pytest.mark.parametrize("K,N", [(65600, 32800),    # transposing quantiser (K > 8192)
                                 (8192, 262208)])   # one-pass quantiser
def test_quant_weight_past_2g(dev, K, N):
    assert K * N > TWO31
    log("weight quantiser past 2^31 weights", K, N)
    w = synth.device_matrix(5, K, N, "f16", dev, scale=0.02)
    w[:, N - 3].zero_()  # an all-zero output channel near the end
    wq, sw = sq.quant_weight_perchannel(w)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([_pick(N, 24, 5), [N - 3]]))
    ct = torch.from_numpy(cols).to(dev)
    wq_r, sw_r = ref.quant_weight_perchannel(w[:, ct].float().cpu().numpy())
    assert_equal(sw[ct], sw_r, "w_scale")
    assert_equal(wq[ct], wq_r, "wq")
    del w, wq, sw
    _free()
