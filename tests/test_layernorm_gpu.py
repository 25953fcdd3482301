"""GPU parity for sq_layernorm_quant_pertoken: the LayerNorm that carries the
folded smoothing factors, fused with per-token quantisation, against the
oracle (oracle/layernorm.py).

Bar: codes, steps and the stored LayerNorm output bit-exact on every row the
oracle does not flag as ambiguous (an exact statistic within the double
summation's error bound of an fp32 rounding boundary: more than one fp32
(mean, rstd) is correct there); a flagged row must equal, codes, step and
stored output together, the oracle's row under one of its admissible
statistics (``admissible_stats``).
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


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _inputs(M, K, dt, seed):
    """Residual-stream-like rows (a few persistent outlier channels), and the
    LayerNorm's gamma and beta divided by a smoothing vector."""
    r = np.random.default_rng([M, K, seed])
    cols = r.choice(K, min(6, K), replace=False).tolist()
    x = synth.random_matrix(seed, M, K, dt, outlier_cols=cols, factor=20.0)
    g = (1 + 0.1 * r.standard_normal(K)).astype(np.float32)
    b = (0.1 * r.standard_normal(K)).astype(np.float32)
    s = np.exp(0.5 * r.standard_normal(K)).astype(np.float32)
    gf, bf = ref.fold_norm(s, g, b)
    return x, gf, bf


def _check(dev, x, g, b, eps, dt):
    M, K = x.shape
    xd = x.contiguous().to(dev)
    gd, bd = torch.from_numpy(g).to(dev), torch.from_numpy(b).to(dev)
    xq, sx, xh = sq.layernorm_quant_pertoken(xd, gd, bd, eps, want_x_hat=True)
    xq2, sx2 = sq.layernorm_quant_pertoken(xd, gd, bd, eps)
    torch.cuda.synchronize()
    assert_equal(xq2, to_np(xq), "codes without x_hat")
    assert_equal(sx2, to_np(sx), "steps without x_hat")
    x32 = x.float().numpy()
    xq_r, sx_r, xh_r = lnref.layernorm_quant_pertoken(x32, g, b, eps, dt)
    amb = lnref.ambiguous_rows(x32, eps)
    ok = np.ones(M, bool)
    ok[amb] = False
    log("  ambiguous rows:", amb)
    g_xq, g_sx, g_xh = to_np(xq), to_np(sx), to_np(xh)
    assert_equal(g_xh[ok], xh_r[ok], "stored LayerNorm output")
    assert_equal(g_xq[ok], xq_r[ok], "codes")
    assert_equal(g_sx[ok], sx_r[ok], "steps")
    for m in amb:
        alts = lnref.row_alternatives(x32[m], g, b, eps, dt)
        hit = [i for i, (q, st, h) in enumerate(alts)
               if np.array_equal(g_xq[m], q) and g_sx[m] == st and np.array_equal(g_xh[m], h)]
        log("  row %d: %d admissible statistics, the GPU's is #%s" % (m, len(alts), hit))
        assert hit, "row %d equals none of its %d admissible results" % (m, len(alts))


CASES = [(1, 512, "f32"), (16, 4096, "f16"), (37, 1000, "f16"), (5, 1001, "bf16"),
         (300, 4096, "bf16"), (64, 12288, "f16"), (3, 16384, "f16"), (2, 65536, "f16"),
         (4, 16383, "f32"), (2, 32768, "f32"), (7, 3, "f16"), (129, 5120, "f16"),
         (2048, 4096, "f16"), (2048, 12288, "bf16")]


@pytest.mark.parametrize("M,K,dt", CASES)
def test_layernorm_quant(ref, dev, M, K, dt):
    log("layernorm_quant", M, K, dt)
    x, g, b = _inputs(M, K, dt, 7 * M + K)
    _check(dev, x, g, b, 1e-5, dt)


def test_layernorm_quant_constant_and_special_rows(ref, dev):
    # a constant row (variance 0: the output is beta), a zero row, a row with
    # one huge value, and ordinary rows
    K = 256
    r = np.random.default_rng(5)
    x = r.standard_normal((6, K)).astype(np.float32)
    x[0] = 3.25
    x[1] = 0.0
    x[2, 17] = 6.0e4
    g = np.ones(K, np.float32)
    b = (0.1 * r.standard_normal(K)).astype(np.float32)
    for dt in ("f32", "f16"):
        xt = torch.from_numpy(x)
        xt = xt.half() if dt == "f16" else xt
        _check(dev, xt, g, b, 1e-5, dt)


@pytest.mark.parametrize("cid", [2, 4])
def test_layernorm_quant_config(ref, dev, cid):
    """2048 tokens of the residual stream through the QKV layer's folded
    LayerNorm: OPT-6.7B-like (hidden 4096, fp16, 0.5% persistent outlier
    channels x60) and OPT-175B-like (hidden 12288, bf16); the calibration,
    smoothing and fold are the library's own."""
    cfg = synth.CONFIGS[cid]
    x = synth.activations(cfg, "qkv", 2048)
    xc = synth.activations(cfg, "qkv", cfg.T, calibration=True)
    w = synth.weight(cfg, "qkv")
    gamma, beta = synth.layernorm_params(cfg, "qkv")
    a = sq.calibrate_absmax(xc.to(dev))
    gd = torch.as_tensor(gamma, dtype=torch.float32).contiguous().to(dev)
    bd = torch.as_tensor(beta, dtype=torch.float32).contiguous().to(dev)
    sq.smooth_fold(a, w.to(dev), 0.5, gd, bd)
    torch.cuda.synchronize()
    _check(dev, x, to_np(gd), to_np(bd), 1e-5, cfg.act)
