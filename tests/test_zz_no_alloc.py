"""The allocation-free split-K entry point (sq_w8a8_gemm_dequant_packed_noalloc,
for callers that cannot allocate: graph capture, serving loops) against the
workspace form sq_w8a8_gemm_dequant_packed_ws on the same inputs: bit-equal
outputs on two calls in a row (the second smaller, so the shared static
scratch holds the first call's partial sums and counters when it starts),
and the oracle on the first call's outputs."""
import numpy as np
import pytest
import torch

import synth
import w8a8_int8_post_amd as sq
from sqtest_util import assert_equal, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _layer(dev, M, N, K, seed):
    xq = synth.random_int8(seed, M, K)
    wq = synth.random_int8(seed + 1, N, K)
    r = np.random.default_rng([M, N, K, seed])
    sx = (r.uniform(0.01, 2.0, M) / 127).astype(np.float32)
    sw = (r.uniform(1e-4, 0.05, N) / 127).astype(np.float32)
    d = [torch.from_numpy(a).contiguous().to(dev) for a in (xq, sx, wq, sw)]
    return (xq, sx, wq, sw), d[0], d[1], sq.pack_weight(d[2]), d[3]


# (first call, second call): both split K (the second with fewer tiles,
# splits or a different K range), then a shape the library does not split
PAIRS = [((128, 4096, 16384), (65, 2048, 12288)),    # 4 splits, then 4 of fewer tiles
         ((256, 4096, 28672), (128, 4096, 16384)),   # 2 splits, then 4
         ((65, 8192, 49152), (70, 300, 24576))]      # 2 splits, then 8 of 5 tiles


@pytest.mark.parametrize("first,second", PAIRS)
@pytest.mark.parametrize("ydt", [torch.float16, torch.bfloat16])
def test_noalloc_matches_workspace_form(ref, dev, first, second, ydt):
    for i, (M, N, K) in enumerate((first, second)):
        log("noalloc call %d: M=%d N=%d K=%d %s" % (i, M, N, K, ydt))
        need = sq.sq_gemm_workspace_bytes(M, N, K)
        assert 0 < need <= sq.sq_noalloc_scratch_bytes()
        host, xq, sx, wp, sw = _layer(dev, M, N, K, 7 * M + N + K)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        y_ws = torch.empty(M, N, dtype=ydt, device=dev)
        y_na = torch.empty(M, N, dtype=ydt, device=dev)
        sq.sq_w8a8_gemm_dequant_packed_ws(xq, sx, wp, sw, N, y_ws, ws)
        sq.sq_w8a8_gemm_dequant_packed_noalloc(xq, sx, wp, sw, N, y_na)
        torch.cuda.synchronize()
        assert_equal(y_na.cpu().view(torch.int16), y_ws.cpu().view(torch.int16).numpy(),
                     "noalloc vs workspace form (call %d)" % i)
        if i == 0:  # the oracle on sampled rows x all channels
            xq_h, sx_h, wq_h, sw_h = host
            rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 14)])
            acc = ref.gemm_i32(xq_h[rows], wq_h)
            y32 = torch.from_numpy(ref.dequant_bias_act_f32(acc, sx_h[rows], sw_h)).to(ydt)
            assert_equal(y_na.cpu()[torch.from_numpy(rows)].view(torch.int16),
                         y32.view(torch.int16).numpy(), "noalloc vs oracle (fp32 order, bits)")


def test_noalloc_unsplit_shape_is_plain_gemm(dev):
    M, N, K = 512, 4096, 4096
    assert sq.sq_gemm_workspace_bytes(M, N, K) == 0
    _, xq, sx, wp, sw = _layer(dev, M, N, K, 3)
    y0 = torch.empty(M, N, dtype=torch.float16, device=dev)
    y1 = torch.empty_like(y0)
    sq.sq_w8a8_gemm_dequant_packed(xq, sx, wp, sw, N, y0)
    sq.sq_w8a8_gemm_dequant_packed_noalloc(xq, sx, wp, sw, N, y1)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
