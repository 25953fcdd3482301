"""GPU parity for the split-K entry points (sq_w8a8_gemm_dequant_ws and
sq_w8a8_gemm_dequant_packed_ws): few tokens against narrow, deep layers,
where K is split into 2, 4 or 8 ranges whose int32 partial products meet in
a caller-owned workspace (128 x 64 output tiles, two wave groups per
workgroup, each over half of its split's range).

Bar: outputs bit-equal to the oracle's fp32 evaluation of the scale back
(RN(RN(fp32(acc) * sx) * sw), one rounding to the output dtype) and to the
plain entry point's; one zero-filled workspace serves every call of the
module in turn (its counters must be back at zero after each call).
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_int8_post_amd as sq
from sqtest_util import assert_equal, log

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def workspace(dev):
    need = max(sq.sq_gemm_workspace_bytes(M, N, K) for M, N, K, _ in CASES)
    return torch.zeros(need + 256, dtype=torch.uint8, device=dev)


CASES = [
    # split: 128 x 64 output tiles at most half the CUs, K >= 8192, K % 256 == 0;
    # 2, 4 or 8 splits with tiles x splits <= the CUs and K / splits >= 2048
    (65, 4096, 16384, "f16"),     # 64 tiles: 4 splits
    (128, 1000, 8192, "bf16"),    # 16 tiles: 4 splits of 2048
    (128, 1000, 12288, "bf16"),   # 16 tiles: 4 splits of 3072
    (300, 4100, 8192, "f32"),     # 195 tiles: no split
    (100, 4100, 12288, "f32"),    # ragged M and N tiles, 65 tiles: 2 splits
    (300, 1000, 28672, "f32"),    # ragged M and N tiles above 256 tokens, 48 tiles: 4 splits
    (512, 4096, 16384, "f16"),    # 256 tiles, one per CU: no split (the plain kernel)
    (128, 4096, 16384, "bf16"),   # 64 tiles: 4 splits
    (512, 4096, 28672, "f16"),    # 256 tiles: no split
    (100, 8192, 28672, "bf16"),   # 128 tiles: 2 splits
    (129, 2048, 9216, "f16"),     # 64 tiles: 4 splits of 2304 (two groups of 9 k-tiles)
    (120, 2048, 13824, "f16"),    # 32 tiles; K = 54 x 256: 2 splits of 6912
    (128, 1024, 16384, "f16"),    # 16 tiles: 8 splits
    (70, 300, 24576, "bf16"),     # 5 tiles, N % 64 != 0: 8 splits
    (128, 1000, 8320, "f16"),     # K % 256 != 0: no split (the plain 64-deep two-group form)
    (1000, 4096, 8192, "f16"),    # 512 tiles: no split
    (100, 12288, 4096, "bf16"),   # K < 8192: no split
    (2048, 4096, 16384, "f16"),   # 1024 tiles: no split (the plain GEMM)
    (16, 4096, 16384, "f16"),     # few tokens: no split
    (200, 1002, 16384, "f16"),    # N % 4 != 0: no split
    # the plain entry points on deep layers: 128 x 64 tiles (at most one per
    # CU) or 128 x 128 tiles, two wave groups over K
    (129, 8320, 16384, "f16"),    # 260 narrow tiles, 130 wide: the 128 x 128 form
    (700, 4096, 16384, "bf16"),   # 192 wide tiles: the 128 x 128 form
    (300, 5120, 20480, "f16"),    # 240 narrow tiles: no split
    (65, 12288, 49152, "bf16"),   # 192 narrow tiles, K = 49152: no split
    (200, 28672, 8192, "f16"),    # 129-256 rows, wide and deep: 224 tiles of 256 x 128
    (160, 36864, 12288, "bf16"),  # 129-256 rows: 144 tiles of 256 x 256
]


def _inputs(M, N, K, seed):
    xq = synth.random_int8(seed, M, K)
    wq = synth.random_int8(seed + 1, N, K)
    r = np.random.default_rng([M, N, K, seed])
    sx = (r.uniform(0.01, 2.0, M) / 127).astype(np.float32)
    sw = (r.uniform(1e-4, 0.05, N) / 127).astype(np.float32)
    return xq, wq, sx, sw


def _check_counters(workspace):
    # the tile counters (the workspace's first 4096 int32) are zero between calls
    assert int(workspace[:4 * 4096].count_nonzero()) == 0, "tile counters not back at zero"


@pytest.mark.parametrize("M,N,K,ydt", CASES)
@pytest.mark.parametrize("packed", [True, False])
def test_splitk_gemm_dequant(ref, dev, workspace, M, N, K, ydt, packed):
    need = sq.sq_gemm_workspace_bytes(M, N, K)
    log("split-K", M, N, K, ydt, "packed" if packed else "row-major", "workspace", need)
    xq, wq, sx, sw = _inputs(M, N, K, 7 * M + N + K)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    xq_d, wq_d, sx_d, sw_d = g(xq), g(wq), g(sx), g(sw)
    y = torch.empty(M, N, dtype=DT[ydt], device=dev)
    y0 = torch.empty(M, N, dtype=DT[ydt], device=dev)
    if packed:
        wp = sq.pack_weight(wq_d)
        for _ in range(2):  # a second call on the same workspace
            sq.sq_w8a8_gemm_dequant_packed_ws(xq_d, sx_d, wp, sw_d, N, y, workspace)
        sq.sq_w8a8_gemm_dequant_packed(xq_d, sx_d, wp, sw_d, N, y0)
    else:
        for _ in range(2):
            sq.sq_w8a8_gemm_dequant_ws(xq_d, sx_d, wq_d, sw_d, y, workspace)
        sq.sq_w8a8_gemm_dequant(xq_d, sx_d, wq_d, sw_d, y0)
    torch.cuda.synchronize()
    _check_counters(workspace)
    bits = torch.int16 if ydt != "f32" else torch.int32
    assert torch.equal(y.view(bits), y0.view(bits)), "split-K differs from the plain GEMM"
    # the oracle: every output when small, else sampled rows x columns
    if M * N * K <= 2e9:
        rows, cols = np.arange(M), np.arange(N)
        acc = ref.gemm_i32(xq, wq)
    else:
        r = np.random.default_rng(M + N)
        rows = np.sort(np.concatenate([[0, M - 1], r.choice(M, 30, replace=False)]))
        cols = np.sort(np.concatenate([[0, N - 1], r.choice(N, 30, replace=False)]))
        acc = ref.gemm_i32_sampled(xq, wq, rows, cols)
    y32 = torch.from_numpy(ref.dequant_bias_act_f32(acc, sx[rows], sw[cols])).to(DT[ydt])
    got = y.cpu()[torch.from_numpy(rows)][:, torch.from_numpy(cols)]
    assert_equal(got.view(bits), y32.view(bits).numpy(), "y (fp32 order, bits)")


def test_splitk_workspace_errors(dev):
    M, N, K = 128, 4096, 16384
    xq = torch.zeros(M, K, dtype=torch.int8, device=dev)
    wp = sq.pack_weight(torch.zeros(N, K, dtype=torch.int8, device=dev))
    sx = torch.ones(M, device=dev)
    sw = torch.ones(N, device=dev)
    y = torch.empty(M, N, dtype=torch.float16, device=dev)
    small = torch.zeros(1024, dtype=torch.uint8, device=dev)
    for ws in (small, None):
        with pytest.raises(sq.SQError) as ei:
            sq.sq_w8a8_gemm_dequant_packed_ws(xq, sx, wp, sw, N, y, ws)
        assert ei.value.code == 11 and "SQ_ERR_WORKSPACE" in str(ei.value)
