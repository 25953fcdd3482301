"""GPU parity of sq_w8a8_linear_packed_ws: the few-token layer whose
quantiser also writes a fragment-packed copy of the codes, which the GEMM
reads (P1 推論方法: per-token dynamic quantisation, then the INT8 GEMM; P4
section 3: the scale multiplied back).  Codes and steps must equal the
oracle's per-token quantiser bit for bit, y must meet the output tolerance
against the oracle's double scale back and equal sq_w8a8_linear_packed bit
for bit; the workspace must hold exactly the packed layout of the codes
where it is used and stay untouched elsewhere."""
import numpy as np
import pytest
import torch

import synth
import w8a8_int8_post_amd as sq
from sqtest_util import assert_equal, assert_y_close, log

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
SENTINEL = 0x5A


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _weights(dev, N, K, seed):
    wq = synth.random_int8(seed, N, K)
    wq[0, :] = 127
    if N > 1:
        wq[N - 1, :] = -127
    sw = (np.random.default_rng([N, K, seed]).uniform(1e-4, 0.05, N) / 127).astype(np.float32)
    wp = sq.pack_weight(torch.from_numpy(wq).to(dev))
    return wq, sw, wp, torch.from_numpy(sw).to(dev)


def _packed_codes(xq_r, K):
    """The packed layout, written out from its definition: 64-byte k-group c
    of token row m, 16-byte piece g, at byte c * 1024 + (16 g + m) * 16."""
    M = xq_r.shape[0]
    out = np.full(16 * K, SENTINEL, dtype=np.uint8)
    v = xq_r.view(np.uint8)
    for m in range(M):
        for c in range(K // 64):
            for g in range(4):
                o = c * 1024 + (16 * g + m) * 16
                out[o:o + 16] = v[m, c * 64 + 16 * g:c * 64 + 16 * g + 16]
    return out


def _run(ref, dev, x, wq, sw, wp, sw_d, ydt, xq=None, sx=None, y=None, ws=None, what=""):
    M, K = x.shape
    N = wq.shape[0]
    need = sq.sq_linear_workspace_bytes(x.dtype, M, N, K)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws.fill_(SENTINEL)
    if xq is None:
        xq = torch.empty(M, K, dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        y = torch.empty(M, N, dtype=DT[ydt], device=dev)
    sq.sq_w8a8_linear_packed_ws(x, wp, sw_d, xq, sx, y, ws)
    torch.cuda.synchronize()
    xh = x.cpu()
    xq_r, sx_r = ref.quant_act_pertoken(xh if xh.dtype != torch.float32 else xh.numpy())
    assert_equal(xq, xq_r, "xq" + what)
    assert_equal(sx, sx_r, "x_scale" + what)
    acc_r = ref.gemm_i32(xq_r, wq)
    assert_y_close(y, ref.dequant(acc_r, sx_r, sw), "y" + what)
    y2, _, _ = sq.linear_w8a8_packed(x, wp, sw_d, y.dtype)
    torch.cuda.synchronize()
    iv = torch.int32 if y.dtype == torch.float32 else torch.int16
    assert_equal(y.cpu().view(iv), y2.cpu().view(iv).numpy(), "y vs sq_w8a8_linear_packed" + what)
    wsn = ws.cpu().numpy()
    if need > 0:
        assert need == 16 * K
        assert_equal(wsn[:need], _packed_codes(xq_r, K), "packed codes" + what)
    else:
        assert (wsn == SENTINEL).all(), "workspace touched by a shape that needs none"
    return need


# (M, N, K, x dtype, y dtype)
CASES = [
    (16, 8192, 28672, "f16", "f16"),    # 512 blocks: two per 8-wave workgroup (Llama-70B-like down)
    (16, 28672, 8192, "f16", "f16"),    # 1792 blocks: four per 4-wave workgroup (Llama-70B-like up)
    (13, 12288, 4096, "f16", "bf16"),   # 768 blocks in one round: four per 8-wave workgroup
    (14, 8200, 2048, "f32", "f32"),     # ragged last block
    (15, 12290, 1024, "bf16", "bf16"),  # ragged, four blocks per workgroup
    (16, 8192, 4096, "bf16", "f32"),
    (16, 8192, 28672, "f32", "f16"),    # fp32 rows of 7168 pieces
    (16, 4096, 16384, "f16", "f16"),    # 256 blocks, K >= 16384: the lean kernel on the packed copy
    (13, 4100, 16384, "bf16", "f32"),   # ragged last block
    (15, 16, 20480, "f32", "bf16"),     # one block
    # shapes that run as sq_w8a8_linear_packed (workspace untouched)
    (12, 8192, 4096, "f16", "f16"), (16, 4096, 4096, "f16", "f16"), (1, 4096, 4096, "f16", "f16"),
    (17, 8192, 1024, "f16", "f16"), (16, 8177, 32896, "f32", "f16"),  # fp32 row past 8192 pieces
]


@pytest.mark.parametrize("M,N,K,xdt,ydt", CASES)
def test_linear_packed_ws(ref, dev, M, N, K, xdt, ydt):
    log("linear_packed_ws", M, N, K, xdt, ydt)
    x = synth.random_matrix(13 * M + K + N, M, K, xdt, outlier_cols=[1, K - 3], factor=30.0).to(dev)
    wq, sw, wp, sw_d = _weights(dev, N, K, M * 3 + N + K)
    _run(ref, dev, x, wq, sw, wp, sw_d, ydt)


def test_linear_packed_ws_reused_buffers(ref, dev):
    """Calls in a row on the same xq / x_scale / y buffers and workspace with
    new activations each time."""
    M, N, K = 16, 8192, 16384
    wq, sw, wp, sw_d = _weights(dev, N, K, 5)
    ws = sq.linear_workspace(torch.float16, M, N, K, dev)
    xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty(M, N, dtype=torch.float16, device=dev)
    for i in range(3):
        x = synth.random_matrix(500 + i, M, K, "f16", scale=10.0 ** (i - 1),
                                outlier_cols=[i, K - 1 - i], factor=40.0).to(dev)
        assert _run(ref, dev, x, wq, sw, wp, sw_d, "f16", xq, sx, y, ws, " (call %d)" % i) > 0


@pytest.mark.parametrize("M,pattern", [(13, (0.0, 1e-40, 1e31, 1.0)), (16, (0.0, 1e-40, 1e31, 1.0) * 4)])
def test_linear_packed_ws_special_rows(ref, dev, M, pattern):
    """Zero rows (step 0), subnormal steps and steps above 2^96 (the IEEE
    division path) with the packed copy."""
    K, N = 2048, 8200
    scale = np.resize(np.array(pattern), M)[:, None]
    x = torch.from_numpy((np.random.default_rng(16 + M).standard_normal((M, K)) * scale)
                         .astype(np.float32)).to(dev)
    wq, sw, wp, sw_d = _weights(dev, N, K, 21)
    assert _run(ref, dev, x, wq, sw, wp, sw_d, "f32") > 0


def test_linear_packed_ws_graph_replays(ref, dev):
    """The call captured in a HIP graph and replayed with new activations
    copied in between (eager work and a sync between replays): every replay
    matches the oracle and sq_w8a8_linear_packed."""
    M, N, K = 16, 12288, 4096
    wq, sw, wp, sw_d = _weights(dev, N, K, 77)
    ws = sq.linear_workspace(torch.float16, M, N, K, dev)
    x = torch.empty(M, K, dtype=torch.float16, device=dev)
    xq = torch.empty(M, K, dtype=torch.int8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty(M, N, dtype=torch.float16, device=dev)
    x.copy_(synth.random_matrix(700, M, K, "f16").to(dev))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sq.sq_w8a8_linear_packed_ws(x, wp, sw_d, xq, sx, y, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sq.sq_w8a8_linear_packed_ws(x, wp, sw_d, xq, sx, y, ws)
    torch.cuda.synchronize()
    for i in range(4):
        x.copy_(synth.random_matrix(701 + i, M, K, "f16", outlier_cols=[3 * i], factor=50.0).to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        xq_r, sx_r = ref.quant_act_pertoken(x.cpu())
        assert_equal(xq, xq_r, "xq (replay %d)" % i)
        assert_equal(sx, sx_r, "x_scale (replay %d)" % i)
        assert_y_close(y, ref.dequant(ref.gemm_i32(xq_r, wq), sx_r, sw), "y (replay %d)" % i)
