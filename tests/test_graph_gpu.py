"""The run-time entry points under HIP-graph capture.

One graph records the whole run-time path: the per-token quantiser and the
packed GEMM of a prefill layer, the one-call decode layer (2 tokens), the
quantiser and the 4-block packed GEMM at 16 tokens, the fused LayerNorm +
quantisation, the dynamic per-tensor quantiser (partial maxima, reduction,
codes), both attention products (the one-stage K = 128 product and P V),
both forms of the batched per-channel quantiser (the one-pass kernel, and
zero fill + atomic column maxima + transposing quantiser) and the split-K
GEMM (its tile counters reset by the last split of each tile).  The graph is
replayed four times, each time on new inputs copied into its buffers, with
eager calls and synchronisations in between; every replay must give, bit for
bit, what the same calls give eagerly on the same inputs.  The library
records no memset nodes: every buffer that must start at zero is cleared by a
kernel of its own.
"""
import numpy as np
import pytest
import torch

import synth
import w8a8_int8_post_amd as sq
from sqtest_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.load_library()
    return torch.device("cuda:0")


def _i8(seed, *shape):
    r = np.random.default_rng([77, seed])
    return torch.from_numpy(r.integers(-127, 128, size=shape, dtype=np.int16).astype(np.int8))


def test_graph_replay_matches_eager(dev):
    K, N, M = 4096, 1000, 300
    f16 = torch.float16
    # weights: quantised and packed once, eagerly
    w = synth.random_matrix(5, K, N, "f16", scale=0.02).to(dev)
    wq, sw = sq.quant_weight_perchannel(w)
    wp = sq.pack_weight(wq)
    gamma = torch.from_numpy(np.random.default_rng(6).uniform(0.5, 1.5, K).astype(np.float32)).to(dev)
    beta = torch.from_numpy(np.random.default_rng(7).uniform(-0.1, 0.1, K).astype(np.float32)).to(dev)
    H, S, D = 4, 256, 128

    # input buffers the graph reads (refilled before every replay)
    ins = {
        "x": torch.empty(M, K, dtype=f16, device=dev),
        "x2": torch.empty(2, K, dtype=f16, device=dev),
        "x16": torch.empty(16, K, dtype=f16, device=dev),
        "qq": torch.empty(H, S, D, dtype=torch.int8, device=dev),
        "kq": torch.empty(H, S, D, dtype=torch.int8, device=dev),
        "pq": torch.empty(H, S, S, dtype=torch.int8, device=dev),
        "v": torch.empty(H, S, 64, dtype=f16, device=dev),
        "v_odd": torch.empty(3, 100, 40, dtype=f16, device=dev),
    }
    # a deep, narrow layer at 128 tokens: the split-K form (8 splits), whose
    # tile counters must be back at zero for every replay
    Ks, Ns, Ms = 16384, 1024, 128
    wsk = sq.pack_weight(_i8(11, Ns, Ks).to(dev))
    sx_sk = torch.from_numpy(np.random.default_rng(12).uniform(1e-3, 2e-2, Ms).astype(np.float32)).to(dev)
    sw_sk = torch.from_numpy(np.random.default_rng(13).uniform(1e-4, 1e-3, Ns).astype(np.float32)).to(dev)
    assert sq.sq_gemm_workspace_bytes(Ms, Ns, Ks) > 0
    workspace = sq.gemm_workspace(Ms, Ns, Ks, dev)
    ins["xsk"] = torch.empty(Ms, Ks, dtype=torch.int8, device=dev)
    sxa = torch.from_numpy(np.random.default_rng(8).uniform(1e-3, 2e-2, (H, S)).astype(np.float32)).to(dev)
    vq_scores = torch.from_numpy(np.random.default_rng(9).uniform(1e-3, 2e-2, (H, D)).astype(np.float32)).to(dev)
    vq_pv = _i8(10, H, D, S).to(dev)

    def outputs():
        return {
            "xq": torch.empty(M, K, dtype=torch.int8, device=dev),
            "sx": torch.empty(M, dtype=torch.float32, device=dev),
            "y": torch.empty(M, N, dtype=f16, device=dev),
            "xq2": torch.empty(2, K, dtype=torch.int8, device=dev),
            "sx2": torch.empty(2, dtype=torch.float32, device=dev),
            "y2": torch.empty(2, N, dtype=f16, device=dev),
            "xq16": torch.empty(16, K, dtype=torch.int8, device=dev),
            "sx16": torch.empty(16, dtype=torch.float32, device=dev),
            "y16": torch.empty(16, N, dtype=f16, device=dev),
            "lq": torch.empty(M, K, dtype=torch.int8, device=dev),
            "ls": torch.empty(M, dtype=torch.float32, device=dev),
            "lh": torch.empty(M, K, dtype=f16, device=dev),
            "tq": torch.empty(M, K, dtype=torch.int8, device=dev),
            "ts": torch.empty(M, dtype=torch.float32, device=dev),
            "scores": torch.empty(H, S, S, dtype=f16, device=dev),
            "o": torch.empty(H, S, D, dtype=f16, device=dev),
            "vq": torch.empty(H, 64, S, dtype=torch.int8, device=dev),
            "vs": torch.empty(H, 64, dtype=torch.float32, device=dev),
            "vq_odd": torch.empty(3, 40, 100, dtype=torch.int8, device=dev),
            "vs_odd": torch.empty(3, 40, dtype=torch.float32, device=dev),
            "ysk": torch.empty(Ms, Ns, dtype=f16, device=dev),
        }

    def run(o):
        sq.sq_quant_act_pertoken(ins["x"], o["xq"], o["sx"])
        sq.sq_w8a8_gemm_dequant_packed(o["xq"], o["sx"], wp, sw, N, o["y"])
        sq.sq_w8a8_linear_packed(ins["x2"], wp, sw, o["xq2"], o["sx2"], o["y2"])
        sq.sq_quant_act_pertoken(ins["x16"], o["xq16"], o["sx16"])
        sq.sq_w8a8_gemm_dequant_packed(o["xq16"], o["sx16"], wp, sw, N, o["y16"])
        sq.sq_layernorm_quant_pertoken(ins["x"], gamma, beta, 1e-5, o["lq"], o["ls"], o["lh"])
        sq.sq_quant_act_pertensor(ins["x"], o["tq"], o["ts"])
        sq.sq_w8a8_bmm_dequant(ins["qq"], sxa, ins["kq"], sxa, o["scores"])
        sq.sq_w8a8_bmm_dequant(ins["pq"], sxa, vq_pv, vq_scores, o["o"])
        sq.sq_quant_weight_perchannel_batched(ins["v"], o["vq"], o["vs"])
        sq.sq_quant_weight_perchannel_batched(ins["v_odd"], o["vq_odd"], o["vs_odd"])
        sq.sq_w8a8_gemm_dequant_packed_ws(ins["xsk"], sx_sk, wsk, sw_sk, Ns, o["ysk"], workspace)

    def refill(seed):
        r = np.random.default_rng([55, seed])
        for name, t in ins.items():
            if t.dtype == torch.int8:
                t.copy_(_i8(seed * 997 + sum(map(ord, name)), *t.shape))
            else:
                z = r.standard_normal(tuple(t.shape), dtype=np.float32)
                if name in ("x", "x2", "x16"):
                    z[..., [3, 700, 2049]] *= 40.0  # persistent outlier channels
                t.copy_(torch.from_numpy(z).to(f16))

    graph_out = outputs()
    refill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(graph_out)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(graph_out)

    eager_out = outputs()
    prev = None
    for rep in range(4):
        refill(rep + 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        snap = {k: v.clone() for k, v in graph_out.items()}
        run(eager_out)
        torch.cuda.synchronize()
        for k in snap:
            a, b = snap[k], eager_out[k]
            if a.dtype in (torch.float16, torch.bfloat16):
                a, b = a.view(torch.int16), b.view(torch.int16)
            elif a.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), "replay %d: %s differs from the eager call" % (rep, k)
        assert int(workspace[:4 * 4096].count_nonzero()) == 0, "split-K tile counters not reset"
        # each replay computed from its own inputs, not the previous ones
        if prev is not None:
            assert not torch.equal(snap["y"], prev["y"]) and not torch.equal(snap["vq"], prev["vq"])
        prev = snap
        log("  replay %d: every output bit-equal to the eager calls" % rep)
