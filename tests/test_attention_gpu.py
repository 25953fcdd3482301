"""GPU parity for the INT8 attention products: sq_w8a8_bmm_dequant /
sq_w8a8_bmm_i32 (batch x heads products in one launch) and
sq_quant_weight_perchannel_batched (V per head-dim channel, transposed).

Bar: codes, steps and accumulators bit-exact; outputs bit-equal to the
oracle's fp32 evaluation of the scale back (RN(RN(fp32(acc) * sx) * sw), then
one rounding to the output dtype) and within 1e-3 relative or one output ulp
of its double value.
"""
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


def _g(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _codes(B, M, N, K, seed):
    xq = np.stack([synth.random_int8(seed + 2 * b, M, K) for b in range(B)])
    wq = np.stack([synth.random_int8(seed + 2 * b + 1, N, K) for b in range(B)])
    xq[0, 0, :] = 127
    wq[-1, -1, :] = -127
    r = np.random.default_rng([B, M, N, K, seed])
    sx = (r.uniform(0.01, 2.0, (B, M)) / 127).astype(np.float32)
    sw = (r.uniform(1e-3, 0.05, (B, N)) / 127).astype(np.float32)
    return xq, wq, sx, sw


BMM_SHAPES = [
    (4, 256, 256, 128),    # Q K^T per head (head_dim 128): DMA tiles
    (4, 256, 128, 512),    # P V (N = head_dim): DMA tiles
    (3, 300, 513, 64),     # head_dim 64: register-staged tiles
    (2, 65, 37, 200),      # K not a multiple of 16: byte-masked tiles
    (3, 70, 130, 128),     # N not a multiple of 4: scales of later entries unaligned
    (8, 1, 2048, 128),     # decode: one query per head (few-token kernel)
    (6, 16, 300, 80),      # few-token kernel, K a multiple of 16
    (5, 3, 77, 33),        # few-token kernel, byte-masked K
    (1, 129, 255, 48),     # batch of one
]


@pytest.mark.parametrize("B,M,N,K", BMM_SHAPES)
@pytest.mark.parametrize("ydt", ["f16", "bf16", "f32"])
def test_bmm(ref, dev, B, M, N, K, ydt):
    log("bmm", B, M, N, K, ydt)
    xq, wq, sx, sw = _codes(B, M, N, K, B * 101 + M * 7 + N + K)
    acc = sq.w8a8_bmm_i32(_g(xq, dev), _g(wq, dev))
    y = sq.w8a8_bmm_dequant(_g(xq, dev), _g(sx, dev), _g(wq, dev), _g(sw, dev), DT[ydt])
    torch.cuda.synchronize()
    acc_r = ref.bmm_i32(xq, wq)
    assert_equal(acc, acc_r, "acc")
    y32 = torch.from_numpy(np.stack([ref.dequant_bias_act_f32(acc_r[b], sx[b], sw[b])
                                     for b in range(B)])).to(DT[ydt])
    bits = torch.int16 if ydt != "f32" else torch.int32
    assert_equal(y.cpu().view(bits), y32.view(bits).numpy(), "y (bits)")
    assert_y_close(y.reshape(B * M, N), ref.bmm_dequant(acc_r, sx, sw).reshape(B * M, N))


@pytest.mark.parametrize("B,K,N,dt", [(4, 256, 128, "f32"), (3, 1000, 64, "f16"),
                                      (2, 77, 33, "bf16"), (32, 2048, 128, "f16"),
                                      (1, 5, 3, "f16")])
def test_quant_weight_perchannel_batched(ref, dev, B, K, N, dt):
    log("quant_weight_perchannel_batched", B, K, N, dt)
    w = torch.stack([synth.random_matrix(B * 13 + b, K, N, dt, outlier_cols=[b % N], factor=9.0)
                     for b in range(B)])
    wq, sw = sq.quant_weight_perchannel_batched(w.to(dev))
    torch.cuda.synchronize()
    wq_r, sw_r = ref.quant_weight_perchannel_batched(w.float().numpy())
    assert_equal(wq, wq_r, "codes")
    assert_equal(sw, sw_r, "steps")


@pytest.mark.parametrize("B,S,D", [(4, 256, 128), (2, 300, 64)])
def test_int8_attention_chain(ref, dev, B, S, D):
    """Q K^T and P V of B heads in INT8: Q and K per token, P per row, V per
    head-dim channel; every code, step and accumulator bit-exact, outputs to
    the bar, and the whole within a few percent of float attention.  P (the
    softmax of the scores) is formed on the host from the oracle's scores and
    given to both sides."""
    r = np.random.default_rng([B, S, D])
    dims = r.choice(D, 4, replace=False)
    q = r.standard_normal((B, S, D)).astype(np.float32)
    k = r.standard_normal((B, S, D)).astype(np.float32)
    q[:, :, dims] *= 8.0  # a few head dimensions with persistent large values
    k[:, :, dims] *= 4.0
    v = r.standard_normal((B, S, D)).astype(np.float32)
    qh, kh, vh = (torch.from_numpy(a).half() for a in (q, k, v))

    # scores = Q K^T
    xq, sx = sq.quant_act_pertoken(qh.reshape(B * S, D).to(dev))
    kq, sk = sq.quant_act_pertoken(kh.reshape(B * S, D).to(dev))
    scores = sq.w8a8_bmm_dequant(xq.reshape(B, S, D), sx.reshape(B, S), kq.reshape(B, S, D),
                                 sk.reshape(B, S), torch.float32)
    torch.cuda.synchronize()
    xq_r, sx_r = ref.quant_act_pertoken(qh.float().numpy().reshape(B * S, D))
    kq_r, sk_r = ref.quant_act_pertoken(kh.float().numpy().reshape(B * S, D))
    assert_equal(xq, xq_r, "Q codes")
    assert_equal(kq, kq_r, "K codes")
    acc_r = ref.bmm_i32(xq_r.reshape(B, S, D), kq_r.reshape(B, S, D))
    s_r = ref.bmm_dequant(acc_r, sx_r.reshape(B, S), sk_r.reshape(B, S))
    assert_y_close(scores.reshape(B * S, S), s_r.reshape(B * S, S), "scores")

    # P = softmax(scores / sqrt(D)) (host, from the oracle's scores), then P V
    z = s_r / np.sqrt(D)
    p = np.exp(z - z.max(axis=-1, keepdims=True))
    p = (p / p.sum(axis=-1, keepdims=True)).astype(np.float16)
    pq, sp = sq.quant_act_pertoken(torch.from_numpy(p).reshape(B * S, S).to(dev))
    vq, sv = sq.quant_weight_perchannel_batched(vh.to(dev))
    out = sq.w8a8_bmm_dequant(pq.reshape(B, S, S), sp.reshape(B, S), vq, sv, torch.float16)
    torch.cuda.synchronize()
    pq_r, sp_r = ref.quant_act_pertoken(p.astype(np.float32).reshape(B * S, S))
    vq_r, sv_r = ref.quant_weight_perchannel_batched(vh.float().numpy())
    assert_equal(pq, pq_r, "P codes")
    assert_equal(vq, vq_r, "V codes")
    assert_equal(sv, sv_r, "V steps")
    acc2 = ref.bmm_i32(pq_r.reshape(B, S, S), vq_r)
    o_r = ref.bmm_dequant(acc2, sp_r.reshape(B, S), sv_r)
    assert_y_close(out.reshape(B * S, D), o_r.reshape(B * S, D), "attention output")

    # against float attention in double
    zf = np.einsum("bsd,btd->bst", qh.double().numpy(), kh.double().numpy()) / np.sqrt(D)
    pf = np.exp(zf - zf.max(axis=-1, keepdims=True))
    pf /= pf.sum(axis=-1, keepdims=True)
    of = np.einsum("bst,btd->bsd", pf, vh.double().numpy())
    rel = np.linalg.norm(to_np(out).astype(np.float64) - of) / np.linalg.norm(of)
    log("  relative error vs float attention:", rel)
    assert rel < 0.08
