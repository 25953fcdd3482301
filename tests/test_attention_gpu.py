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
                                      (1, 5, 3, "f16"), (5, 8192, 16, "bf16"), (7, 528, 24, "f32"),
                                      (3, 4096, 160, "f16"), (2, 16, 8, "f32"),
                                      (9, 2048, 64, "bf16")])
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


def test_attention_full_size_sampled(ref, dev):
    """Both products at the timed attention shape (32 heads, 2048 tokens,
    head_dim 128), fp16 out, in the launch configuration the benchmark uses:
    every code and step of Q, K, P and V compared in full on sampled heads;
    accumulators and outputs at sampled (head, query, key / channel) triples."""
    H, S, D = 32, 2048, 128
    r = np.random.default_rng([11, H, S, D])
    q = torch.from_numpy(r.standard_normal((H * S, D), dtype=np.float32)).half()
    k = torch.from_numpy(r.standard_normal((H * S, D), dtype=np.float32)).half()
    v = torch.from_numpy(r.standard_normal((H, S, D), dtype=np.float32)).half()
    # a row-normalised positive matrix standing in for the softmax output
    p32 = r.exponential(1.0, (H * S, S)).astype(np.float32)
    p = torch.from_numpy(p32 / p32.sum(axis=1, keepdims=True)).half()
    del p32
    qq, sq_ = sq.quant_act_pertoken(q.to(dev))
    kq, sk = sq.quant_act_pertoken(k.to(dev))
    pq, sp = sq.quant_act_pertoken(p.to(dev))
    vq, sv = sq.quant_weight_perchannel_batched(v.to(dev))
    scores = sq.w8a8_bmm_dequant(qq.view(H, S, D), sq_.view(H, S), kq.view(H, S, D),
                                 sk.view(H, S), torch.float16)
    out = sq.w8a8_bmm_dequant(pq.view(H, S, S), sp.view(H, S), vq, sv, torch.float16)
    torch.cuda.synchronize()
    rs = np.random.default_rng([12, H, S, D])
    for h in (0, 13, H - 1):
        rows = np.sort(rs.choice(S, 40, replace=False))
        cols = np.sort(rs.choice(S, 40, replace=False))
        dcols = np.sort(rs.choice(D, 24, replace=False))
        sl = slice(h * S, (h + 1) * S)
        xq_r, sx_r = ref.quant_act_pertoken(q[sl].float().numpy())
        kq_r, sk_r = ref.quant_act_pertoken(k[sl].float().numpy())
        pq_r, sp_r = ref.quant_act_pertoken(p[sl].float().numpy())
        vq_r, sv_r = ref.quant_weight_perchannel_batched(v[h:h + 1].float().numpy())
        assert_equal(qq[sl], xq_r, "Q codes, head %d" % h)
        assert_equal(sq_[sl], sx_r, "Q steps, head %d" % h)
        assert_equal(kq[sl], kq_r, "K codes, head %d" % h)
        assert_equal(sk[sl], sk_r, "K steps, head %d" % h)
        assert_equal(pq[sl], pq_r, "P codes, head %d" % h)
        assert_equal(sp[sl], sp_r, "P steps, head %d" % h)
        assert_equal(vq[h], vq_r[0], "V codes, head %d" % h)
        assert_equal(sv[h], sv_r[0], "V steps, head %d" % h)
        for name, y, a, sa, b, sb, c in (
                ("scores", scores, xq_r, sx_r, kq_r, sk_r, cols),
                ("output", out, pq_r, sp_r, vq_r[0], sv_r[0], dcols)):
            acc_r = ref.gemm_i32_sampled(a, b, rows, c)
            y32 = torch.from_numpy(ref.dequant_bias_act_f32(acc_r, sa[rows], sb[c])).half()
            ys = y[h].cpu()[torch.from_numpy(rows)][:, torch.from_numpy(c)]
            assert_equal(ys.view(torch.int16), y32.view(torch.int16).numpy(),
                         "%s bits, head %d" % (name, h))
            assert_y_close(ys, ref.dequant(acc_r, sa[rows], sb[c]), "%s, head %d" % (name, h))
        log("  head %d: ok" % h)
