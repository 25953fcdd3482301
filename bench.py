#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear-layer hot path on one MI355X.

Headline workload (one step): the three linear layers of an OPT-175B-like
block -- QKV [12288 x 36864], FC1 [12288 x 49152], FC2 [49152 x 12288],
bf16 -- each called on 8192 tokens: per-token INT8 activation quantisation
followed by the INT8 GEMM with fused scale back (the run-time part of the
method; the offline calibration / smoothing / weight quantisation runs once,
untimed for the headline).  Inputs are seeded synthetic activations with 0.1%
persistent outlier channels x100 and N(0, 0.02) weights, smoothed with
alpha = 0.5, all resident in HBM before timing starts.  The step is timed as
W warm-up steps, then 5 repeats of K steps between HIP events, the median
reported; two buffer sets (weights included) alternate.

Also reported: the OPT-6.7B-like layers (fp16) at 2048 and 512 tokens, the
OPT-13B-like layers at 4096 tokens and the OPT-175B-like ones at 2048, decode
shapes (1 and 16 tokens; the Llama-70B-like layers at 1-16 tokens) in GB/s
with weights streamed from HBM, the fused LayerNorm + quantiser, the INT8
attention products, the per-tensor levels, the offline transform, and the CPU
oracle on slices of the headline layers.

Prints one JSON line.  `--gpus N` with N > 1 exits: the benchmark measures
one GPU (one GPU's share of a layer at its real shape).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402
import w8a8_int8_post_amd as sq  # noqa: E402

METRIC = "W8A8 GEMM+quant TOPS & % INT8 MFMA peak (prefill); GB/s % HBM (decode M≤16)"
PEAK_I8_TOPS = 5000.0   # MI355X dense INT8 MFMA, AMD published (5.0 POP/s)
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, AMD published (8 TB/s)
CFG = synth.CONFIGS[2]  # OPT-6.7B-like layers
ALPHA = 0.5
PREFILL_M = 2048
DECODE_M = (1, 16)
HEAD_CFG = synth.CONFIGS[4]  # OPT-175B-like layers (bf16): the headline
HEAD_M = 8192
REPEATS = 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- set-up

class Layer:
    """Offline-prepared layer: Wq [N x K], sw [N], smoothing factors s [K]."""

    def __init__(self, name, dev):
        ly = CFG.layer(name)
        self.name, self.K, self.N = name, ly.K, ly.N
        w = synth.weight(CFG, name).to(dev)
        xc = synth.activations(CFG, name, CFG.T, calibration=True).to(dev)
        self.x_eval_host = synth.activations(CFG, name, PREFILL_M)
        a = sq.calibrate_absmax(xc)
        # the LayerNorm in front of the layer takes the smoothing (gamma / s, beta / s)
        g, b = synth.layernorm_params(CFG, name)
        self.ln_g = torch.as_tensor(g, dtype=torch.float32).contiguous().to(dev)
        self.ln_b = torch.as_tensor(b, dtype=torch.float32).contiguous().to(dev)
        self.s, w_hat = sq.smooth_fold(a, w, ALPHA, self.ln_g, self.ln_b)
        self.wq, self.sw = sq.quant_weight_perchannel(w_hat)
        self.wp = sq.pack_weight(self.wq)  # fragment-packed copy (offline re-layout)
        # O2/O3: per-tensor weights; O3's static activation step from calibration
        wq_t, self.sw_t = sq.quant_weight_pertensor(w_hat)
        self.wp_t = sq.pack_weight(wq_t)
        self.step = sq.static_act_step(a, self.s)
        del wq_t
        x = self.x_eval_host.to(dev)
        self.x_hat = sq.smooth_activation(x, self.s)   # what a folded LayerNorm emits
        self.x_res = x.clone()  # stand-in for the residual stream the LayerNorm reads
        torch.cuda.synchronize()
        self.w_host = None
        del w, xc, w_hat, x


def offline_time(dev):
    """Time calibration + smoothing/fold + weight quantisation of the three layers."""
    ws, xcs = [], []
    for ly in CFG.layers:
        ws.append(synth.weight(CFG, ly.name).to(dev))
        xcs.append(synth.activations(CFG, ly.name, CFG.T, calibration=True).to(dev))
    outs = []
    for (ly, w) in zip(CFG.layers, ws):
        outs.append((torch.empty(ly.K, device=dev), torch.empty(ly.K, device=dev),
                     torch.empty(ly.K, ly.N, device=dev),
                     torch.empty(ly.N, ly.K, dtype=torch.int8, device=dev),
                     torch.empty(ly.N, device=dev)))

    def run():
        for (ly, w, xc, (a, s, wh, wq, sw)) in zip(CFG.layers, ws, xcs, outs):
            sq.sq_calibrate_absmax(xc, a, False)
            sq.sq_smooth_fold(a, w, ALPHA, s, wh)
            sq.sq_quant_weight_perchannel(wh, wq, sw)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # bytes: X_cal read, W read twice (max + fold), W_hat written and read twice
    # (column max + quantise), Wq written
    nbytes = 0
    for ly in CFG.layers:
        nbytes += CFG.T * ly.K * 2 + 2 * ly.K * ly.N * 2 + ly.K * ly.N * 4 * 3 + ly.K * ly.N
    return {"ms": round(ms, 3), "layers": [ly.name for ly in CFG.layers],
            "steps": "calibrate_absmax(512 tokens) + smooth_fold + quant_weight_perchannel",
            "gbs": round(nbytes / ms / 1e6, 1), "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 3)}


class Bufs:
    """One rotating set of run-time buffers for every layer at M tokens, with
    the weights either row-major (canonical) or fragment-packed."""

    def __init__(self, layers, M, dev, packed, mode="o1"):
        self.items = []
        self.packed = packed
        self.mode = mode
        self.steps = []
        # split-K entry point ("ws"): one zero-filled workspace per set, the
        # size of its largest layer's need (the calls run one after another)
        self.ws = None
        # one-call layer ("o1", packed): the few-token entry point's workspace
        # (the fragment-packed copy of the codes; the calls run one after another)
        self.lws = None
        if mode == "o1" and packed:
            need = max(sq.sq_linear_workspace_bytes(ly.x_hat.dtype, M, ly.N, ly.K) for ly in layers)
            self.lws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        if mode == "ws":
            need = max(sq.sq_gemm_workspace_bytes(M, ly.N, ly.K) for ly in layers)
            self.ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
        for ly in layers:
            x_hat = ly.x_hat[:M].clone()
            if mode in ("o1", "ws"):
                w = (ly.wp if packed else ly.wq).clone()
                sw = ly.sw.clone()
            else:  # per-tensor weights
                assert packed
                w, sw = ly.wp_t.clone(), ly.sw_t.clone()
            self.steps.append(ly.step.clone())
            xq = torch.empty(M, ly.K, dtype=torch.int8, device=dev)
            sx = torch.empty(M, dtype=torch.float32, device=dev)
            y = torch.empty(M, ly.N, dtype=torch.float16, device=dev)
            self.items.append((x_hat, w, sw, xq, sx, y, ly.N))

    def _gemm(self, xq, sx, w, sw, y, N):
        if self.packed:
            sq.sq_w8a8_gemm_dequant_packed(xq, sx, w, sw, N, y)
        else:
            sq.sq_w8a8_gemm_dequant(xq, sx, w, sw, y)

    def step(self):
        for (x_hat, w, sw, xq, sx, y, N), st in zip(self.items, self.steps):
            if self.mode == "o3":  # one call per layer, static per-tensor step
                sq.sq_w8a8_linear_packed_static(x_hat, w, sw, st, xq, sx, y)
            elif self.mode == "o2":
                sq.sq_quant_act_pertensor(x_hat, xq, sx)
                self._gemm(xq, sx, w, sw, y, N)
            elif self.mode == "ws":
                sq.sq_quant_act_pertoken(x_hat, xq, sx)
                sq.sq_w8a8_gemm_dequant_packed_ws(xq, sx, w, sw, N, y, self.ws)
            elif self.packed:  # one call per layer; one kernel for one or two tokens
                sq.sq_w8a8_linear_packed_ws(x_hat, w, sw, xq, sx, y, self.lws)
            else:
                sq.sq_quant_act_pertoken(x_hat, xq, sx)
                self._gemm(xq, sx, w, sw, y, N)

    def gemm_only(self):
        for (x_hat, w, sw, xq, sx, y, N) in self.items:
            self._gemm(xq, sx, w, sw, y, N)

    def quant_only(self):
        for (x_hat, w, sw, xq, sx, y, N), st in zip(self.items, self.steps):
            if self.mode == "o3":
                sq.sq_quant_act_pertensor(x_hat, xq, sx, None, st)
            elif self.mode == "o2":
                sq.sq_quant_act_pertensor(x_hat, xq, sx)
            else:
                sq.sq_quant_act_pertoken(x_hat, xq, sx)


def capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graphs(graphs, iters, warmup):
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters  # ms per replay


def time_rotation(fns, iters, warmup, min_calls=4):
    """ms per call of fns[i]: one graph runs the functions back to back in
    order (a rotation over buffer sets, repeated to at least `min_calls`
    calls), as a serving loop would, and is replayed until `iters` calls
    have run between the events."""
    seq = list(fns) * max(1, -(-min_calls // len(fns)))
    g = capture(lambda: [f() for f in seq])
    reps = max(1, -(-iters // len(seq)))
    wreps = max(1, -(-warmup // len(seq)))
    return time_graphs([g], reps, wreps) / len(seq)


def time_rotation_median(fns, iters, warmup, reps=3, min_calls=4):
    """As time_rotation, the median of `reps` timed runs of one captured
    graph (for the short decode steps, where one run can catch a hiccup)."""
    seq = list(fns) * max(1, -(-min_calls // len(fns)))
    g = capture(lambda: [f() for f in seq])
    n = max(1, -(-iters // len(seq)))
    w = max(1, -(-warmup // len(seq)))
    return float(np.median([time_graphs([g], n, w) / len(seq) for _ in range(reps)]))


def time_steps(fns, steps, warmup, repeats=REPEATS):
    """Median ms per call of fns (one graph each, replayed in rotation):
    `warmup` untimed calls, then `repeats` timed runs of exactly `steps`
    calls between HIP events on the current stream.  Returns (median, runs)."""
    graphs = [capture(f) for f in fns]
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    runs = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / steps)
    return float(np.median(runs)), runs


def headline_record(hd, steps, warmup):
    """The JSON line's common part from the headline measurement (hd as
    headline() returns it: step ms, ops per step and per GEMM launch, average
    GEMM and quantiser launch us)."""
    tops = hd["ops"] / (hd["ms"] * 1e-3) / 1e12
    gemm_tops = hd["per_launch_ops"] / (hd["gemm_avg_us"] * 1e-6) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(hd["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "OPT-175B-like linear layers QKV 12288x36864, FC1 12288x49152, FC2 "
                        "49152x12288; bf16 activations/weights/output; 8192 tokens per layer "
                        "call; 0.1% persistent outlier channels x100; alpha 0.5",
            "tokens": hd["M"],
            "step": "per layer: sq_quant_act_pertoken + sq_w8a8_gemm_dequant_packed (3 layers)",
            "weights": "fragment-packed",
            "timing": "median of %d runs of %d steps (HIP events; two buffer sets alternate); "
                      "runs ms/step %s" % (REPEATS, steps,
                                          ", ".join("%.4f" % r for r in hd["runs"])),
            "frac_of_int8_peak": round(tops / PEAK_I8_TOPS, 4),
            "layers": hd["layers"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "gemm_dma_kernel (i8 MFMA GEMM + fused scale back), 256x256 tiles",
            "bound": "mfma",
            "achieved": round(gemm_tops, 2),
            "peak": PEAK_I8_TOPS,
            "unit": "TOP/s",
            "frac": round(gemm_tops / PEAK_I8_TOPS, 4),
            "traffic": profiled_traffic("gemm_prefill_opt175b.md"),
            "traffic_unit": "HBM-side bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE, "
                            "profiles/gemm_prefill_opt175b.md)",
            "avg_launch_us": round(hd["gemm_avg_us"], 2),
            "per_launch_ops": hd["per_launch_ops"],
        },
        "act_quant": {"avg_launch_us": round(hd["quant_avg_us"], 2),
                      "gbs": round(hd["quant_bytes"] / hd["quant_avg_us"] / 1e3, 1),
                      "hbm_frac": round(hd["quant_bytes"] / hd["quant_avg_us"] / 1e3
                                        / PEAK_HBM_GBS, 3)},
    }
    return out


def check_peak_fractions(obj, path="out"):
    """Every fraction of the INT8 MFMA peak in the JSON line must lie in
    (0, 1]: a value above 1 is a unit error, never a measurement."""
    if isinstance(obj, dict):
        for k, v in obj.items():
            here = "%s.%s" % (path, k)
            if isinstance(v, (int, float)) and (k.endswith("frac_of_int8_peak")
                                                or (k == "frac" and obj.get("bound") == "mfma")):
                if not 0.0 < v <= 1.0:
                    raise RuntimeError("%s = %r is not a fraction of the peak" % (here, v))
            else:
                check_peak_fractions(v, here)
    return obj


def profiled_traffic(summary):
    """HBM bytes per GEMM launch from a committed rocprofv3 summary under
    profiles/, if it was taken on the current GEMM source (else None)."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", summary)
    csrc = os.path.join(ROOT, "w8a8_int8_post_amd", "csrc")
    try:
        fields = dict(ln.split(": ", 1) for ln in open(prof).read().splitlines()
                      if ln.startswith(("traffic_bytes_per_launch:", "gemm_source_sha256:")))
        h = hashlib.sha256()
        for f in ("sq_gemm.hip", "sq_gemm_common.h", "sq_device.h"):
            h.update(open(os.path.join(csrc, f), "rb").read())
        digest = h.hexdigest()
        if fields.get("gemm_source_sha256", "").strip() != digest:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def attention_time(dev, args, H=32, S=2048, D=128):
    """Time the two INT8 attention products and their quantisers."""
    r = np.random.default_rng([7, H, S, D])
    q = torch.from_numpy(r.standard_normal((H * S, D), dtype=np.float32)).half().to(dev)
    k = torch.from_numpy(r.standard_normal((H * S, D), dtype=np.float32)).half().to(dev)
    v = torch.from_numpy(r.standard_normal((H, S, D), dtype=np.float32)).half().to(dev)
    z = torch.softmax(torch.from_numpy(r.standard_normal((H * S, S), dtype=np.float32)), -1)
    p = z.half().to(dev)
    del z
    qq, sq_ = sq.quant_act_pertoken(q)
    kq, sk = sq.quant_act_pertoken(k)
    pq, sp = sq.quant_act_pertoken(p)
    vq, sv = sq.quant_weight_perchannel_batched(v)
    scores = torch.empty(H, S, S, dtype=torch.float16, device=dev)
    o = torch.empty(H, S, D, dtype=torch.float16, device=dev)

    def qk():
        sq.sq_w8a8_bmm_dequant(qq.view(H, S, D), sq_.view(H, S), kq.view(H, S, D), sk.view(H, S),
                               scores)

    def pv():
        sq.sq_w8a8_bmm_dequant(pq.view(H, S, S), sp.view(H, S), vq, sv, o)

    def quants():
        sq.sq_quant_act_pertoken(q, qq, sq_)
        sq.sq_quant_act_pertoken(k, kq, sk)
        sq.sq_quant_act_pertoken(p, pq, sp)
        sq.sq_quant_weight_perchannel_batched(v, vq, sv)

    ops = 2.0 * H * S * S * D
    res = {"heads": H, "tokens": S, "head_dim": D, "dtype_out": "fp16"}
    for name, fn, nbytes in (
            ("qk", qk, 2 * H * S * D + 2 * H * S * S + 8 * H * S),
            ("pv", pv, H * S * S + H * S * D + 2 * H * S * D + 4 * H * S + 4 * H * D)):
        ms = time_rotation([fn], args.steps, args.warmup)
        res[name] = {"us": round(ms * 1e3, 2), "tops": round(ops / (ms * 1e-3) / 1e12, 1),
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                     "bytes": nbytes}
        log("attention %s: %.1f us, %.1f TOPS, %.0f GB/s" % (name, ms * 1e3, res[name]["tops"],
                                                             res[name]["gbs"]))
    ms = time_rotation([quants], args.steps, args.warmup)
    qbytes = 3 * H * S * D * 2 + H * S * S * 3 + H * S * D * 2 + 12 * H * S
    res["quant_all_us"] = round(ms * 1e3, 2)
    res["quant_gbs"] = round(qbytes / (ms * 1e-3) / 1e9, 1)
    res["step"] = ("sq_w8a8_bmm_dequant for Q K^T (scores fp16) and for P V; quantisers: "
                   "sq_quant_act_pertoken for Q, K, P and sq_quant_weight_perchannel_batched for V")
    log("attention quantisers: %.1f us" % (ms * 1e3))
    del q, k, v, p, qq, kq, pq, vq, scores, o
    torch.cuda.synchronize()
    return res


def decode_llama70b(dev, args):
    """The decode configuration of the workload set: Llama-70B-like up
    [8192 x 28672] and down [28672 x 8192] layers, fp16, N(0, 0.015) weights
    quantised per output channel, 8 persistent outlier channels x50, 1 to 16
    tokens; one call per layer (sq_w8a8_linear_packed_ws: at 13-16 tokens the
    GEMM reads the quantiser's fragment-packed copy of the codes), weights
    rotated over buffer sets so that every call streams them from HBM."""
    cfg = synth.CONFIGS[5]
    lys = []
    for ly in cfg.layers:
        w = synth.weight(cfg, ly.name).to(dev)
        xc = synth.activations(cfg, ly.name, cfg.T, calibration=True).to(dev)
        a = sq.calibrate_absmax(xc)
        s_, w_hat = sq.smooth_fold(a, w, ALPHA)
        wq, sw = sq.quant_weight_perchannel(w_hat)
        wp = sq.pack_weight(wq)
        x = sq.smooth_activation(synth.activations(cfg, ly.name, max(cfg.M)).to(dev), s_)
        lys.append((ly, wp, sw, x))
        del w, xc, a, w_hat, wq
        torch.cuda.synchronize()
    res = {"layers": [[ly.name, ly.K, ly.N] for ly, _, _, _ in lys]}
    for Md in cfg.M:
        foot = sum(ly.N * ly.K + Md * ly.K * 3 + Md * ly.N * 2 for ly, _, _, _ in lys)
        R = n_sets(foot)
        sets = []
        for _ in range(R):
            sets.append([(x[:Md].clone(), wp.clone(), sw.clone(),
                          torch.empty(Md, ly.K, dtype=torch.int8, device=dev),
                          torch.empty(Md, dtype=torch.float32, device=dev),
                          torch.empty(Md, ly.N, dtype=torch.float16, device=dev),
                          sq.linear_workspace(x.dtype, Md, ly.N, ly.K, dev))
                         for ly, wp, sw, x in lys])
        ent = {"buffer_sets": R}

        def run(bset, which):
            for i in which:
                xh, wp, sw, xq, sx, y, lws = bset[i]
                sq.sq_w8a8_linear_packed_ws(xh, wp, sw, xq, sx, y, lws)
        for key, which in (("step", (0, 1)), ("up", (0,)), ("down", (1,))):
            nbytes = sum(lys[i][0].N * lys[i][0].K + 4 * lys[i][0].N + 2 * Md * lys[i][0].K
                         + 2 * Md * lys[i][0].N + 4 * Md for i in which)
            ms = time_rotation_median([lambda b=b, w_=which: run(b, w_) for b in sets],
                                      max(args.steps, 4 * R), args.warmup)
            gbs = nbytes / (ms * 1e-3) / 1e9
            ent[key] = {"us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        log("llama-70b decode M=%d: step %.1f us (%.1f%% HBM); up %.1f us (%.1f%%), down %.1f us "
            "(%.1f%%)" % (Md, ent["step"]["us"], 100 * ent["step"]["hbm_frac"], ent["up"]["us"],
                          100 * ent["up"]["hbm_frac"], ent["down"]["us"],
                          100 * ent["down"]["hbm_frac"]))
        res["M=%d" % Md] = ent
        del sets
        torch.cuda.synchronize()
    res["step"] = ("per layer sq_w8a8_linear_packed_ws (per-token quantisation + packed INT8 GEMM "
                   "+ scale back), up then down; bytes: weights + w_scale + fp16 x + fp16 y")
    del lys
    torch.cuda.synchronize()
    return res


def prefill_512(layers, dev, args, M5=512):
    """The OPT-6.7B-like layers at 512 tokens: the plain packed path and the
    split-K entry point (which splits K only where that beats the plain
    kernels; "split_layers" names those layers).  Besides TOPS, the step is
    given as a fraction of its roofline floor, sum over layers of
    max(ops / INT8 peak, algorithmic bytes / HBM bandwidth): at 512 tokens
    these layers sit just right of the ridge point (about 770 ops/byte)."""
    ops5 = sum(2.0 * M5 * ly.N * ly.K for ly in layers)
    floor_ms = 0.0
    for ly in layers:
        nbytes = ly.N * ly.K + 4 * ly.N + 2 * M5 * ly.K + 2 * M5 * ly.N + 4 * M5
        floor_ms += max(2.0 * M5 * ly.N * ly.K / (PEAK_I8_TOPS * 1e9),
                        nbytes / (PEAK_HBM_GBS * 1e6))
    p512 = {"tokens": M5,
            "split_layers": [ly.name for ly in layers
                             if sq.sq_gemm_workspace_bytes(M5, ly.N, ly.K) > 0],
            "roofline_floor_ms": round(floor_ms, 4)}
    # the two entry points alternate (three rounds each, medians): timed one
    # after the other, the first read up to 4% slower on the same kernels
    modes = ("o1", "ws")
    sets = {mode: [Bufs(layers, M5, dev, True, mode) for _ in range(2)] for mode in modes}
    times = {mode: [] for mode in modes}
    for _ in range(3):
        for mode in modes:
            times[mode].append(time_rotation([b.step for b in sets[mode]], args.steps, args.warmup))
    for mode in modes:
        ms5 = float(np.median(times[mode]))
        p512["split_k" if mode == "ws" else "plain"] = {
            "ms_per_step": round(ms5, 4), "tops": round(ops5 / ms5 / 1e9, 1),
            "frac_of_int8_peak": round(ops5 / ms5 / 1e9 / PEAK_I8_TOPS, 4),
            "frac_of_roofline": round(floor_ms / ms5, 4)}
        log("prefill at %d tokens (%s): step %.3f ms, %.1f TOPS, %.1f%% of the roofline floor"
            % (M5, "split-K entry point" if mode == "ws" else "plain", ms5, ops5 / ms5 / 1e9,
               100 * floor_ms / ms5))
    del sets
    torch.cuda.synchronize()
    p512["step"] = ("per layer: sq_quant_act_pertoken + packed GEMM; plain: sq_w8a8_linear_packed_ws "
                    "(as sq_w8a8_linear_packed at this size), "
                    "split_k: sq_w8a8_gemm_dequant_packed_ws")
    return p512


def prepare_layers(cfg, M, dev, keep_host_rows=0):
    """Each layer of cfg through the library's offline path (calibration on
    the config's calibration tokens, smoothing factors and fold, per-channel
    weight quantisation, packing) plus its smoothed evaluation activations
    (M tokens), as a folded LayerNorm would emit them.  With keep_host_rows,
    host copies of the row-major codes, steps and the first rows of X_hat are
    kept for the CPU oracle."""
    prep, host = [], []
    for ly in cfg.layers:
        w = synth.weight(cfg, ly.name).to(dev)
        xc = synth.activations(cfg, ly.name, cfg.T, calibration=True).to(dev)
        s_, w_hat = sq.smooth_fold(sq.calibrate_absmax(xc), w, ALPHA)
        del w, xc
        wq, sw = sq.quant_weight_perchannel(w_hat)
        del w_hat
        wp = sq.pack_weight(wq)
        x = synth.activations(cfg, ly.name, M).to(dev)
        x_hat = sq.smooth_activation(x, s_)
        del x
        torch.cuda.synchronize()
        if keep_host_rows:
            host.append((x_hat[:keep_host_rows].float().cpu().numpy(), wq.cpu().numpy(),
                         sw.cpu().numpy(), ly.N, ly.K))
        del wq
        prep.append((ly, wp, sw, x_hat))
        torch.cuda.synchronize()
    return prep, host


def layer_sets(prep, M, ydt, dev, R=2):
    """R independent run-time buffer sets (weights included) for M tokens."""
    sets = []
    for _ in range(R):
        sets.append([(x_hat[:M].clone(), wp.clone(), sw.clone(),
                      torch.empty(M, ly.K, dtype=torch.int8, device=dev),
                      torch.empty(M, dtype=torch.float32, device=dev),
                      torch.empty(M, ly.N, dtype=ydt, device=dev), ly.N)
                     for (ly, wp, sw, x_hat) in prep])
    return sets


def headline(dev, args):
    """The OPT-175B-like block at 8192 tokens: step = per layer the per-token
    quantiser and the packed GEMM with the scale back (bf16 out); each GEMM
    and each quantiser also alone.  Returns (result dict, host data for the
    CPU baseline)."""
    cfg, M = HEAD_CFG, HEAD_M
    ydt = synth.DTYPES[cfg.ydt]
    log("setting up the headline layers", [(ly.name, ly.K, ly.N) for ly in cfg.layers])
    prep, host = prepare_layers(cfg, M, dev, keep_host_rows=CPU_SLICE_ROWS)
    sets = layer_sets(prep, M, ydt, dev)
    del prep
    torch.cuda.synchronize()

    def step(bs):
        for (x_hat, wp, sw, xq, sx, y, N) in bs:
            sq.sq_quant_act_pertoken(x_hat, xq, sx)
            sq.sq_w8a8_gemm_dequant_packed(xq, sx, wp, sw, N, y)

    ops = sum(2.0 * M * ly.N * ly.K for ly in cfg.layers)
    ms, runs = time_steps([lambda bs=bs: step(bs) for bs in sets], args.steps, args.warmup)
    log("headline %s at %d tokens: step %.3f ms (runs %s), %.1f TOPS"
        % (cfg.name, M, ms, ", ".join("%.3f" % r for r in runs), ops / ms / 1e9))
    layers = {}
    gemm_us, quant_us = [], []
    for i, ly in enumerate(cfg.layers):
        def gemm(bs, i=i):
            x_hat, wp, sw, xq, sx, y, N = bs[i]
            sq.sq_w8a8_gemm_dequant_packed(xq, sx, wp, sw, N, y)

        def quant(bs, i=i):
            x_hat, wp, sw, xq, sx, y, N = bs[i]
            sq.sq_quant_act_pertoken(x_hat, xq, sx)
        ms_g, _ = time_steps([lambda bs=bs: gemm(bs) for bs in sets], args.steps, args.warmup)
        ms_q, _ = time_steps([lambda bs=bs: quant(bs) for bs in sets], args.steps, args.warmup)
        lops = 2.0 * M * ly.N * ly.K
        qbytes = M * ly.K * 2 + M * ly.K + 4 * M
        layers[ly.name] = {"gemm_us": round(ms_g * 1e3, 1),
                           "gemm_tops": round(lops / ms_g / 1e9, 1),
                           "frac_of_int8_peak": round(lops / ms_g / 1e9 / PEAK_I8_TOPS, 4),
                           "act_quant_us": round(ms_q * 1e3, 2),
                           "act_quant_gbs": round(qbytes / ms_q / 1e6, 1)}
        gemm_us.append(ms_g * 1e3)
        quant_us.append(ms_q * 1e3)
        log("  %s: gemm %.1f us (%.1f TOP/s), quantiser %.1f us"
            % (ly.name, ms_g * 1e3, lops / ms_g / 1e9, ms_q * 1e3))
    del sets
    torch.cuda.synchronize()
    return {"cfg": cfg, "M": M, "ms": ms, "runs": runs, "ops": ops, "layers": layers,
            "gemm_avg_us": float(np.mean(gemm_us)), "quant_avg_us": float(np.mean(quant_us)),
            "per_launch_ops": ops / len(cfg.layers),
            "quant_bytes": sum(M * ly.K * 2 + M * ly.K + 4 * M for ly in cfg.layers)
            / len(cfg.layers)}, host


LARGER = ((3, (4096,)), (4, (2048,)))  # OPT-13B-like, OPT-175B-like (config, tokens)


def larger_prefill(dev, args):
    """Prefill steps of the larger layer sets: OPT-13B-like (fp16, 4096 tokens)
    and OPT-175B-like (bf16, 2048 and 8192 tokens).  Each layer goes through
    the offline path (calibration on 512 tokens, smoothing and fold, per-channel
    weight quantisation, packing); a step is, per layer, the per-token
    quantiser and the packed GEMM with the scale back, output in the layer's
    dtype.  Two buffer sets, weights included, alternate (each step moves far
    more than the 256 MB last-level cache)."""
    res = {}
    for cid, Ms in LARGER:
        cfg = synth.CONFIGS[cid]
        ydt = synth.DTYPES[cfg.ydt]
        prep = []
        for ly in cfg.layers:
            w = synth.weight(cfg, ly.name).to(dev)
            xc = synth.activations(cfg, ly.name, cfg.T, calibration=True).to(dev)
            s, w_hat = sq.smooth_fold(sq.calibrate_absmax(xc), w, ALPHA)
            del w, xc
            wq, sw = sq.quant_weight_perchannel(w_hat)
            del w_hat
            wp = sq.pack_weight(wq)
            del wq
            x = synth.activations(cfg, ly.name, max(Ms)).to(dev)
            prep.append((ly, wp, sw, sq.smooth_activation(x, s)))
            del x
            torch.cuda.synchronize()
        ent = {"layers": [[ly.name, ly.K, ly.N] for ly in cfg.layers], "dtype": cfg.act}
        for M in Ms:
            ops = sum(2.0 * M * ly.N * ly.K for ly in cfg.layers)
            sets = []
            for _ in range(2):
                sets.append([(x_hat[:M].clone(), wp.clone(), sw.clone(),
                              torch.empty(M, ly.K, dtype=torch.int8, device=dev),
                              torch.empty(M, dtype=torch.float32, device=dev),
                              torch.empty(M, ly.N, dtype=ydt, device=dev), ly.N)
                             for (ly, wp, sw, x_hat) in prep])

            def step(bs):
                for (x_hat, wp, sw, xq, sx, y, N) in bs:
                    sq.sq_quant_act_pertoken(x_hat, xq, sx)
                    sq.sq_w8a8_gemm_dequant_packed(xq, sx, wp, sw, N, y)

            def gemm(bs, i):
                x_hat, wp, sw, xq, sx, y, N = bs[i]
                sq.sq_w8a8_gemm_dequant_packed(xq, sx, wp, sw, N, y)

            iters = max(4, args.steps // 4)
            ms = time_rotation([lambda bs=bs: step(bs) for bs in sets], iters, 2)
            per_layer = {}
            for i, (ly, _, _, _) in enumerate(prep):
                ms_g = time_rotation([lambda bs=bs, i=i: gemm(bs, i) for bs in sets], iters, 2)
                tops_g = 2.0 * M * ly.N * ly.K / ms_g / 1e9
                per_layer[ly.name] = {"gemm_us": round(ms_g * 1e3, 1), "gemm_tops": round(tops_g, 1),
                                      "frac_of_int8_peak": round(tops_g / PEAK_I8_TOPS, 4)}
            tops = ops / ms / 1e9
            ent["M=%d" % M] = {"ms_per_step": round(ms, 4), "tops": round(tops, 1),
                               "frac_of_int8_peak": round(tops / PEAK_I8_TOPS, 4),
                               "layers": per_layer}
            log("%s prefill at %d tokens: step %.3f ms, %.1f TOPS (%.1f%% of peak); gemm %s"
                % (cfg.name, M, ms, tops, 100 * tops / PEAK_I8_TOPS,
                   ", ".join("%s %.1f us" % (k, v["gemm_us"]) for k, v in per_layer.items())))
            del sets
            torch.cuda.synchronize()
        res[cfg.name] = ent
        del prep
        torch.cuda.synchronize()
    res["step"] = ("per layer: sq_quant_act_pertoken + sq_w8a8_gemm_dequant_packed, output in the "
                   "layer dtype; gemm: the packed GEMM alone")
    return res


def n_sets(footprint_bytes):
    return max(2, math.ceil((1 << 30) / footprint_bytes))


# ---------------------------------------------------------------- cpu baseline

CPU_SLICE_ROWS = 256     # all host cores: 256-token slice of every headline layer
CPU_SLICE_ROWS_1T = 16   # one thread: 16-token slice


def cpu_baseline(host, M, cfg):
    """The CPU oracle (per-token quant + INT8 GEMM + scale back, OpenMP over
    token rows) on slices of the headline layers: the first CPU_SLICE_ROWS
    tokens of each layer on all host cores and the first CPU_SLICE_ROWS_1T on
    one thread, each the median of 3 runs.  GEMM work is linear in the token
    count, so the rate is the full step's, extrapolated."""
    import oracle

    def run(rows):
        t0 = time.perf_counter()
        for (xh, wq, sw, N, K) in host:
            oracle.linear_w8a8(xh[:rows], wq, sw)
        return time.perf_counter() - t0

    def ops(rows):
        return sum(2.0 * rows * N * K for (_, _, _, N, K) in host)

    cores = oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    run(2)  # start the thread pool
    t_all = float(np.median([run(CPU_SLICE_ROWS) for _ in range(3)]))
    oracle.set_threads(1)
    t_one = float(np.median([run(CPU_SLICE_ROWS_1T) for _ in range(3)]))
    oracle.set_threads(cores)
    tops_all = ops(CPU_SLICE_ROWS) / t_all / 1e12
    tops_one = ops(CPU_SLICE_ROWS_1T) / t_one / 1e12
    return {"value": round(tops_all, 6), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": "first %d of %d tokens of each of the 3 %s layers (quant + INT8 GEMM + scale "
                      "back), median of 3 runs of %.1f s; extrapolated linearly in tokens"
                      % (CPU_SLICE_ROWS, M, cfg.name, t_all),
            "extrapolated_step_s": round(t_all * M / CPU_SLICE_ROWS, 1),
            "one_thread": {"value": round(tops_one, 6), "unit": "TOPS", "cores": 1,
                           "sample": "first %d tokens of each layer, median of 3 runs of %.1f s"
                                     % (CPU_SLICE_ROWS_1T, t_one),
                           "extrapolated_step_s": round(t_one * M / CPU_SLICE_ROWS_1T, 1)}}


def decode_phase(layers, dev, args):
    """The OPT-6.7B-like layers at DECODE_M tokens (packed and row-major
    weights, rotated past the Infinity Cache), per step and per GEMM launch."""
    dec = {}
    for Md in DECODE_M:
        foot = sum(ly.N * ly.K + Md * ly.K * 3 + Md * ly.N * 2 for ly in layers)
        R = n_sets(foot)
        nbytes = sum(ly.N * ly.K + 4 * ly.N + 2 * Md * ly.K + 2 * Md * ly.N + 4 * Md
                     for ly in layers)
        entry = {"buffer_sets": R}
        for packed in (True, False):
            sets = [Bufs(layers, Md, dev, packed) for _ in range(R)]
            ms_d = time_rotation_median([b.step for b in sets], max(args.steps, 4 * R),
                                        args.warmup)
            ms_g = time_rotation_median([b.gemm_only for b in sets], max(args.steps, 4 * R),
                                        args.warmup) / len(layers)
            gbs = nbytes / (ms_d * 1e-3) / 1e9
            gbs_g = nbytes / len(layers) / (ms_g * 1e-3) / 1e9
            key = "packed" if packed else "row_major"
            entry[key] = {"us_per_step": round(ms_d * 1e3, 2), "gbs": round(gbs, 1),
                          "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                          "gemm_avg_launch_us": round(ms_g * 1e3, 2),
                          "gemm_gbs": round(gbs_g, 1),
                          "gemm_hbm_frac": round(gbs_g / PEAK_HBM_GBS, 4)}
            log("decode M=%d (%s): %.2f us/step, %.0f GB/s (%.1f%% HBM); gemm %.2f us, %.0f GB/s"
                % (Md, key, ms_d * 1e3, gbs, 100 * gbs / PEAK_HBM_GBS, ms_g * 1e3, gbs_g))
            del sets
            torch.cuda.synchronize()
        dec["M=%d" % Md] = entry
    return dec


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-offline", action="store_true")
    ap.add_argument("--no-levels", action="store_true", help="skip the O2/O3 measurements")
    ap.add_argument("--no-attention", action="store_true", help="skip the INT8 attention products")
    ap.add_argument("--no-prefill-512", action="store_true",
                    help="skip the 512-token prefill (plain and split-K)")
    ap.add_argument("--no-larger", action="store_true",
                    help="skip the OPT-13B-like (4096 tokens) and OPT-175B-like (2048 tokens) layers")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline step (OPT-175B-like, 8192 tokens; for profiling)")
    ap.add_argument("--opt67b-only", action="store_true",
                    help="only the OPT-6.7B-like layers at 2048 tokens (for profiling)")
    ap.add_argument("--prefill-512-only", action="store_true",
                    help="only the 512-token prefill (prints {\"prefill_512\": ...}; for profiling)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode phases (OPT-6.7B-like and Llama-70B-like; for profiling)")
    ap.add_argument("--larger-only", action="store_true",
                    help="only the OPT-13B-like (4096 tokens) and OPT-175B-like (2048 tokens) layers "
                         "(for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (to scale HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the SmoothQuant W8A8 path is benchmarked on a single "
              "MI355X (one GPU's shard at its real shape); it has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    sq.load_library()

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 5}))
        return

    if args.decode_only or args.larger_only:
        part = {}
        if args.larger_only:
            part["larger_prefill"] = larger_prefill(dev, args)
        if args.decode_only:
            layers = [Layer(ly.name, dev) for ly in CFG.layers]
            part["decode"] = decode_phase(layers, dev, args)
            part["decode_llama70b"] = decode_llama70b(dev, args)
        print(json.dumps(check_peak_fractions(part)), flush=True)
        return

    out = {}
    host = None
    if not (args.opt67b_only or args.prefill_512_only):
        # ---- the headline: OPT-175B-like block, 8192 tokens, bf16
        hd, host = headline(dev, args)
        out = headline_record(hd, args.steps, args.warmup)
        if args.headline_only:
            print(json.dumps(check_peak_fractions(out)), flush=True)
            return

    log("setting up the OPT-6.7B-like layers", [(ly.name, ly.K, ly.N) for ly in CFG.layers])
    layers = [Layer(ly.name, dev) for ly in CFG.layers]
    if args.prefill_512_only:
        print(json.dumps({"prefill_512": prefill_512(layers, dev, args)}), flush=True)
        return

    # ---- the OPT-6.7B-like layers at 2048 tokens, row-major and packed weights
    M = PREFILL_M
    ops_step = sum(2.0 * M * ly.N * ly.K for ly in layers)
    quant_bytes = sum(M * ly.K * 2 + M * ly.K + 4 * M for ly in layers) / len(layers)
    res = {}
    for packed in (False, True):
        sets = [Bufs(layers, M, dev, packed) for _ in range(2)]
        ms, runs = time_steps([b.step for b in sets], args.steps, args.warmup)
        gemm_ms = time_rotation([b.gemm_only for b in sets], args.steps, args.warmup) / len(layers)
        quant_ms = time_rotation([b.quant_only for b in sets], args.steps,
                                 args.warmup) / len(layers)
        res[packed] = (ms, gemm_ms, quant_ms)
        log("opt-6.7b prefill (%s weights): step %.3f ms  %.1f TOPS; gemm avg %.1f us (%.1f TOPS); "
            "quant avg %.1f us (%.0f GB/s)" % ("packed" if packed else "row-major", ms,
                                               ops_step / ms / 1e9, gemm_ms * 1e3,
                                               ops_step / len(layers) / gemm_ms / 1e9,
                                               quant_ms * 1e3, quant_bytes / quant_ms / 1e6))
        del sets
        torch.cuda.synchronize()
    ms, gemm_ms, quant_ms = res[True]
    tops67 = ops_step / (ms * 1e-3) / 1e12
    gemm67 = ops_step / len(layers) / (gemm_ms * 1e-3) / 1e12
    out["opt6.7b_2048"] = {
        "workload": "OPT-6.7B-like linear layers QKV 4096x12288, FC1 4096x16384, FC2 16384x4096; "
                    "fp16; 2048 tokens; 0.5% persistent outlier channels x60; alpha 0.5",
        "step": "per layer: sq_w8a8_linear_packed_ws (quantiser + packed GEMM; as "
                "sq_w8a8_linear_packed at this size)",
        "ms_per_step": round(ms, 4), "tops": round(tops67, 2),
        "frac_of_int8_peak": round(tops67 / PEAK_I8_TOPS, 4),
        "row_major_ms_per_step": round(res[False][0], 4),
        "gemm_avg_launch_us": round(gemm_ms * 1e3, 2), "gemm_tops": round(gemm67, 1),
        "gemm_frac_of_int8_peak": round(gemm67 / PEAK_I8_TOPS, 4),
        "gemm_traffic": profiled_traffic("gemm_prefill_opt6.7b.md"),
        "act_quant_avg_launch_us": round(quant_ms * 1e3, 2),
        "act_quant_gbs": round(quant_bytes / quant_ms / 1e6, 1),
        "act_quant_hbm_frac": round(quant_bytes / quant_ms / 1e6 / PEAK_HBM_GBS, 3),
    }
    if args.opt67b_only:
        print(json.dumps(check_peak_fractions(out)), flush=True)
        return

    # ---- the same layers at 512 tokens (the configuration's smaller prefill)
    if not args.no_prefill_512:
        out["prefill_512"] = prefill_512(layers, dev, args)

    # ---- the LayerNorm in front of QKV and FC1 (it carries the folded
    # smoothing) fused with the per-token quantisation: reads the residual
    # stream once and writes only codes and steps
    ln_layers = [ly for ly in layers if ly.name in ("qkv", "fc1")]
    ln_bytes = sum(M * ly.K * 2 + M * ly.K + 4 * M + 8 * ly.K for ly in ln_layers) / len(ln_layers)
    ln_ms = {}
    for hat in (False, True):
        bufs = []
        for _ in range(2):
            bufs.append([(ly.x_res.clone(), ly.ln_g, ly.ln_b,
                          torch.empty(M, ly.K, dtype=torch.int8, device=dev),
                          torch.empty(M, dtype=torch.float32, device=dev),
                          torch.empty(M, ly.K, dtype=torch.float16, device=dev) if hat else None)
                         for ly in ln_layers])

        def ln_fn(bset):
            for (x, g, b, xq, sx, xh) in bset:
                sq.sq_layernorm_quant_pertoken(x, g, b, 1e-5, xq, sx, xh)
        ln_ms[hat] = time_rotation([lambda bs=bs: ln_fn(bs) for bs in bufs], args.steps,
                                   args.warmup) / len(ln_layers)
        del bufs
        torch.cuda.synchronize()
    out["layernorm_quant"] = {
        "avg_launch_us": round(ln_ms[False] * 1e3, 2),
        "gbs": round(ln_bytes / ln_ms[False] / 1e6, 1),
        "hbm_frac": round(ln_bytes / ln_ms[False] / 1e6 / PEAK_HBM_GBS, 3),
        "with_x_hat_avg_launch_us": round(ln_ms[True] * 1e3, 2),
        "layers": [ly.name for ly in ln_layers], "tokens": M,
        "step": "sq_layernorm_quant_pertoken (LayerNorm with gamma/s, beta/s + per-token "
                "quantisation, one kernel); bytes: fp16 x read + int8 codes + steps + gamma/beta",
    }
    log("layernorm+quant (fused): %.2f us per launch (%.0f GB/s); with X_hat also written %.2f us"
        % (ln_ms[False] * 1e3, ln_bytes / ln_ms[False] / 1e6, ln_ms[True] * 1e3))

    # ---- INT8 attention products at the OPT-6.7B-like block's attention
    # shape (32 heads x head_dim 128, 2048 tokens): Q K^T with Q and K per
    # token, P V with P per row and V per head-dim channel; codes resident
    if not args.no_attention:
        out["attention"] = attention_time(dev, args)

    # ---- the larger prefill layer sets (OPT-13B-like, OPT-175B-like)
    if not args.no_larger:
        out["larger_prefill"] = larger_prefill(dev, args)

    # ---- decode shapes
    if not args.no_decode:
        out["decode"] = decode_phase(layers, dev, args)
        out["decode_llama70b"] = decode_llama70b(dev, args)

    # ---- O2 (per-tensor dynamic) and O3 (per-tensor static) activations with
    # per-tensor weights, packed layout
    if not args.no_levels:
        lv = {}
        for mode in ("o2", "o3"):
            sets = [Bufs(layers, M, dev, True, mode) for _ in range(2)]
            ms_l = time_rotation([b.step for b in sets], args.steps, args.warmup)
            q_l = time_rotation([b.quant_only for b in sets], args.steps,
                                args.warmup) / len(layers)
            ent = {"prefill_ms_per_step": round(ms_l, 4),
                   "prefill_tops": round(ops_step / (ms_l * 1e-3) / 1e12, 2),
                   "act_quant_avg_us": round(q_l * 1e3, 2)}
            log("%s prefill: step %.3f ms (%.1f TOPS); act quant avg %.2f us"
                % (mode, ms_l, ops_step / ms_l / 1e9, q_l * 1e3))
            del sets
            torch.cuda.synchronize()
            if mode == "o3" and not args.no_decode:
                for Md in DECODE_M:
                    foot = sum(ly.N * ly.K + Md * ly.K * 3 + Md * ly.N * 2 for ly in layers)
                    R = n_sets(foot)
                    nbytes = sum(ly.N * ly.K + 4 * ly.N + 2 * Md * ly.K + 2 * Md * ly.N + 4 * Md
                                 for ly in layers)
                    sets = [Bufs(layers, Md, dev, True, mode) for _ in range(R)]
                    ms_d = time_rotation([b.step for b in sets], max(args.steps, 4 * R),
                                         args.warmup)
                    gbs = nbytes / (ms_d * 1e-3) / 1e9
                    ent["decode_M=%d" % Md] = {"us_per_step": round(ms_d * 1e3, 2),
                                               "gbs": round(gbs, 1),
                                               "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
                    log("o3 decode M=%d: %.2f us/step, %.0f GB/s (%.1f%% HBM)"
                        % (Md, ms_d * 1e3, gbs, 100 * gbs / PEAK_HBM_GBS))
                    del sets
                    torch.cuda.synchronize()
            lv[mode] = ent
        lv["step"] = ("o2: sq_quant_act_pertensor (dynamic) + sq_w8a8_gemm_dequant_packed; "
                      "o3: sq_w8a8_linear_packed_static (static step from calibration); "
                      "per-tensor weights; 3 layers")
        out["per_tensor_levels"] = lv

    if not args.no_offline:
        out["offline"] = offline_time(dev)
        log("offline", out["offline"])

    if not args.no_cpu_baseline and host is not None:
        out["cpu_baseline"] = cpu_baseline(host, HEAD_M, HEAD_CFG)
        log("cpu baseline", out["cpu_baseline"])
    else:
        out["cpu_baseline"] = None

    print(json.dumps(check_peak_fractions(out)), flush=True)


if __name__ == "__main__":
    main()
