"""CPU oracle for the SmoothQuant W8A8 linear layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library
(``w8a8_int8_post_amd``) never imports it, and it imports nothing from the
GPU library: the two share no code.

The arithmetic lives in ``sqref.c`` (plain C, built with gcc
``-O2 -ffp-contract=off -fno-fast-math``); this module only marshals numpy
arrays into it.  The LayerNorm that carries the folded smoothing (fused with
per-token quantisation) is in ``layernorm.py`` (numpy and ``math.fsum``).  Every function takes and returns host numpy arrays.
Input tensors of 16-bit types are widened to float32 by numpy before the call
(exact for fp16 and bf16).

Pages (titles and sections) that each function follows are cited in
``sqref.c``; the short form here:

* P1 = abeam.tech explainer of "SmoothQuant: Accurate and Efficient
  Post-Training Quantization for Large Language Models" (arXiv 2211.10438).
* P4 = blogs.itmedia.co.jp, 「LLMのダイエット術、『量子化（Quantization）』」.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sqref.c")
_LIB = os.path.join(_HERE, "libsqref.so")

MAX_K = 133144  # largest K with K * 127 * 127 < 2**31


def build(force: bool = False) -> str:
    """Compile sqref.c into oracle/libsqref.so with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.sqref_calibrate_absmax.argtypes = [P, I, I, P, ctypes.c_int]
        lib.sqref_weight_row_absmax.argtypes = [P, I, I, P]
        lib.sqref_smoothing_factors.argtypes = [P, P, I, ctypes.c_double, P]
        lib.sqref_fold_weight.argtypes = [P, P, I, I, P]
        lib.sqref_fold_norm.argtypes = [P, I, P, P]
        lib.sqref_smooth_activation.argtypes = [P, P, I, I, P]
        lib.sqref_step.argtypes = [ctypes.c_float]
        lib.sqref_step.restype = ctypes.c_float
        lib.sqref_quantize_value.argtypes = [ctypes.c_float, ctypes.c_float]
        lib.sqref_quantize_value.restype = ctypes.c_int8
        lib.sqref_quantize_vector.argtypes = [P, I, I, P, I]
        lib.sqref_quantize_vector.restype = ctypes.c_float
        lib.sqref_quant_act_pertoken.argtypes = [P, I, I, P, P]
        lib.sqref_quant_weight_perchannel.argtypes = [P, I, I, P, P]
        lib.sqref_quant_act_pertensor.argtypes = [P, I, I, P, P, P]
        lib.sqref_static_act_step.argtypes = [P, P, I]
        lib.sqref_static_act_step.restype = ctypes.c_float
        lib.sqref_quant_weight_pertensor.argtypes = [P, I, I, P, P]
        lib.sqref_gemm_i32.argtypes = [P, P, I, I, I, P]
        lib.sqref_gemm_i32.restype = ctypes.c_int
        lib.sqref_gemm_i32_sampled.argtypes = [P, P, I, P, I, P, I, P]
        lib.sqref_gemm_i32_sampled.restype = ctypes.c_int
        lib.sqref_dequant.argtypes = [P, P, P, I, I, P]
        lib.sqref_dequant_bias_act.argtypes = [P, P, P, P, ctypes.c_int, I, I, P]
        lib.sqref_dequant_bias_act_f32.argtypes = [P, P, P, P, ctypes.c_int, I, I, P]
        lib.sqref_fold_prev_linear.argtypes = [P, P, I, I, P, P]
        lib.sqref_linear_w8a8.argtypes = [P, P, P, I, I, I, P]
        lib.sqref_linear_w8a8.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x) -> np.ndarray:
    """Host float32 C-contiguous copy/view of a numpy array or CPU torch tensor."""
    if hasattr(x, "detach"):  # torch tensor (CPU); widen 16-bit types exactly
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# Offline steps (P1: calibration, smoothing factor, fold; per-channel weights)

def calibrate_absmax(x, a=None):
    """a_j = max_t |x[t, j]|; continues a running max when ``a`` is given."""
    x = _f32(x)
    T, K = x.shape
    acc = 0 if a is None else 1
    out = np.zeros(K, np.float32) if a is None else np.array(a, dtype=np.float32, copy=True)
    _load().sqref_calibrate_absmax(_ptr(x), T, K, _ptr(out), acc)
    return out


def weight_row_absmax(w):
    w = _f32(w)
    K, N = w.shape
    b = np.empty(K, np.float32)
    _load().sqref_weight_row_absmax(_ptr(w), K, N, _ptr(b))
    return b


def smoothing_factors(a, b, alpha: float):
    a = _f32(a)
    b = _f32(b)
    s = np.empty(a.shape[0], np.float32)
    _load().sqref_smoothing_factors(_ptr(a), _ptr(b), a.shape[0], float(alpha), _ptr(s))
    return s


def fold_weight(w, s):
    w = _f32(w)
    s = _f32(s)
    K, N = w.shape
    out = np.empty((K, N), np.float32)
    _load().sqref_fold_weight(_ptr(w), _ptr(s), K, N, _ptr(out))
    return out


def fold_norm(s, gamma=None, beta=None):
    s = _f32(s)
    K = s.shape[0]
    g = None if gamma is None else np.array(_f32(gamma), copy=True)
    bt = None if beta is None else np.array(_f32(beta), copy=True)
    _load().sqref_fold_norm(_ptr(s), K, None if g is None else _ptr(g),
                            None if bt is None else _ptr(bt))
    return g, bt


def smooth_fold(a, w, alpha: float, gamma=None, beta=None):
    """The whole offline transform: (s, W_hat, gamma', beta')."""
    b = weight_row_absmax(w)
    s = smoothing_factors(a, b, alpha)
    w_hat = fold_weight(w, s)
    g, bt = fold_norm(s, gamma, beta)
    return s, w_hat, g, bt


def fold_prev_linear(s, w_prev, bias=None):
    """(W_prev / s per output column [Kp x K] fp32, bias / s or None): the
    smoothing of the next layer folded into the layer before it."""
    s = _f32(s)
    w = _f32(w_prev)
    Kp, K = w.shape
    assert s.shape[0] == K
    out = np.empty((Kp, K), np.float32)
    b = None if bias is None else _f32(bias).copy()
    _load().sqref_fold_prev_linear(_ptr(s), _ptr(w), Kp, K, _ptr(out), None if b is None else _ptr(b))
    return out, b


def smooth_activation(x, s):
    x = _f32(x)
    s = _f32(s)
    M, K = x.shape
    out = np.empty((M, K), np.float32)
    _load().sqref_smooth_activation(_ptr(x), _ptr(s), M, K, _ptr(out))
    return out


# --------------------------------------------------------------------------
# Quantiser (P1 range set by absmax; P4 section 3 range -> scale -> round)

def step(absmax: float) -> float:
    return float(_load().sqref_step(float(absmax)))


def quantize_value(v: float, step_: float) -> int:
    return int(_load().sqref_quantize_value(float(v), float(step_)))


def quantize_vector(v):
    v = _f32(v).ravel()
    q = np.empty(v.shape[0], np.int8)
    st = _load().sqref_quantize_vector(_ptr(v), v.shape[0], 1, _ptr(q), 1)
    return q, np.float32(st)


def quant_act_pertoken(x_hat):
    """(Xq int8 [M x K], sx float32 [M])."""
    x = _f32(x_hat)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    sx = np.empty(M, np.float32)
    _load().sqref_quant_act_pertoken(_ptr(x), M, K, _ptr(xq), _ptr(sx))
    return xq, sx


def quant_act_pertensor(x_hat, step_in=None):
    """(Xq int8 [M x K], sx float32 [M]) with one step for the whole tensor:
    dynamic (absmax / 127) when step_in is None, else the given static step."""
    x = _f32(x_hat)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    sx = np.empty(M, np.float32)
    st = None if step_in is None else np.array([step_in], np.float32)
    _load().sqref_quant_act_pertensor(_ptr(x), M, K, None if st is None else _ptr(st),
                                     _ptr(xq), _ptr(sx))
    return xq, sx


def static_act_step(a, s) -> np.float32:
    """O3 step from the calibration maxima a and the smoothing factors s."""
    a = _f32(a)
    s = _f32(s)
    return np.float32(_load().sqref_static_act_step(_ptr(a), _ptr(s), a.shape[0]))


def quant_weight_pertensor(w_hat):
    """(Wq int8 [N x K], sw float32 [N]) from W_hat [K x N], one step."""
    w = _f32(w_hat)
    K, N = w.shape
    wq = np.empty((N, K), np.int8)
    sw = np.empty(N, np.float32)
    _load().sqref_quant_weight_pertensor(_ptr(w), K, N, _ptr(wq), _ptr(sw))
    return wq, sw


def quant_weight_perchannel(w_hat):
    """(Wq int8 [N x K], sw float32 [N]) from W_hat [K x N]."""
    w = _f32(w_hat)
    K, N = w.shape
    wq = np.empty((N, K), np.int8)
    sw = np.empty(N, np.float32)
    _load().sqref_quant_weight_perchannel(_ptr(w), K, N, _ptr(wq), _ptr(sw))
    return wq, sw


# --------------------------------------------------------------------------
# INT8 GEMM and scale back

def gemm_i32(xq, wq):
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    M, K = xq.shape
    N, K2 = wq.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    rc = _load().sqref_gemm_i32(_ptr(xq), _ptr(wq), M, N, K, _ptr(acc))
    if rc != 0:
        raise ValueError("K=%d exceeds the int32 accumulator bound %d" % (K, MAX_K))
    return acc


def gemm_i32_sampled(xq, wq, rows, cols):
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    K = xq.shape[1]
    assert wq.shape[1] == K
    acc = np.empty((rows.shape[0], cols.shape[0]), np.int32)
    rc = _load().sqref_gemm_i32_sampled(_ptr(xq), _ptr(wq), K, _ptr(rows), rows.shape[0],
                                        _ptr(cols), cols.shape[0], _ptr(acc))
    if rc != 0:
        raise ValueError("K out of range")
    return acc


def dequant(acc, sx, sw):
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    sx = _f32(sx)
    sw = _f32(sw)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    _load().sqref_dequant(_ptr(acc), _ptr(sx), _ptr(sw), M, N, _ptr(y))
    return y


def dequant_bias_act(acc, sx, sw, bias=None, relu=False):
    """acc*sx*sw + bias, then ReLU if asked (double [M x N])."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    sx = _f32(sx)
    sw = _f32(sw)
    M, N = acc.shape
    b = None if bias is None else _f32(bias)
    y = np.empty((M, N), np.float64)
    _load().sqref_dequant_bias_act(_ptr(acc), _ptr(sx), _ptr(sw), None if b is None else _ptr(b),
                                   1 if relu else 0, M, N, _ptr(y))
    return y


def dequant_bias_act_f32(acc, sx, sw, bias=None, relu=False):
    """The same in fp32: RN(RN(fp32(acc) * sx) * sw + bias) with one rounding
    for the multiply-add, then ReLU (float32 [M x N]).  Used where the output
    feeds a quantiser, so that the codes are decided in fp32."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    sx = _f32(sx)
    sw = _f32(sw)
    M, N = acc.shape
    b = None if bias is None else _f32(bias)
    y = np.empty((M, N), np.float32)
    _load().sqref_dequant_bias_act_f32(_ptr(acc), _ptr(sx), _ptr(sw),
                                       None if b is None else _ptr(b), 1 if relu else 0, M, N,
                                       _ptr(y))
    return y


# --------------------------------------------------------------------------
# Attention products (P1 推論方法: the BMMs run in INT8 as well): the same
# steps applied to each batch entry (batch x heads), nothing else.


def bmm_i32(xq, wq):
    """acc [B x M x N] = per entry xq[b] wq[b]^T (exact)."""
    return np.stack([gemm_i32(xq[b], wq[b]) for b in range(xq.shape[0])])


def bmm_dequant(acc, sx, sw):
    """y [B x M x N] (double) = per entry dequant(acc[b], sx[b], sw[b])."""
    return np.stack([dequant(acc[b], sx[b], sw[b]) for b in range(acc.shape[0])])


def quant_weight_perchannel_batched(w):
    """(wq [B x N x K], sw [B x N]) = per entry quant_weight_perchannel(w[b])."""
    outs = [quant_weight_perchannel(w[b]) for b in range(w.shape[0])]
    return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])


def linear_w8a8(x_hat, wq, sw):
    """Per-token quant + INT8 GEMM + scale back, row by row; y float64 [M x N]."""
    x = _f32(x_hat)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    sw = _f32(sw)
    M, K = x.shape
    N = wq.shape[0]
    y = np.empty((M, N), np.float64)
    rc = _load().sqref_linear_w8a8(_ptr(x), _ptr(wq), _ptr(sw), M, N, K, _ptr(y))
    if rc != 0:
        raise ValueError("oracle linear failed (%d)" % rc)
    return y


def set_threads(n: int) -> int:
    """OpenMP threads for the oracle's parallel loops (over token rows); returns
    the number now in effect.  Timing plumbing only: no arithmetic changes."""
    _load()
    gomp = ctypes.CDLL("libgomp.so.1")
    gomp.omp_set_num_threads.argtypes = [ctypes.c_int]
    gomp.omp_set_num_threads(int(n))
    gomp.omp_get_max_threads.restype = ctypes.c_int
    return int(gomp.omp_get_max_threads())
