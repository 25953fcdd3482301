"""SmoothQuant W8A8 linear layer on AMD MI355X (gfx950).

Thin Python binding of ``libsq.so`` (C ABI in ``include/sq.h``).  The
functions below carry the C names and only marshal arguments: torch tensors
provide device memory and the HIP stream; every step of the computation runs
in the library's HIP kernels.  There is no fallback: if ``libsq.so`` is not
built, or a tensor is not on the GPU, the call raises.

Method pages (title, section): abeam.tech explainer of "SmoothQuant: Accurate
and Efficient Post-Training Quantization for Large Language Models"
(calibration, smoothing factor, fold, O1 per-token activations, INT8 GEMM);
blogs.itmedia.co.jp 「LLMのダイエット術、『量子化（Quantization）』」 section 3
(range -> scale -> round, scale back).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SQError", "load_library", "version",
    "sq_calibrate_absmax", "sq_smooth_fold", "sq_quant_weight_perchannel",
    "sq_quant_act_pertoken", "sq_w8a8_gemm_dequant", "sq_w8a8_gemm_i32",
    "sq_smooth_activation", "sq_packed_weight_bytes", "sq_pack_weight",
    "sq_w8a8_gemm_dequant_packed", "sq_w8a8_gemm_i32_packed", "pack_weight",
    "w8a8_gemm_dequant_packed", "w8a8_gemm_i32_packed", "linear_w8a8_packed",
    "sq_w8a8_linear_packed", "sq_w8a8_linear_packed_static", "sq_quant_act_pertensor", "sq_static_act_step",
    "sq_quant_weight_pertensor", "quant_act_pertensor", "static_act_step",
    "quant_weight_pertensor", "linear_w8a8_packed_static", "sq_w8a8_gemm_dequant_ex",
    "sq_w8a8_gemm_dequant_packed_ex", "sq_fold_prev_linear", "w8a8_gemm_dequant_ex",
    "w8a8_gemm_dequant_packed_ex", "fold_prev_linear", "SQ_ACT_NONE", "SQ_ACT_RELU",
    "sq_layernorm_quant_pertoken", "layernorm_quant_pertoken", "sq_w8a8_bmm_dequant",
    "sq_w8a8_bmm_i32", "sq_quant_weight_perchannel_batched", "w8a8_bmm_dequant", "w8a8_bmm_i32",
    "quant_weight_perchannel_batched", "sq_w8a8_gemm_dequant_packed_noalloc",
    "sq_noalloc_scratch_bytes", "sq_w8a8_linear_packed_ws", "sq_linear_workspace_bytes",
    "linear_workspace", "linear_w8a8_packed_ws",
    "calibrate_absmax", "smooth_fold", "quant_weight_perchannel", "quant_act_pertoken",
    "w8a8_gemm_dequant", "w8a8_gemm_i32", "smooth_activation", "linear_w8a8",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsq.so")

STATUS = {0: "SQ_OK", 1: "SQ_ERR_NULL", 2: "SQ_ERR_SHAPE", 3: "SQ_ERR_DTYPE",
          4: "SQ_ERR_K_OVERFLOW", 5: "SQ_ERR_ALIGN", 6: "SQ_ERR_ALPHA", 7: "SQ_ERR_HIP",
          8: "SQ_ERR_ALIAS", 9: "SQ_ERR_ACT", 10: "SQ_ERR_EPS",
          11: "SQ_ERR_WORKSPACE"}
SQ_F32, SQ_F16, SQ_BF16 = 0, 1, 2
SQ_ACT_NONE, SQ_ACT_RELU = 0, 1
_DT = {torch.float32: SQ_F32, torch.float16: SQ_F16, torch.bfloat16: SQ_BF16}
MAX_K = 133144


class SQError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__("%s returned %s" % (fn, STATUS.get(code, code)))
        self.code = code


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libsq.so and declare the C signatures (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsq.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, E = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sigs = {
            "sq_calibrate_absmax": [P, E, I64, I64, P, E, P],
            "sq_smooth_fold": [P, P, E, I64, I64, ctypes.c_double, P, P, P, P, P],
            "sq_quant_weight_perchannel": [P, E, I64, I64, P, P, P],
            "sq_quant_act_pertoken": [P, E, I64, I64, P, P, P, P],
            "sq_w8a8_gemm_dequant": [P, P, P, P, I64, I64, I64, P, E, P],
            "sq_w8a8_gemm_i32": [P, P, I64, I64, I64, P, P],
            "sq_smooth_activation": [P, E, I64, I64, P, P, P],
            "sq_pack_weight": [P, I64, I64, P, P],
            "sq_w8a8_gemm_dequant_packed": [P, P, P, P, I64, I64, I64, P, E, P],
            "sq_w8a8_gemm_i32_packed": [P, P, I64, I64, I64, P, P],
            "sq_w8a8_linear_packed": [P, E, I64, I64, P, P, I64, P, P, P, E, P],
            "sq_w8a8_linear_packed_static": [P, E, I64, I64, P, P, I64, P, P, P, P, E, P],
            "sq_quant_act_pertensor": [P, E, I64, I64, P, P, P, P, P],
            "sq_w8a8_gemm_dequant_ex": [P, P, P, P, P, E, I64, I64, I64, P, E, P],
            "sq_w8a8_gemm_dequant_packed_ex": [P, P, P, P, P, E, I64, I64, I64, P, E, P],
            "sq_fold_prev_linear": [P, P, E, I64, I64, P, P, P],
            "sq_layernorm_quant_pertoken": [P, E, I64, I64, P, P, ctypes.c_double, P, P, P, P],
            "sq_w8a8_bmm_dequant": [P, P, P, P, I64, I64, I64, I64, P, E, P],
            "sq_w8a8_bmm_i32": [P, P, I64, I64, I64, I64, P, P],
            "sq_quant_weight_perchannel_batched": [P, E, I64, I64, I64, P, P, P],
            "sq_static_act_step": [P, P, I64, P, P],
            "sq_quant_weight_pertensor": [P, E, I64, I64, P, P, P],
            "sq_w8a8_gemm_dequant_ws": [P, P, P, P, I64, I64, I64, P, E, P, I64, P],
            "sq_w8a8_gemm_dequant_packed_ws": [P, P, P, P, I64, I64, I64, P, E, P, I64, P],
            "sq_w8a8_gemm_dequant_packed_noalloc": [P, P, P, P, I64, I64, I64, P, E, P],
            "sq_w8a8_linear_packed_ws": [P, E, I64, I64, P, P, I64, P, P, P, E, P, I64, P],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.sq_packed_weight_bytes.argtypes = [I64, I64]
        lib.sq_packed_weight_bytes.restype = I64
        lib.sq_gemm_workspace_bytes.argtypes = [I64, I64, I64]
        lib.sq_gemm_workspace_bytes.restype = I64
        lib.sq_noalloc_scratch_bytes.argtypes = []
        lib.sq_noalloc_scratch_bytes.restype = I64
        lib.sq_linear_workspace_bytes.argtypes = [E, I64, I64, I64]
        lib.sq_linear_workspace_bytes.restype = I64
        lib.sq_version.argtypes = []
        lib.sq_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def version() -> str:
    return load_library().sq_version().decode()


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s" % (name, t.dtype))
    return t.data_ptr()


def _opt(t, name, dtype=None):
    return None if t is None else _dev(t, name, dtype)


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _call(name: str, *args):
    rc = getattr(load_library(), name)(*args)
    if rc != 0:
        raise SQError(name, rc)


# --------------------------------------------------------------------------
# C entry points (same names, same argument order, tensors for pointers)

def sq_calibrate_absmax(x, a, accumulate: bool = False, stream=None):
    T, K = x.shape
    _call("sq_calibrate_absmax", _dev(x, "x"), _DT[x.dtype], T, K, _dev(a, "a", torch.float32),
          1 if accumulate else 0, _stream(x, stream))


def sq_smooth_fold(a, w, alpha: float, s_out, w_out, gamma=None, beta=None, stream=None):
    K, N = w.shape
    _call("sq_smooth_fold", _dev(a, "a", torch.float32), _dev(w, "w"), _DT[w.dtype], K, N,
          float(alpha), _dev(s_out, "s_out", torch.float32), _dev(w_out, "w_out", torch.float32),
          _opt(gamma, "gamma", torch.float32), _opt(beta, "beta", torch.float32),
          _stream(w, stream))


def sq_quant_weight_perchannel(w, wq, w_scale, stream=None):
    K, N = w.shape
    _call("sq_quant_weight_perchannel", _dev(w, "w"), _DT[w.dtype], K, N,
          _dev(wq, "wq", torch.int8), _dev(w_scale, "w_scale", torch.float32), _stream(w, stream))


def sq_quant_act_pertoken(x, xq, x_scale, smooth=None, stream=None):
    M, K = x.shape
    _call("sq_quant_act_pertoken", _dev(x, "x"), _DT[x.dtype], M, K,
          _opt(smooth, "smooth", torch.float32), _dev(xq, "xq", torch.int8),
          _dev(x_scale, "x_scale", torch.float32), _stream(x, stream))


def sq_w8a8_linear_packed_static(x, wq_packed, w_scale, step_in, xq, x_scale, y, stream=None):
    M, K = x.shape
    N = w_scale.shape[0]
    if tuple(xq.shape) != (M, K) or tuple(y.shape) != (M, N) or x_scale.shape[0] != M:
        raise ValueError("shape mismatch")
    _check_packed(wq_packed, N, K)
    _call("sq_w8a8_linear_packed_static", _dev(x, "x"), _DT[x.dtype], M, K,
          _dev(wq_packed, "wq_packed", torch.int8), _dev(w_scale, "w_scale", torch.float32), N,
          _dev(step_in, "step_in", torch.float32), _dev(xq, "xq", torch.int8),
          _dev(x_scale, "x_scale", torch.float32), _dev(y, "y"), _DT[y.dtype], _stream(x, stream))


def sq_quant_act_pertensor(x, xq, x_scale, smooth=None, step_in=None, stream=None):
    M, K = x.shape
    if tuple(xq.shape) != (M, K) or x_scale.shape[0] != M:
        raise ValueError("shape mismatch")
    _call("sq_quant_act_pertensor", _dev(x, "x"), _DT[x.dtype], M, K,
          _opt(smooth, "smooth", torch.float32), _opt(step_in, "step_in", torch.float32),
          _dev(xq, "xq", torch.int8), _dev(x_scale, "x_scale", torch.float32), _stream(x, stream))


def sq_static_act_step(a, s, step_out, stream=None):
    K = a.shape[0]
    if s.shape[0] != K or step_out.numel() < 1:
        raise ValueError("shape mismatch")
    _call("sq_static_act_step", _dev(a, "a", torch.float32), _dev(s, "s", torch.float32), K,
          _dev(step_out, "step_out", torch.float32), _stream(a, stream))


def sq_quant_weight_pertensor(w, wq, w_scale, stream=None):
    K, N = w.shape
    _call("sq_quant_weight_pertensor", _dev(w, "w"), _DT[w.dtype], K, N,
          _dev(wq, "wq", torch.int8), _dev(w_scale, "w_scale", torch.float32), _stream(w, stream))


def sq_w8a8_gemm_dequant(xq, x_scale, wq, w_scale, y, stream=None):
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError("shape mismatch")
    _call("sq_w8a8_gemm_dequant", _dev(xq, "xq", torch.int8), _dev(x_scale, "x_scale", torch.float32),
          _dev(wq, "wq", torch.int8), _dev(w_scale, "w_scale", torch.float32), M, N, K,
          _dev(y, "y"), _DT[y.dtype], _stream(xq, stream))


def sq_w8a8_gemm_dequant_ex(xq, x_scale, wq, w_scale, bias, act, y, stream=None):
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or tuple(y.shape) != (M, N) or (bias is not None and bias.shape[0] != N):
        raise ValueError("shape mismatch")
    _call("sq_w8a8_gemm_dequant_ex", _dev(xq, "xq", torch.int8),
          _dev(x_scale, "x_scale", torch.float32), _dev(wq, "wq", torch.int8),
          _dev(w_scale, "w_scale", torch.float32), _opt(bias, "bias", torch.float32), int(act),
          M, N, K, _dev(y, "y"), _DT[y.dtype], _stream(xq, stream))


def sq_w8a8_gemm_i32(xq, wq, acc, stream=None):
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or tuple(acc.shape) != (M, N):
        raise ValueError("shape mismatch")
    _call("sq_w8a8_gemm_i32", _dev(xq, "xq", torch.int8), _dev(wq, "wq", torch.int8), M, N, K,
          _dev(acc, "acc", torch.int32), _stream(xq, stream))


def sq_w8a8_bmm_dequant(xq, x_scale, wq, w_scale, y, stream=None):
    B, M, K = xq.shape
    N = wq.shape[1]
    if tuple(wq.shape) != (B, N, K) or tuple(x_scale.shape) != (B, M) \
            or tuple(w_scale.shape) != (B, N) or tuple(y.shape) != (B, M, N):
        raise ValueError("shape mismatch")
    _call("sq_w8a8_bmm_dequant", _dev(xq, "xq", torch.int8), _dev(x_scale, "x_scale", torch.float32),
          _dev(wq, "wq", torch.int8), _dev(w_scale, "w_scale", torch.float32), B, M, N, K,
          _dev(y, "y"), _DT[y.dtype], _stream(xq, stream))


def sq_w8a8_bmm_i32(xq, wq, acc, stream=None):
    B, M, K = xq.shape
    N = wq.shape[1]
    if tuple(wq.shape) != (B, N, K) or tuple(acc.shape) != (B, M, N):
        raise ValueError("shape mismatch")
    _call("sq_w8a8_bmm_i32", _dev(xq, "xq", torch.int8), _dev(wq, "wq", torch.int8), B, M, N, K,
          _dev(acc, "acc", torch.int32), _stream(xq, stream))


def sq_quant_weight_perchannel_batched(w, wq, w_scale, stream=None):
    B, K, N = w.shape
    if tuple(wq.shape) != (B, N, K) or tuple(w_scale.shape) != (B, N):
        raise ValueError("shape mismatch")
    _call("sq_quant_weight_perchannel_batched", _dev(w, "w"), _DT[w.dtype], B, K, N,
          _dev(wq, "wq", torch.int8), _dev(w_scale, "w_scale", torch.float32), _stream(w, stream))


def sq_smooth_activation(x, s, x_hat, stream=None):
    M, K = x.shape
    if x_hat.dtype != x.dtype or x_hat.shape != x.shape:
        raise ValueError("x_hat must match x")
    _call("sq_smooth_activation", _dev(x, "x"), _DT[x.dtype], M, K, _dev(s, "s", torch.float32),
          _dev(x_hat, "x_hat"), _stream(x, stream))


def sq_packed_weight_bytes(N: int, K: int) -> int:
    return int(load_library().sq_packed_weight_bytes(N, K))


def sq_pack_weight(wq, wq_packed, stream=None):
    N, K = wq.shape
    _check_packed(wq_packed, N, K)
    _call("sq_pack_weight", _dev(wq, "wq", torch.int8), N, K, _dev(wq_packed, "wq_packed", torch.int8),
          _stream(wq, stream))


def _check_packed(wq_packed, N, K):
    need = sq_packed_weight_bytes(N, K)
    if need < 0 or wq_packed.numel() * wq_packed.element_size() < need:
        raise ValueError("packed weight buffer too small for N=%d K=%d" % (N, K))


def sq_w8a8_gemm_dequant_packed(xq, x_scale, wq_packed, w_scale, N, y, stream=None):
    M, K = xq.shape
    if tuple(y.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check_packed(wq_packed, N, K)
    _call("sq_w8a8_gemm_dequant_packed", _dev(xq, "xq", torch.int8),
          _dev(x_scale, "x_scale", torch.float32), _dev(wq_packed, "wq_packed", torch.int8),
          _dev(w_scale, "w_scale", torch.float32), M, N, K, _dev(y, "y"), _DT[y.dtype],
          _stream(xq, stream))


def sq_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes the split-K entry points need for this shape on the
    current device (0: no split, the plain GEMM runs)."""
    n = load_library().sq_gemm_workspace_bytes(M, N, K)
    if n < 0:
        raise ValueError("invalid shape")
    return n


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def sq_w8a8_gemm_dequant_ws(xq, x_scale, wq, w_scale, y, workspace, stream=None):
    M, K = xq.shape
    N = wq.shape[0]
    if tuple(wq.shape) != (N, K) or tuple(y.shape) != (M, N):
        raise ValueError("shape mismatch")
    wp, wb = _ws(workspace)
    _call("sq_w8a8_gemm_dequant_ws", _dev(xq, "xq", torch.int8),
          _dev(x_scale, "x_scale", torch.float32), _dev(wq, "wq", torch.int8),
          _dev(w_scale, "w_scale", torch.float32), M, N, K, _dev(y, "y"), _DT[y.dtype], wp, wb,
          _stream(xq, stream))


def sq_w8a8_gemm_dequant_packed_ws(xq, x_scale, wq_packed, w_scale, N, y, workspace,
                                   stream=None):
    M, K = xq.shape
    if tuple(y.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check_packed(wq_packed, N, K)
    wp, wb = _ws(workspace)
    _call("sq_w8a8_gemm_dequant_packed_ws", _dev(xq, "xq", torch.int8),
          _dev(x_scale, "x_scale", torch.float32), _dev(wq_packed, "wq_packed", torch.int8),
          _dev(w_scale, "w_scale", torch.float32), M, N, K, _dev(y, "y"), _DT[y.dtype], wp, wb,
          _stream(xq, stream))


def sq_w8a8_gemm_dequant_packed_noalloc(xq, x_scale, wq_packed, w_scale, N, y, stream=None):
    """Split-K packed GEMM with the library's static scratch (allocates nothing)."""
    M, K = xq.shape
    if tuple(y.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check_packed(wq_packed, N, K)
    _call("sq_w8a8_gemm_dequant_packed_noalloc", _dev(xq, "xq", torch.int8),
          _dev(x_scale, "x_scale", torch.float32), _dev(wq_packed, "wq_packed", torch.int8),
          _dev(w_scale, "w_scale", torch.float32), M, N, K, _dev(y, "y"), _DT[y.dtype],
          _stream(xq, stream))


def sq_noalloc_scratch_bytes() -> int:
    return int(load_library().sq_noalloc_scratch_bytes())


def sq_w8a8_gemm_dequant_packed_ex(xq, x_scale, wq_packed, w_scale, bias, act, N, y,
                                   stream=None):
    M, K = xq.shape
    if tuple(y.shape) != (M, N) or (bias is not None and bias.shape[0] != N):
        raise ValueError("shape mismatch")
    _check_packed(wq_packed, N, K)
    _call("sq_w8a8_gemm_dequant_packed_ex", _dev(xq, "xq", torch.int8),
          _dev(x_scale, "x_scale", torch.float32), _dev(wq_packed, "wq_packed", torch.int8),
          _dev(w_scale, "w_scale", torch.float32), _opt(bias, "bias", torch.float32), int(act),
          M, N, K, _dev(y, "y"), _DT[y.dtype], _stream(xq, stream))


def sq_fold_prev_linear(s, w_prev, w_out, bias=None, stream=None):
    Kp, K = w_prev.shape
    if s.shape[0] != K or tuple(w_out.shape) != (Kp, K) or (bias is not None and bias.shape[0] != K):
        raise ValueError("shape mismatch")
    _call("sq_fold_prev_linear", _dev(s, "s", torch.float32), _dev(w_prev, "w_prev"),
          _DT[w_prev.dtype], Kp, K, _dev(w_out, "w_out", torch.float32),
          _opt(bias, "bias", torch.float32), _stream(w_prev, stream))


def sq_layernorm_quant_pertoken(x, gamma, beta, eps, xq, x_scale, x_hat=None, stream=None):
    M, K = x.shape
    if gamma.shape[0] != K or beta.shape[0] != K or tuple(xq.shape) != (M, K) \
            or x_scale.shape[0] != M or (x_hat is not None and tuple(x_hat.shape) != (M, K)):
        raise ValueError("shape mismatch")
    if x_hat is not None and x_hat.dtype != x.dtype:
        raise TypeError("x_hat must have x's dtype")
    _call("sq_layernorm_quant_pertoken", _dev(x, "x"), _DT[x.dtype], M, K,
          _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32), float(eps),
          _dev(xq, "xq", torch.int8), _dev(x_scale, "x_scale", torch.float32),
          _opt(x_hat, "x_hat"), _stream(x, stream))


def sq_w8a8_gemm_i32_packed(xq, wq_packed, N, acc, stream=None):
    M, K = xq.shape
    if tuple(acc.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check_packed(wq_packed, N, K)
    _call("sq_w8a8_gemm_i32_packed", _dev(xq, "xq", torch.int8),
          _dev(wq_packed, "wq_packed", torch.int8), M, N, K, _dev(acc, "acc", torch.int32),
          _stream(xq, stream))


def sq_w8a8_linear_packed(x, wq_packed, w_scale, xq, x_scale, y, stream=None):
    M, K = x.shape
    N = w_scale.shape[0]
    if tuple(xq.shape) != (M, K) or tuple(y.shape) != (M, N) or x_scale.shape[0] != M:
        raise ValueError("shape mismatch")
    _check_packed(wq_packed, N, K)
    _call("sq_w8a8_linear_packed", _dev(x, "x"), _DT[x.dtype], M, K,
          _dev(wq_packed, "wq_packed", torch.int8), _dev(w_scale, "w_scale", torch.float32), N,
          _dev(xq, "xq", torch.int8), _dev(x_scale, "x_scale", torch.float32), _dev(y, "y"),
          _DT[y.dtype], _stream(x, stream))


def sq_linear_workspace_bytes(x_dtype, M: int, N: int, K: int) -> int:
    n = load_library().sq_linear_workspace_bytes(_DT[x_dtype], M, N, K)
    if n < 0:
        raise ValueError("invalid shape")
    return n


def sq_w8a8_linear_packed_ws(x, wq_packed, w_scale, xq, x_scale, y, workspace, stream=None):
    M, K = x.shape
    N = w_scale.shape[0]
    if tuple(xq.shape) != (M, K) or tuple(y.shape) != (M, N) or x_scale.shape[0] != M:
        raise ValueError("shape mismatch")
    _check_packed(wq_packed, N, K)
    wp, wb = _ws(workspace)
    _call("sq_w8a8_linear_packed_ws", _dev(x, "x"), _DT[x.dtype], M, K,
          _dev(wq_packed, "wq_packed", torch.int8), _dev(w_scale, "w_scale", torch.float32), N,
          _dev(xq, "xq", torch.int8), _dev(x_scale, "x_scale", torch.float32), _dev(y, "y"),
          _DT[y.dtype], wp, wb, _stream(x, stream))


# --------------------------------------------------------------------------
# Allocating conveniences (outputs from torch.empty on the input's device)

def calibrate_absmax(x, a=None, stream=None):
    if a is None:
        a = torch.empty(x.shape[1], dtype=torch.float32, device=x.device)
        sq_calibrate_absmax(x, a, False, stream)
    else:
        sq_calibrate_absmax(x, a, True, stream)
    return a


def smooth_fold(a, w, alpha: float, gamma=None, beta=None, stream=None):
    K, N = w.shape
    s = torch.empty(K, dtype=torch.float32, device=w.device)
    w_hat = torch.empty(K, N, dtype=torch.float32, device=w.device)
    sq_smooth_fold(a, w, alpha, s, w_hat, gamma, beta, stream)
    return s, w_hat


def quant_weight_perchannel(w, stream=None):
    K, N = w.shape
    wq = torch.empty(N, K, dtype=torch.int8, device=w.device)
    sw = torch.empty(N, dtype=torch.float32, device=w.device)
    sq_quant_weight_perchannel(w, wq, sw, stream)
    return wq, sw


def quant_act_pertoken(x, smooth=None, stream=None):
    M, K = x.shape
    xq = torch.empty(M, K, dtype=torch.int8, device=x.device)
    sx = torch.empty(M, dtype=torch.float32, device=x.device)
    sq_quant_act_pertoken(x, xq, sx, smooth, stream)
    return xq, sx


def quant_act_pertensor(x, smooth=None, step_in=None, stream=None):
    """O2 (step_in None: dynamic) or O3 (step_in: a 1-element device step)."""
    M, K = x.shape
    xq = torch.empty(M, K, dtype=torch.int8, device=x.device)
    sx = torch.empty(M, dtype=torch.float32, device=x.device)
    sq_quant_act_pertensor(x, xq, sx, smooth, step_in, stream)
    return xq, sx


def static_act_step(a, s, stream=None):
    out = torch.empty(1, dtype=torch.float32, device=a.device)
    sq_static_act_step(a, s, out, stream)
    return out


def quant_weight_pertensor(w, stream=None):
    K, N = w.shape
    wq = torch.empty(N, K, dtype=torch.int8, device=w.device)
    sw = torch.empty(N, dtype=torch.float32, device=w.device)
    sq_quant_weight_pertensor(w, wq, sw, stream)
    return wq, sw


def w8a8_gemm_dequant(xq, x_scale, wq, w_scale, out_dtype=torch.float16, stream=None):
    y = torch.empty(xq.shape[0], wq.shape[0], dtype=out_dtype, device=xq.device)
    sq_w8a8_gemm_dequant(xq, x_scale, wq, w_scale, y, stream)
    return y


def w8a8_gemm_dequant_ex(xq, x_scale, wq, w_scale, bias=None, act=SQ_ACT_NONE,
                         out_dtype=torch.float16, stream=None):
    y = torch.empty(xq.shape[0], wq.shape[0], dtype=out_dtype, device=xq.device)
    sq_w8a8_gemm_dequant_ex(xq, x_scale, wq, w_scale, bias, act, y, stream)
    return y


def w8a8_gemm_dequant_packed_ex(xq, x_scale, wq_packed, w_scale, bias=None, act=SQ_ACT_NONE,
                                out_dtype=torch.float16, stream=None):
    N = w_scale.shape[0]
    y = torch.empty(xq.shape[0], N, dtype=out_dtype, device=xq.device)
    sq_w8a8_gemm_dequant_packed_ex(xq, x_scale, wq_packed, w_scale, bias, act, N, y, stream)
    return y


def fold_prev_linear(s, w_prev, bias=None, stream=None):
    """(W_prev / s per output column, fp32; bias is divided in place)."""
    out = torch.empty(w_prev.shape, dtype=torch.float32, device=w_prev.device)
    sq_fold_prev_linear(s, w_prev, out, bias, stream)
    return out


def layernorm_quant_pertoken(x, gamma, beta, eps=1e-5, want_x_hat=False, stream=None):
    """(xq, x_scale[, x_hat]): LayerNorm with the folded (gamma, beta), then
    per-token quantisation, in one kernel."""
    M, K = x.shape
    xq = torch.empty(M, K, dtype=torch.int8, device=x.device)
    sx = torch.empty(M, dtype=torch.float32, device=x.device)
    xh = torch.empty_like(x) if want_x_hat else None
    sq_layernorm_quant_pertoken(x, gamma, beta, eps, xq, sx, xh, stream)
    return (xq, sx, xh) if want_x_hat else (xq, sx)


def w8a8_bmm_dequant(xq, x_scale, wq, w_scale, out_dtype=torch.float16, stream=None):
    """y [B x M x N] = scale back of the batched INT8 products xq[b] wq[b]^T."""
    B, M, _ = xq.shape
    y = torch.empty(B, M, wq.shape[1], dtype=out_dtype, device=xq.device)
    sq_w8a8_bmm_dequant(xq, x_scale, wq, w_scale, y, stream)
    return y


def w8a8_bmm_i32(xq, wq, stream=None):
    B, M, _ = xq.shape
    acc = torch.empty(B, M, wq.shape[1], dtype=torch.int32, device=xq.device)
    sq_w8a8_bmm_i32(xq, wq, acc, stream)
    return acc


def quant_weight_perchannel_batched(w, stream=None):
    """(wq [B x N x K], w_scale [B x N]) from w [B x K x N] (e.g. V per head)."""
    B, K, N = w.shape
    wq = torch.empty(B, N, K, dtype=torch.int8, device=w.device)
    sw = torch.empty(B, N, dtype=torch.float32, device=w.device)
    sq_quant_weight_perchannel_batched(w, wq, sw, stream)
    return wq, sw


def w8a8_gemm_i32(xq, wq, stream=None):
    acc = torch.empty(xq.shape[0], wq.shape[0], dtype=torch.int32, device=xq.device)
    sq_w8a8_gemm_i32(xq, wq, acc, stream)
    return acc


def smooth_activation(x, s, stream=None):
    out = torch.empty_like(x)
    sq_smooth_activation(x, s, out, stream)
    return out


def pack_weight(wq, stream=None):
    """Fragment-packed copy of wq [N x K] (1-D int8 tensor)."""
    N, K = wq.shape
    nbytes = sq_packed_weight_bytes(N, K)
    if nbytes < 0:
        raise SQError("sq_packed_weight_bytes", 2)
    wp = torch.empty(nbytes, dtype=torch.int8, device=wq.device)
    sq_pack_weight(wq, wp, stream)
    return wp


def w8a8_gemm_dequant_packed(xq, x_scale, wq_packed, w_scale, out_dtype=torch.float16,
                             stream=None):
    N = w_scale.shape[0]
    y = torch.empty(xq.shape[0], N, dtype=out_dtype, device=xq.device)
    sq_w8a8_gemm_dequant_packed(xq, x_scale, wq_packed, w_scale, N, y, stream)
    return y


def gemm_workspace(M: int, N: int, K: int, device) -> torch.Tensor:
    """A zero-filled workspace for the split-K entry points (at least 16
    bytes, so that a shape without a split still gets a valid pointer)."""
    n = max(sq_gemm_workspace_bytes(M, N, K), 16)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def w8a8_gemm_dequant_packed_ws(xq, x_scale, wq_packed, w_scale, out_dtype=torch.float16,
                                workspace=None, stream=None):
    N = w_scale.shape[0]
    M, K = xq.shape
    if workspace is None:
        workspace = gemm_workspace(M, N, K, xq.device)
    y = torch.empty(M, N, dtype=out_dtype, device=xq.device)
    sq_w8a8_gemm_dequant_packed_ws(xq, x_scale, wq_packed, w_scale, N, y, workspace, stream)
    return y


def w8a8_gemm_i32_packed(xq, wq_packed, N, stream=None):
    acc = torch.empty(xq.shape[0], N, dtype=torch.int32, device=xq.device)
    sq_w8a8_gemm_i32_packed(xq, wq_packed, N, acc, stream)
    return acc


def linear_w8a8_packed(x_hat, wq_packed, w_scale, out_dtype=torch.float16, stream=None):
    """Run-time layer on packed weights (sq_w8a8_linear_packed): (y, xq, sx)."""
    M, K = x_hat.shape
    N = w_scale.shape[0]
    xq = torch.empty(M, K, dtype=torch.int8, device=x_hat.device)
    sx = torch.empty(M, dtype=torch.float32, device=x_hat.device)
    y = torch.empty(M, N, dtype=out_dtype, device=x_hat.device)
    sq_w8a8_linear_packed(x_hat, wq_packed, w_scale, xq, sx, y, stream)
    return y, xq, sx


def linear_workspace(x_dtype, M: int, N: int, K: int, device) -> torch.Tensor:
    """A workspace for sq_w8a8_linear_packed_ws (at least 16 bytes, so that a
    shape that needs none still gets a valid pointer)."""
    n = max(sq_linear_workspace_bytes(x_dtype, M, N, K), 16)
    return torch.empty(n, dtype=torch.uint8, device=device)


def linear_w8a8_packed_ws(x_hat, wq_packed, w_scale, out_dtype=torch.float16, workspace=None,
                          stream=None):
    """sq_w8a8_linear_packed_ws: (y, xq, sx)."""
    M, K = x_hat.shape
    N = w_scale.shape[0]
    if workspace is None:
        workspace = linear_workspace(x_hat.dtype, M, N, K, x_hat.device)
    xq = torch.empty(M, K, dtype=torch.int8, device=x_hat.device)
    sx = torch.empty(M, dtype=torch.float32, device=x_hat.device)
    y = torch.empty(M, N, dtype=out_dtype, device=x_hat.device)
    sq_w8a8_linear_packed_ws(x_hat, wq_packed, w_scale, xq, sx, y, workspace, stream)
    return y, xq, sx


def linear_w8a8_packed_static(x_hat, wq_packed, w_scale, step_in, out_dtype=torch.float16,
                              stream=None):
    """O3 run-time layer on packed weights (sq_w8a8_linear_packed_static): (y, xq, sx)."""
    M, K = x_hat.shape
    N = w_scale.shape[0]
    xq = torch.empty(M, K, dtype=torch.int8, device=x_hat.device)
    sx = torch.empty(M, dtype=torch.float32, device=x_hat.device)
    y = torch.empty(M, N, dtype=out_dtype, device=x_hat.device)
    sq_w8a8_linear_packed_static(x_hat, wq_packed, w_scale, step_in, xq, sx, y, stream)
    return y, xq, sx


def linear_w8a8(x_hat, wq, w_scale, out_dtype=torch.float16, stream=None):
    """Run-time layer: per-token quantisation then INT8 GEMM + scale back."""
    xq, sx = quant_act_pertoken(x_hat, None, stream)
    return w8a8_gemm_dequant(xq, sx, wq, w_scale, out_dtype, stream)
