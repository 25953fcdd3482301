"""Comparison helpers for the GPU-vs-oracle parity tests."""
from __future__ import annotations

import sys

import numpy as np
import torch


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        t = t.float()
    return t.numpy()


def out_ulp(ref: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Spacing of the output dtype at |ref| (fp64 array)."""
    a = np.abs(ref)
    if dtype == torch.float16:
        return np.spacing(a.astype(np.float16)).astype(np.float64)
    if dtype == torch.bfloat16:
        # bf16 keeps fp32's exponent with 8 significant bits
        return np.spacing(a.astype(np.float32)).astype(np.float64) * 65536.0
    return np.spacing(a.astype(np.float32)).astype(np.float64)


def assert_y_close(y_gpu: torch.Tensor, y_ref: np.ndarray, what: str = "y"):
    """Pass where |y - y_ref| <= 1e-3 |y_ref| or <= one ulp of the output dtype.

    1e-3 relative is the stated bar for 16-bit outputs; bf16's half-ulp
    (up to 2^-8 relative) exceeds it, so one output ulp is accepted too.  For
    fp32 outputs the bar is 1e-6 relative (three fp32 roundings)."""
    g = to_np(y_gpu).astype(np.float64)
    assert g.shape == y_ref.shape, (g.shape, y_ref.shape)
    diff = np.abs(g - y_ref)
    rel = 1e-6 if y_gpu.dtype == torch.float32 else 1e-3
    ok = (diff <= rel * np.abs(y_ref)) | (diff <= out_ulp(y_ref, y_gpu.dtype))
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError("%s: %d/%d outside tolerance, e.g. %s" % (
            what, int((~ok).sum()), ok.size,
            [(tuple(b), g[tuple(b)], y_ref[tuple(b)]) for b in bad]))
    # rounding the same fp32 value the same way: report how many are bit-equal
    same = (g == np.asarray(torch.from_numpy(y_ref).to(y_gpu.dtype).double().numpy())).mean()
    return float(same)


def assert_equal(gpu, ref, what: str):
    g = to_np(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    r = np.asarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if not np.array_equal(g, r):
        bad = np.argwhere(g != r)
        raise AssertionError("%s: %d mismatches, first at %s: gpu=%s ref=%s" % (
            what, len(bad), tuple(bad[0]), g[tuple(bad[0])], r[tuple(bad[0])]))


def f32_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in fp32 ulps between positive finite fp32 arrays."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)
