"""Pure-Python brute force for tiny inputs -- TEST INFRASTRUCTURE.

Independent second statements of two oracle steps, used only to pin the C
oracle in ``sqref.c``:

* the INT8 GEMM as the textbook triple loop over Python integers (no numpy
  integer arithmetic, so no int8 wrap-around);
* the symmetric quantiser with fp32 division done by numpy float32 scalars
  and the half-away-from-zero rounding done exactly in Python's double
  (``floor(|t| + 0.5)`` is exact in double for an fp32 ``t``), with the step
  either taken from the values' own range or given (a static step, where the
  clamp to +-127 becomes active).

P1 = abeam.tech SmoothQuant explainer (用語解説 "INT8 GEMM"; 推論方法 O1);
P4 = blogs.itmedia.co.jp 量子化 blog, section 3 (range -> scale -> round).
"""
from __future__ import annotations

import math

import numpy as np


def gemm_int(xq, wq):
    """acc[m][n] = sum_k xq[m][k] * wq[n][k] over Python ints."""
    xs = [[int(v) for v in row] for row in xq]
    ws = [[int(v) for v in row] for row in wq]
    return [[sum(a * b for a, b in zip(xr, wr)) for wr in ws] for xr in xs]


def round_half_away(t: float) -> int:
    a = math.floor(abs(t) + 0.5)
    return -a if t < 0 else a


def quantize_vector(values):
    """Codes and step for one vector, as P4 section 3 and P1 describe it."""
    vals = [np.float32(v) for v in values]
    m = np.float32(0.0)
    for v in vals:
        if abs(v) > m:
            m = np.float32(abs(v))
    step = np.float32(m / np.float32(127.0))
    if step == 0:
        return [0] * len(vals), step
    codes = []
    for v in vals:
        t = float(np.float32(v / step))
        q = round_half_away(t)
        codes.append(max(-127, min(127, q)))
    return codes, step


def quantize_with_step(values, step):
    """Codes for a given fp32 step: round half away from zero, clamp +-127."""
    step = np.float32(step)
    if step == 0:
        return [0] * len(values)
    codes = []
    for v in values:
        t = float(np.float32(np.float32(v) / step))
        codes.append(max(-127, min(127, round_half_away(t))))
    return codes
