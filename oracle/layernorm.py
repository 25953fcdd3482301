"""CPU oracle for the LayerNorm that carries the folded smoothing factors,
fused with per-token quantisation -- TEST INFRASTRUCTURE (same rules as the
rest of ``oracle/``: only tests, the smoke check and the CPU baseline use it).

P1 (abeam.tech explainer of "SmoothQuant: Accurate and Efficient Post-Training
Quantization for Large Language Models"), section 数学的に何をしているのか,
folds diag(s)^-1 into the LayerNorm in front of a linear layer, so that the
LayerNorm itself emits the smoothed activation X_hat; P1 推論方法 then
quantises X_hat per token (O1).  The pages name the LayerNorm but do not
write it out; this is the standard layer normalisation of each token row
(Ba, Kiros and Hinton, "Layer Normalization", 2016), with epsilon inside the
square root:

    y_k = (x_k - mean(x)) / sqrt(var(x) + eps) * gamma_k + beta_k,
    var(x) = mean((x - mean(x))^2)        (biased, over the K channels).

Precision (the pages fix none; these are the readings, and the quantised
codes downstream depend on them):

* statistics in double from correctly rounded sums (``math.fsum``):
  S = fsum(x), mu_d = S / K, Q = fsum((x - mu_d)^2) with each difference and
  square rounded to double, var_d = Q / K, rstd_d = 1 / sqrt(var_d + eps);
  then mu = fp32(mu_d) and rstd = fp32(rstd_d) (round to nearest even);
* the element-wise part in fp32, one rounding per operation, in the order
  ((x - mu) * rstd) * gamma + beta, no fused multiply-add;
* the result is stored in the activation dtype (round to nearest even), as an
  unfused LayerNorm would write it, and those stored values are quantised
  per token exactly as ``quant_act_pertoken`` does.

A GPU that sums in double in another order reaches the same fp32 mu and
rstd unless the exact statistic lies within that summation's error bound of
an fp32 rounding boundary; ``ambiguous_rows`` reports such rows, and
``admissible_stats`` / ``row_alternatives`` enumerate every fp32 (mu, rstd)
such a summation may give and the row's results under each, so that a test
can require the GPU's row to equal one of them.
"""
from __future__ import annotations

import math

import numpy as np


def _row_stats(row: np.ndarray, eps: float):
    """(mu_d, var_d, rstd_d) of one row of exact float64 values."""
    K = row.shape[0]
    mu_d = math.fsum(row.tolist()) / K
    d = row - mu_d
    var_d = math.fsum((d * d).tolist()) / K
    rstd_d = 1.0 / math.sqrt(var_d + eps)
    return mu_d, var_d, rstd_d


def layernorm_stats(x, eps: float):
    """Per-row (mu fp32 [M], rstd fp32 [M]) following the stated precision."""
    x = np.asarray(x, np.float32).astype(np.float64)
    mu = np.empty(x.shape[0], np.float32)
    rstd = np.empty(x.shape[0], np.float32)
    for m in range(x.shape[0]):
        mu_d, _, rstd_d = _row_stats(x[m], eps)
        mu[m] = np.float32(mu_d)
        rstd[m] = np.float32(rstd_d)
    return mu, rstd


def layernorm_f32(x, gamma, beta, eps: float, stats=None):
    """fp32 LayerNorm output [M x K] (before the store in the activation
    dtype); ``stats`` = (mu, rstd) fp32 [M] replaces the row statistics."""
    x32 = np.asarray(x, np.float32)
    mu, rstd = layernorm_stats(x32, eps) if stats is None else stats
    mu = np.asarray(mu, np.float32)
    rstd = np.asarray(rstd, np.float32)
    g = np.asarray(gamma, np.float32)[None, :]
    b = np.asarray(beta, np.float32)[None, :]
    t = (x32 - mu[:, None]).astype(np.float32)
    t = (t * rstd[:, None]).astype(np.float32)
    t = (t * g).astype(np.float32)
    return (t + b).astype(np.float32)


def _near_f32_boundary(v: float, err: float) -> bool:
    """True when [v - err, v + err] holds a point where rounding to fp32
    changes (a midpoint between two adjacent fp32 values)."""
    f = np.float32(v)
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    mid_lo = (float(lo) + float(f)) / 2.0
    mid_hi = (float(f) + float(hi)) / 2.0
    return abs(v - mid_lo) <= err or abs(v - mid_hi) <= err


def sum_exact_in_any_order(row) -> bool:
    """True when every double sum of the row's values, in any order, is exact:
    all values are integer multiples of 2^q (q the exponent of the lowest set
    bit over the row) and sum|values| stays below 2^(52 + q), so every partial
    sum fits a 53-bit significand.  Holds for 16-bit inputs (fp16, bf16) of
    ordinary range at the hidden sizes of the workloads."""
    v = np.asarray(row, np.float64)
    v = v[v != 0]
    if v.size == 0:
        return True
    mant, ex = np.frexp(np.abs(v))
    ints = (mant * 2.0 ** 53).astype(np.int64)  # exact: mant holds 53 bits
    low = ints & -ints  # lowest set bit of each significand
    q = int((ex - 53 + np.log2(low.astype(np.float64)).astype(np.int64)).min())
    return math.fsum(np.abs(v).tolist()) < math.ldexp(1.0, 52 + q)


def _stat_error_bounds(row: np.ndarray, eps: float):
    """(mu_d, rstd_d, e_mu, e_rstd, exact) for one row of exact float64 values.

    A double sum of K terms in any order is within K * 2^-53 * sum|terms| of
    the exact sum (zero when the sum is exact in any order,
    ``sum_exact_in_any_order``); the bounds carry that through mu_d, var_d and
    rstd_d with margin (a factor of 4) and add two double ulps for each
    correctly rounded operation."""
    K = row.shape[0]
    u = 2.0 ** -53
    mu_d, var_d, rstd_d = _row_stats(row, eps)
    # an exact sum makes mu_d the same correctly rounded quotient on both
    # sides, so fp32(mu_d) is then decided even on a midpoint
    exact = sum_exact_in_any_order(row)
    e_mu = 0.0 if exact else 4 * (u * float(np.abs(row).sum()) + 2 * u * abs(mu_d))
    d = np.abs(row - mu_d)
    e_var = 4 * (K * u * float((d * d).sum()) / K + 2 * e_mu * float(d.sum()) / K
                 + e_mu * e_mu + 2 * u * var_d)
    # rstd = (var + eps)^-1/2: relative error half that of var + eps
    e_rstd = 4 * (0.5 * e_var / (var_d + eps) * rstd_d + 4 * u * rstd_d)
    return mu_d, rstd_d, e_mu, e_rstd, exact


def ambiguous_rows(x, eps: float):
    """Rows whose fp32 mu or rstd may differ by one unit when the double sums
    are taken in another order (the error bounds of ``_stat_error_bounds``
    reach an fp32 rounding boundary)."""
    x = np.asarray(x, np.float32).astype(np.float64)
    out = []
    for m in range(x.shape[0]):
        mu_d, rstd_d, e_mu, e_rstd, exact = _stat_error_bounds(x[m], eps)
        if (not exact and _near_f32_boundary(mu_d, e_mu)) or _near_f32_boundary(rstd_d, e_rstd):
            out.append(m)
    return out


def _f32_candidates(v: float, err: float, limit: int = 64):
    """Every fp32 value that a double within err of v rounds to: rounding is
    monotone, so they are the values between fp32(v - err) and fp32(v + err).
    More than `limit` of them means the row is not a useful test case."""
    lo, hi = np.float32(v - err), np.float32(v + err)
    out = [lo]
    while out[-1] < hi:
        out.append(np.nextafter(out[-1], np.float32(np.inf)))
        if len(out) > limit:
            raise ValueError("statistic %r +- %r spans more than %d fp32 values" % (v, err, limit))
    return out


def admissible_stats(row, eps: float):
    """All (mu, rstd) fp32 pairs that a double summation of the row in some
    order may produce, within the bounds of ``_stat_error_bounds``; the first
    pair is the one ``layernorm_stats`` gives (the correctly rounded sums).
    A row that ``ambiguous_rows`` does not flag has exactly that one pair."""
    r = np.asarray(row, np.float32).astype(np.float64)
    mu_d, rstd_d, e_mu, e_rstd, _ = _stat_error_bounds(r, eps)
    first = (np.float32(mu_d), np.float32(rstd_d))
    pairs = [first]
    for mu in _f32_candidates(mu_d, e_mu):
        for rs in _f32_candidates(rstd_d, e_rstd):
            if (mu, rs) != first:
                pairs.append((mu, rs))
    return pairs


def store_dtype(y32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values rounded to the activation dtype (nearest even), widened
    back to fp32 exactly."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(y32, np.float32))
    if dtype == "f16":
        t = t.half()
    elif dtype == "bf16":
        t = t.bfloat16()
    return t.float().numpy()


def layernorm_quant_pertoken(x, gamma, beta, eps: float, dtype: str, stats=None):
    """(xq int8 [M x K], x_scale fp32 [M], x_hat [M x K] as stored in `dtype`,
    widened to fp32): LayerNorm with the folded (gamma, beta), stored in the
    activation dtype, then per-token quantisation of the stored values.
    ``stats`` = (mu, rstd) replaces the row statistics (see
    ``admissible_stats``)."""
    from . import quant_act_pertoken
    y = store_dtype(layernorm_f32(x, gamma, beta, eps, stats), dtype)
    xq, sx = quant_act_pertoken(y)
    return xq, sx, y


def row_alternatives(row, gamma, beta, eps: float, dtype: str):
    """The results (xq [K], x_scale, x_hat [K]) of one row under each of its
    admissible statistics (``admissible_stats``), the standard one first."""
    x = np.asarray(row, np.float32)[None, :]
    out = []
    for mu, rs in admissible_stats(row, eps):
        xq, sx, y = layernorm_quant_pertoken(x, gamma, beta, eps, dtype,
                                             (np.array([mu]), np.array([rs])))
        out.append((xq[0], sx[0], y[0]))
    return out
