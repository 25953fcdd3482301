"""CPU replay of the library's quantiser arithmetic against the oracle.

The kernels form each code as round(RN(v / step)) through Markstein's
correction from RN(1 / step) (normal-range steps), with v first saturated to
+-128 steps wherever the step is fixed in advance (the static per-tensor
step of P1 推論方法 O3, where values past the calibrated range must clamp to
+-127).  ``tests/host/quant_host.cpp`` builds the library's own helpers from
``sq_device.h`` for the host; these tests compare their codes with the
oracle's IEEE quotient (``oracle/sqref.c``), including quotients that
overflow fp32 -- the case where an unsaturated correction yields NaN and the
clamp then returns -127 for positive values.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import hostbuild


def host_codes(v, steps, sat):
    v = np.ascontiguousarray(v, np.float32)
    steps = np.ascontiguousarray(np.broadcast_to(np.float32(steps), v.shape), np.float32)
    out = np.empty(v.shape, np.int8)
    hostbuild.load().hq_codes(v.ctypes.data, steps.ctypes.data, v.size, int(sat), out.ctypes.data)
    return out


def oracle_codes(v, step):
    """The oracle's codes for the values v with one given step."""
    q, _ = oracle.quant_act_pertensor(np.asarray(v, np.float32).reshape(1, -1), np.float32(step))
    return q.ravel()


# (step, |v|) where |v| * RN(1/step) overflows fp32 although step is in the
# fast range [2^-96, 2^96]
OVERFLOW_CASES = [(2.0 ** -96, 1e10), (1e-20, 1e19), (0.05, 3e37), (1.0, 3.4e38),
                  (2.0 ** 96, 3.4e38), (1e-3, 3.4028235e38)]


@pytest.mark.parametrize("step,mag", OVERFLOW_CASES)
def test_static_step_overflow_keeps_sign(step, mag):
    v = np.array([mag, -mag], np.float32)
    assert list(oracle_codes(v, step)) == [127, -127]
    assert list(host_codes(v, step, sat=True)) == [127, -127]


def test_unsaturated_form_is_wrong_past_overflow():
    # documents why the static callers saturate: without it the positive value
    # of an overflowing quotient gets -127
    v = np.array([1e10], np.float32)
    assert host_codes(v, 2.0 ** -96, sat=False)[0] == -127


def _step_grid(rng, n):
    """Steps spread log-uniformly over and beyond the fast range, plus the
    range's edges and steps with all-ones / power-of-two significands."""
    e = rng.uniform(-110, 110, n)
    st = (2.0 ** e).astype(np.float32)
    edges = np.array([2.0 ** -96, 2.0 ** 96, np.nextafter(np.float32(2.0 ** -96), 0),
                      np.nextafter(np.float32(2.0 ** 96), np.float32(np.inf)), 1.0, 0.5,
                      np.float32(1.9999999) * 2.0 ** -40, 1e-30, 1e30], np.float32)
    return np.concatenate([edges, st])


def test_static_step_codes_match_oracle_everywhere():
    """Random values at quotients from 0 to far past fp32 overflow, ties
    included, both signs, for steps across and beyond the fast range."""
    rng = np.random.default_rng([2025, 3])
    steps = _step_grid(rng, 300)
    for st in steps:
        st = np.float32(st)
        q = np.concatenate([
            rng.uniform(-130, 130, 400),                     # inside and just past the range
            np.arange(-128, 129) + 0.5,                      # ties of the code rounding
            np.sign(rng.standard_normal(200)) * 10.0 ** rng.uniform(2, 45, 200),  # far past
        ])
        with np.errstate(over="ignore"):
            v = (q * np.float64(st)).astype(np.float32)
        v = v[np.isfinite(v)]  # non-finite inputs are outside the contract
        v = np.concatenate([v, np.array([np.finfo(np.float32).max, -np.finfo(np.float32).max,
                                         np.finfo(np.float32).tiny, 0.0, -0.0], np.float32)])
        np.testing.assert_array_equal(host_codes(v, st, sat=True), oracle_codes(v, st),
                                      err_msg="step %r" % float(st))


def test_row_step_codes_match_oracle():
    """The dynamic (per-token) form: the step is the row's absmax / 127, so
    |v| <= 127 steps and no saturation is needed; codes equal the oracle's
    per-token quantiser for rows across the fp32 exponent range."""
    rng = np.random.default_rng([2025, 4])
    for e in list(range(-120, 121, 7)) + [-126, 124]:
        x = (rng.standard_normal((8, 257)) * 2.0 ** e).astype(np.float32)
        x[0, :3] = [np.float32(2.0 ** e * 62.5 / 127), 0.0, -0.0]
        xq_r, sx_r = oracle.quant_act_pertoken(x)
        for m in range(x.shape[0]):
            st = hostbuild.load().hq_row_step(float(np.abs(x[m]).max()))
            assert np.float32(st) == sx_r[m]
            np.testing.assert_array_equal(host_codes(x[m], st, sat=False), xq_r[m])
            np.testing.assert_array_equal(host_codes(x[m], st, sat=True), xq_r[m])


def test_code_rounding_every_fp32():
    """The kernels' rounding of a quotient to a code (one addition of
    copysign(0.5 - 2^-25, t) and the truncating conversion, then the clamp)
    against its definition, roundf clamped to +-127, for all 2^32 fp32 bit
    patterns (ties, the value just below 0.5, infinities and NaN included)."""
    from concurrent.futures import ThreadPoolExecutor

    lib = hostbuild.load()
    chunks = [(i << 28, (i + 1) << 28) for i in range(16)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        bad = list(ex.map(lambda c: lib.hq_rounding_mismatches(c[0], c[1]), chunks))
    assert sum(bad) == 0, bad
