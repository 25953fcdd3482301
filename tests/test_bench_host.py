"""Host-side checks of bench.py's JSON line: the unit conversions of the
headline record (ops and microseconds to TOP/s and fractions of the 5.0 POP/s
INT8 peak) and the guard that rejects a fraction above 1."""
import math

import pytest

import bench


def _hd(ms, gemm_us):
    M = 8192
    shapes = [(12288, 36864), (12288, 49152), (49152, 12288)]
    ops = sum(2.0 * M * n * k for k, n in shapes)
    return {"M": M, "ms": ms, "ops": ops, "per_launch_ops": ops / 3, "gemm_avg_us": gemm_us,
            "quant_avg_us": 100.0, "quant_bytes": 6.0e8, "runs": [ms] * 5, "layers": {}}


def test_headline_record_units():
    hd = _hd(11.438, 3700.5)
    out = bench.headline_record(hd, 20, 5)
    # 2*8192*(12288*36864 + 12288*49152 + 49152*12288) ops in 11.438 ms
    ops = 2 * 8192 * (12288 * 36864 + 12288 * 49152 + 49152 * 12288)
    assert math.isclose(out["value"], ops / 11.438e-3 / 1e12, rel_tol=1e-4)
    assert 2370 < out["value"] < 2390
    rl = out["roofline"]
    assert rl["unit"] == "TOP/s" and rl["peak"] == 5000.0
    assert math.isclose(rl["achieved"], ops / 3 / 3700.5e-6 / 1e12, rel_tol=1e-4)
    assert math.isclose(rl["frac"], rl["achieved"] / 5000.0, rel_tol=1e-3)
    assert 0.48 < rl["frac"] < 0.50
    assert math.isclose(out["config"]["frac_of_int8_peak"], out["value"] / 5000.0, rel_tol=1e-3)
    # 6e8 bytes in 100 us = 6000 GB/s = 0.75 of 8 TB/s
    assert math.isclose(out["act_quant"]["gbs"], 6000.0)
    assert math.isclose(out["act_quant"]["hbm_frac"], 0.75)
    bench.check_peak_fractions(out)


@pytest.mark.parametrize("bad", [{"roofline": {"bound": "mfma", "frac": 490.25}},
                                 {"x": {"gemm_frac_of_int8_peak": 381.04}},
                                 {"x": {"frac_of_int8_peak": 0.0}}])
def test_peak_fraction_guard(bad):
    with pytest.raises(RuntimeError):
        bench.check_peak_fractions(bad)


def test_peak_fraction_guard_ignores_hbm_fractions():
    # an HBM-bound figure may read above 1 when its operands sit in the
    # Infinity Cache; only MFMA-peak fractions are guarded
    bench.check_peak_fractions({"roofline": {"bound": "hbm", "frac": 1.2}, "hbm_frac": 1.1})
