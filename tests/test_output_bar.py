"""The layer-output bar of the parity tests (hmoe_testlib.check_output) checked on
the CPU: the exact result rounded to the bf16 output passes it with no excess even
where the rounding alone is larger than 2e-2 RMS, and planted errors of the sizes the
bar forbids fail it."""
import numpy as np
import pytest

from oracle import formats as F
from hmoe_testlib import bf16_half_ulp, check_output


def _ref(n=200_000, seed=0):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal(n) * 2.68
    y[:50] = rng.choice([-1.0, 1.0], 50) * rng.uniform(16.0, 31.0, 50)   # |y| >= 6 RMS
    return y


def test_half_ulp_matches_bf16_spacing():
    v = np.array([1.0, 1.5, 2.0, 3.99, 16.0, 31.0, -0.75, 2.0 ** -20])
    bits = F.bf16_bits(v.astype(np.float32))
    nxt = F.bf16_value(bits + 1).astype(np.float64)
    assert np.array_equal(bf16_half_ulp(v), (np.abs(nxt) - np.abs(F.bf16_value(bits))) / 2)


def test_rounded_exact_result_passes():
    y = _ref()
    bits = F.bf16_bits(y.astype(np.float32))
    raw = np.abs(F.bf16_value(bits) - y).max() / np.sqrt(np.mean(y ** 2))
    assert raw > 2e-2                     # the format alone exceeds the raw bar here
    s = check_output(bits, y, "exact")
    # fp64 -> fp32 -> bf16 rounds twice: the excess is at most an fp32 ulp
    assert s["max_err_rel"] < 1e-6 and s["frac_gt_1e-2"] == 0.0


def test_one_large_error_fails():
    y = _ref()
    z = y.copy()
    z[1000] += 0.03 * np.sqrt(np.mean(y ** 2))
    with pytest.raises(AssertionError):
        check_output(F.bf16_bits(z.astype(np.float32)), y, "planted max")


def test_many_moderate_errors_fail():
    y = _ref()
    rms = np.sqrt(np.mean(y ** 2))
    z = y.copy()
    idx = np.random.default_rng(1).choice(y.size, int(0.002 * y.size), replace=False)
    z[idx] += 0.015 * rms                 # below the max bar, above the 1e-2 one
    with pytest.raises(AssertionError):
        check_output(F.bf16_bits(z.astype(np.float32)), y, "planted frac")
