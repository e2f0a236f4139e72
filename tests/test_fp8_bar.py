"""The FP8 parity bar of the GPU tests, exercised on the CPU with codes the oracle makes.

A GPU code passes when it is the correct rounding of some value within the fp32 error bound
(delta) of the exact value.  Here the bar must accept codes of values perturbed by less than
delta, and reject the codes of plausible encoder mistakes: rounding toward zero instead of to
nearest, and a scale divisor other than 448.  (Ties to even are pinned bit for bit by the
codec sweep against the device encoder, where midpoints are hit exactly.)"""
import numpy as np
import pytest

import oracle
from gpu_cases import check_fp8_rows, e4m3_halfstep


def _rows(seed, R=64, D=128):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, D)) * 1.3
    x[:, :4] *= 1e-3                    # values near zero, in the subnormal range of the code
    return x


def test_bar_accepts_codes_of_values_within_delta():
    x = _rows(1)
    codes, scales, _ = oracle.fp8_quantize_rows(x)
    delta = np.full_like(x, 2e-5)
    rng = np.random.default_rng(2)
    noisy = x + rng.uniform(-1, 1, x.shape) * delta
    # the same per-row scales (an amax moved by delta changes the scale by ~1e-5 relative)
    ncodes = oracle.e4m3_encode(noisy / scales.astype(np.float64)[:, None])
    far = check_fp8_rows(ncodes, scales, x, codes, delta)
    # delta is about one subnormal step of these rows: near zero a code may move by more than
    # one step and still be a correct rounding; everywhere else at most one
    near_zero = np.abs(x / scales.astype(np.float64)[:, None]) < 2.0 ** -6
    assert far <= int(near_zero.sum())


def test_bar_rejects_rounding_toward_zero():
    x = _rows(3)
    codes, scales, _ = oracle.fp8_quantize_rows(x)
    s = scales.astype(np.float64)[:, None]
    y = x / s
    # truncation: the code of a value moved toward zero by just under half a step
    trunc = oracle.e4m3_encode(y - np.sign(y) * e4m3_halfstep(np.abs(y)) * 0.999)
    with pytest.raises(AssertionError, match="off by more than the bound"):
        check_fp8_rows(trunc, scales, x, codes, np.full_like(x, 1e-7))


def test_bar_rejects_a_wrong_scale_divisor():
    x = _rows(4)
    codes, scales, _ = oracle.fp8_quantize_rows(x)
    wrong = (np.abs(x).max(axis=1) / 480.0).astype(np.float32)
    wcodes = oracle.e4m3_encode(x / wrong.astype(np.float64)[:, None])
    # decoded with the scale the kernel would have stored next to them (448): off by 7%
    with pytest.raises(AssertionError, match="off by more than the bound"):
        check_fp8_rows(wcodes, scales, x, codes, np.full_like(x, 1e-7))
