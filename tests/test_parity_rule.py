"""The parity rule of the GPU tests (tests/gpu_util.close) on planted errors, on the CPU:
it accepts what a correct kernel produces (the oracle's bf16 values, or f32 values a few
f32 ulps away) and refuses a uniform relative error of 1 %, one element off by 10 %, and
a row of the f32 state off by a few percent."""
import numpy as np
import pytest

from oracle import gdn as og
from tests import gpu_util as gu


def _f32(seed, n=20000):
    return np.random.default_rng(seed).normal(0, 0.1, n).astype(np.float32)


def test_accepts_f32_rounding_noise_and_equal_bf16():
    r = _f32(0)
    g = (r.astype(np.float64) * (1 + np.random.default_rng(1).normal(0, 2e-7, r.size))).astype(np.float32)
    gu.close("f32 noise", g, r, bf16=False)
    b = og.f64_to_bf16(r.astype(np.float64) * 30)
    gu.close("bf16 equal", b, b)


@pytest.mark.parametrize("bf16", [True, False])
def test_refuses_a_uniform_one_percent_error(bf16):
    r = _f32(2).astype(np.float64)
    if bf16:
        ref, got = og.f64_to_bf16(r * 30), og.f64_to_bf16(r * 30 * 1.01)
    else:
        ref, got = r.astype(np.float32), (r * 1.01).astype(np.float32)
    with pytest.raises(AssertionError):
        gu.close("uniform 1%", got, ref, bf16=bf16)


@pytest.mark.parametrize("bf16", [True, False])
def test_refuses_one_element_off_by_ten_percent(bf16):
    r = _f32(3).astype(np.float64)
    g = r.copy()
    i = int(np.argmax(np.abs(r)))
    g[i] *= 1.1
    if bf16:
        ref, got = og.f64_to_bf16(r * 30), og.f64_to_bf16(g * 30)
    else:
        ref, got = r.astype(np.float32), g.astype(np.float32)
    with pytest.raises(AssertionError):
        gu.close("one element", got, ref, bf16=bf16)


def test_refuses_a_state_row_off_by_three_percent():
    r = _f32(4, 128 * 160).reshape(-1, 128).astype(np.float64)
    g = r.copy()
    g[7] *= 1.03
    with pytest.raises(AssertionError):
        gu.close("one row", g.astype(np.float32), r.astype(np.float32), bf16=False)
