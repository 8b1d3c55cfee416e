"""The kernels' exponential on the GPU, through the C ABI (fa_exp2_eval).

FA_EXP_POLY: the device polynomial must agree with the host emulation of the
same steps (tests/test_exp2_poly.py: exact split x = n + f, the fitted
coefficients by FMA, n added to the exponent field) to within one unit in the
last place everywhere, and exactly on almost every input (the host emulates
each fused multiply-add in float64, which can differ from a single rounding in
rare double-rounding cases), and stay within the fit's error bound of float64
2^x. FA_EXP_HW: the error of the hardware v_exp_f32 is measured here against
float64 2^x over the normal range, not assumed.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from exact_attention_48_amd import capi  # noqa: E402
from tests.test_exp2_poly import coeffs, exp2_poly_emulated  # noqa: E402


def sample():
    rng = np.random.default_rng(2024)
    grid = rng.uniform(-127.0, 0.0, size=1 << 20).astype(np.float32)
    ints = np.arange(-130, 1, dtype=np.float32)
    near_ints = np.concatenate([ints + np.float32(2.0 ** -20), ints - np.float32(2.0 ** -20)])
    tiny = np.float32(-1.0) * np.logspace(-30, 0, 4096, dtype=np.float64).astype(np.float32)
    special = np.array([0.0, -0.0, -np.inf, -125.0, -125.5, -126.0, -127.0, -1000.0, 1.0, 7.5, 127.0, 127.99,
                        128.0, 140.0, 200.0, 520.0, np.inf], dtype=np.float32)
    high = rng.uniform(100.0, 600.0, size=1 << 14).astype(np.float32)     # up to and past overflow
    return np.concatenate([grid, ints, near_ints, tiny, special, high]).astype(np.float32)


def run(x, mode):
    dev = torch.from_numpy(x).to("cuda:0")
    out = torch.empty_like(dev)
    capi.fa_exp2_eval(dev, out, x.size, mode)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def ulp_diff(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def test_polynomial_matches_host_emulation():
    x = sample()
    got = run(x, capi.FA_EXP_POLY)
    want = exp2_poly_emulated(x)
    assert np.all(got[x >= 128.0] == np.inf), "2^x for x >= 128 must overflow to +inf"
    nan_in = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(np.isnan(run(nan_in, capi.FA_EXP_POLY))), "NaN must stay NaN"
    d = ulp_diff(got, want)
    assert np.max(d) <= 1, (np.max(d), x[np.argmax(d)])
    exact = np.mean(d == 0)
    assert exact >= 0.999, exact
    _, bound = coeffs()
    ok = (x >= -125.0) & (x < 127.0)
    ref = np.exp2(x[ok].astype(np.float64))
    rel = np.max(np.abs(got[ok].astype(np.float64) / ref - 1.0))
    assert rel <= bound + 2.5e-7, rel
    assert np.all(got[x < -125.0] == 0.0)


def test_hardware_exp_error_measured():
    x = sample()
    got = run(x, capi.FA_EXP_HW)
    normal = (x >= -126.0) & (x < 127.0)
    ref = np.exp2(x[normal].astype(np.float64))
    rel = np.abs(got[normal].astype(np.float64) / ref - 1.0)
    worst = float(np.max(rel))
    print(f"v_exp_f32 max relative error over x in [-126, 0]: {worst:.3e} ({worst / 2.0 ** -24:.2f} x 2^-24)")
    assert worst <= 2.0 ** -21, worst               # a few ulp: far below the bf16 rounding of P (2^-9)
    assert got[x == -np.inf][0] == 0.0
    assert got[x == 0.0][0] == 1.0
    assert np.all(got[x >= 128.0] == np.inf)
