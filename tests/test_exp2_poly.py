"""The software exp2's polynomial and its error bound (CPU only).

The kernels' polynomial exponential (exp2_poly in csrc/fa_device.h) splits
x = n + f, n = floor(x), evaluates the fitted polynomial at f with FMAs and
adds n to the exponent field. This test evaluates the same steps in float32
(FMA emulated exactly through float64) over a dense grid and compares with
numpy's exp2 in float64; the GPU path itself is exercised end to end by the
FA_EXP_POLY parity tests. Out-of-range inputs: x < -125 gives 0, x >= 128
gives +inf (2^128 is past the float32 range), and NaN stays NaN.
"""
import os
import re
import subprocess
import sys

import numpy as np

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "exact_attention_48_amd", "csrc")


def coeffs():
    text = open(os.path.join(CSRC, "exp2_poly_coeffs.h")).read()
    body = text[text.index("{") + 1:text.index("}")]
    c = [float(x.strip().rstrip("f")) for x in body.split(",") if x.strip()]
    deg = int(re.search(r"kExp2PolyDegree = (\d+)", text).group(1))
    bound = float(re.search(r"kExp2PolyRelErr = ([0-9.e+-]+)f", text).group(1))
    assert len(c) == deg + 1
    return np.array(c, dtype=np.float32), bound


def fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def exp2_poly_emulated(x):
    c, _ = coeffs()
    x = x.astype(np.float32)
    with np.errstate(invalid="ignore"):
        under = x < np.float32(-125.0)
        xc = np.where(under, np.float32(-125.0), x)          # a select: a NaN stays NaN
        n = np.floor(xc)
        f = (xc - n).astype(np.float32)
    p = np.full_like(f, c[-1])
    for ci in c[-2::-1]:
        p = fma32(p, f, np.full_like(f, ci))
    ni = np.where(np.isfinite(n), np.clip(n, -(2 ** 31), 2 ** 31 - 1), 0).astype(np.int64)
    ni = np.clip(ni, -1000, 1000).astype(np.int32)            # v_ldexp_f32 saturates the same way
    with np.errstate(over="ignore", invalid="ignore"):
        out = np.ldexp(p, ni).astype(np.float32)
        out = np.where(x >= np.float32(128.0), np.float32(np.inf), out)
    return np.where(under, np.float32(0.0), out)


def test_relative_error_within_fit_bound():
    c, bound = coeffs()
    x = np.linspace(-125.0, 8.0, 2_000_001, dtype=np.float32)
    got = exp2_poly_emulated(x).astype(np.float64)
    want = np.exp2(x.astype(np.float64))
    rel = np.max(np.abs(got / want - 1.0))
    assert rel <= bound + 2e-7, rel
    assert rel < 1e-4          # far below the bf16 rounding of P (2^-9)


def test_masked_and_tiny_inputs_give_zero():
    x = np.array([-np.inf, -1000.0, -127.0, -125.5], dtype=np.float32)
    assert np.all(exp2_poly_emulated(x) == 0.0)


def test_overflow_and_nan():
    """Inputs at and above 128 overflow to +inf, as 2^x does in float32; the largest
    finite results stay finite; NaN is passed through (so a non-finite row sum in
    the forward pass still triggers its re-run)."""
    x = np.array([127.0, 127.99, 128.0, 129.5, 140.0, 200.0, 520.0, np.inf, np.nan], dtype=np.float32)
    y = exp2_poly_emulated(x)
    assert np.all(np.isfinite(y[:2])) and y[0] == np.float32(2.0 ** 127) * np.float32(coeffs()[0][0])
    assert np.all(y[2:8] == np.inf), y
    assert np.isnan(y[8])
    grid = np.linspace(100.0, 600.0, 20001, dtype=np.float32)
    g = exp2_poly_emulated(grid)
    assert np.all(np.isfinite(g[grid < 128.0])) and np.all(g[grid >= 128.0] == np.inf)
    assert np.all(np.diff(g[grid < 128.0]) >= 0)


def test_integers_are_near_exact():
    x = np.arange(-125, 8, dtype=np.float32)
    rel = np.abs(exp2_poly_emulated(x).astype(np.float64) / np.exp2(x.astype(np.float64)) - 1)
    c, bound = coeffs()
    assert np.max(rel) <= bound + 1e-7


def test_header_is_reproducible():
    out = subprocess.run([sys.executable, os.path.join(CSRC, "gen_exp2_poly.py"), "3", "--dry-run"],
                         capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    c, _ = coeffs()
    fitted = np.array([float(v) for v in out.stdout.split()[-(len(c)):]], dtype=np.float32)
    assert np.array_equal(fitted, c)
