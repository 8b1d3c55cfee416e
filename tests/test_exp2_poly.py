"""The software exp2's polynomial and its error bound (CPU only).

The kernels' polynomial exponential (exp2_poly in csrc/fa_device.h) splits
x = n + f, n = floor(x), evaluates the fitted polynomial at f with FMAs and
adds n to the exponent field. This test evaluates the same steps in float32
(FMA emulated exactly through float64) over a dense grid and compares with
numpy's exp2 in float64; the GPU path itself is exercised end to end by the
FA_EXP_POLY parity tests.
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
    xc = np.maximum(x, np.float32(-125.0))
    n = np.floor(xc)
    f = (xc - n).astype(np.float32)
    p = np.full_like(f, c[-1])
    for ci in c[-2::-1]:
        p = fma32(p, f, np.full_like(f, ci))
    bits = p.view(np.int32) + (n.astype(np.int32) << 23)
    out = bits.view(np.float32)
    return np.where(x < -125.0, np.float32(0.0), out)


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
