"""The step kernel's binary32 tanh polynomial (CPU only).

The soft cap's transform is cap * tanh(z). Plans without the transform table
evaluate tanh in the kernel: below |z| = 0.625 an odd polynomial z + z^3
p(z^2) with p of degree 5 in binary32 Horner form (coefficients: the Taylor
series' odd terms through z^13, each adjusted by a fit to tanh on that
interval and rounded to binary32). Its error bound is checked here, on what
the kernel computes (coefficients read from its source, every operation in
binary32 with fused multiply-adds):
* every binary32 z in [2^-8, 0.625] and every 97th one below, against tanh
  in binary64 (``tests/tanh_poly.c``): at most 0.73 binary32 ulp;
* the worst case found, again in 50-digit arithmetic (mpmath), so that the
  binary64 reference cannot have hidden an error;
* the coefficients stay near the Taylor series (the fit only adjusts them).
"""

import ctypes
import os
import re
import subprocess
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL = os.path.join(os.path.dirname(HERE), "markov_draft_sampling_step_amd", "csrc", "step_kernel.h")
BOUND_ULP = 0.73


def kernel_coefficients():
    src = open(KERNEL).read()
    body = src[src.index("float tanh_poly(float z)"):]
    body = body[: body.index("\n}\n")]
    hexes = re.findall(r"(-?0x[0-9a-f.]+p-?\d+)f", body)
    assert len(hexes) == 6, hexes
    return [float.fromhex(h) for h in hexes]


def rn32(q: Fraction) -> np.float32:
    """q rounded to binary32, nearest with ties to even (normal range)."""
    if q == 0:
        return np.float32(0.0)
    sign, q = (-1, -q) if q < 0 else (1, q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    scaled = q / Fraction(2) ** (e - 23)             # in [2^23, 2^24)
    m, r = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * r
    if twice > scaled.denominator or (twice == scaled.denominator and m % 2 == 1):
        m += 1
    return np.float32(sign * float(Fraction(m) * Fraction(2) ** (e - 23)))


def eval32(c, z):
    """The kernel's evaluation in binary32: each product and fused
    multiply-add rounded once from its exact value."""
    def fma(a, b, d):
        return rn32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(d)))
    z = np.float32(z)
    t = rn32(Fraction(float(z)) ** 2)
    p = np.float32(c[0])
    for ci in c[1:]:
        p = fma(p, t, np.float32(ci))
    return fma(rn32(Fraction(float(t)) * Fraction(float(z))), p, z)


@pytest.fixture(scope="module")
def sweep_lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("tanh") / "libtanhpoly.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", out,
                           os.path.join(HERE, "tanh_poly.c"), "-lm"])
    lib = ctypes.CDLL(out)
    lib.sweep_tanh_poly.restype = ctypes.c_double
    lib.sweep_tanh_poly.argtypes = [ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_uint32)]
    return lib


def test_rn32():
    for x in (1.0, 1 / 3, 0.1, 1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, -0.7, 6e-39 * 1e6):
        assert rn32(Fraction(x)) == np.float32(x)
    assert rn32(Fraction(1) + Fraction(1, 2 ** 24)) == np.float32(1.0)            # tie to even
    assert rn32(Fraction(1) + Fraction(3, 2 ** 25)) == np.float32(1 + 2.0 ** -23)


def test_coefficients_near_taylor():
    c = kernel_coefficients()[::-1]            # lowest order first: z^3 .. z^13
    taylor = [-1 / 3, 2 / 15, -17 / 315, 62 / 2835, -1382 / 155925, 21844 / 6081075]
    for i, (ci, ti) in enumerate(zip(c, taylor)):
        assert np.sign(ci) == np.sign(ti)
        # the fit moves the low terms by parts per million, the last ones more
        assert abs(ci - ti) <= (1e-6, 1e-4, 1e-2, 2e-2, 0.1, 0.5)[i] * abs(ti), (i, ci, ti)


def test_error_bound(sweep_lib):
    c = np.array(kernel_coefficients(), dtype=np.float32)
    at = ctypes.c_uint32()
    worst = sweep_lib.sweep_tanh_poly(c.ctypes.data, 0.625, 2.0 ** -8, 97, ctypes.byref(at))
    z = float(np.array([at.value], dtype=np.uint32).view(np.float32)[0])
    print(f"tanh polynomial: worst {worst:.4f} ulp at z = {z!r}")
    assert worst <= BOUND_ULP, (worst, z)

    # the worst case in 50-digit arithmetic
    import mpmath
    mpmath.mp.dps = 50
    y = eval32(c, z)
    ref = mpmath.tanh(mpmath.mpf(z))
    e = int(mpmath.floor(mpmath.log(abs(ref), 2)))
    err = abs(mpmath.mpf(float(y)) - ref) / mpmath.mpf(2) ** (e - 23)
    assert abs(float(err) - worst) < 1e-6, (float(err), worst)


def test_worst_region_in_50_digits():
    """A few hundred points around the interval's end and middle, directly
    against mpmath (no binary64 reference involved)."""
    import mpmath
    mpmath.mp.dps = 50
    c = np.array(kernel_coefficients(), dtype=np.float32)
    zs = np.concatenate([np.linspace(0.5, 0.625, 200, dtype=np.float32),
                         np.linspace(1e-3, 0.5, 100, dtype=np.float32)])
    for z in zs:
        y = eval32(c, float(z))
        ref = mpmath.tanh(mpmath.mpf(float(z)))
        e = int(mpmath.floor(mpmath.log(abs(ref), 2)))
        err = abs(mpmath.mpf(float(y)) - ref) / mpmath.mpf(2) ** (e - 23)
        assert float(err) <= BOUND_ULP, (float(z), float(err))
