"""The 16-bit-output GELU (gelu16 in device_common.hpp), evaluated in float32 on the
host with the constants as the header states them, against the exact definition
GELU(v) = v Phi(v) (Phi from scipy's erf / erfc): the accuracy its comment claims,
and the special values. Host logic only; the device code runs in the GPU parity
tests through the FFN and epilogue cases."""
import os
import re

import numpy as np
import pytest
from scipy.special import erf, erfc

HDR = os.path.join(os.path.dirname(__file__), "..", "dense_gemm_15_amd", "csrc", "device_common.hpp")


def _body():
    src = open(HDR).read()
    return src[src.index("float gelu16(float v)"):].split("\n}\n")[0]


def _consts():
    b = _body()
    p0 = float(re.search(r"float p = ([-0-9.e]+)f;", b).group(1))
    rest = [float(x) for x in re.findall(r"p = __builtin_fmaf\(p, s, ([-0-9.e]+)f\);", b)]
    k = float(re.search(r"v \* ([-0-9.e]+)f, p\)", b).group(1))
    r2 = float(re.search(r"fmaf\(av, ([-0-9.e]+)f, 2.0f\)", b).group(1))
    cap = float(re.search(r"av \* s, ([-0-9.e]+)f\)", b).group(1))
    return [p0] + rest, k, r2, cap


def gelu16_host(v):
    coef, k, r2, cap = _consts()
    f = np.float32
    v = np.asarray(v, f)
    av = np.abs(v)
    with np.errstate(all="ignore"):
        s = (f(1) / (av * f(r2) + f(2))).astype(f)
        p = f(coef[0])
        for c in coef[1:]:
            p = (p * s + f(c)).astype(f)
        e = np.exp2((v * (v * f(k)).astype(f) + p).astype(f).astype(np.float64)).astype(f)
        q = np.fmin(av * s, f(cap)).astype(f)  # the device min returns the non-NaN operand
        return (np.fmax(v, f(0)) - q * e).astype(f)


def gelu_exact(v):
    v = np.asarray(v, np.float64)
    out = 0.5 * v * (1 + erf(v / np.sqrt(2)))
    neg = v < 0
    out[neg] = 0.5 * v[neg] * erfc(-v[neg] / np.sqrt(2))  # no cancellation in the tail
    return out


def test_gelu16_constants_present():
    coef, k, r2, cap = _consts()
    assert len(coef) == 6  # degree 5
    assert k == pytest.approx(-0.5 / np.log(2), rel=1e-7)
    assert r2 == pytest.approx(1 / np.sqrt(2), rel=1e-7)
    assert cap == pytest.approx(np.sqrt(2), rel=1e-7)


def test_gelu16_accuracy():
    v = np.concatenate([np.linspace(-12, 12, 400001), -np.logspace(-8, 1.2, 5001),
                        np.logspace(-8, 1.2, 5001)]).astype(np.float32)
    want = gelu_exact(v.astype(np.float64))
    got = gelu16_host(v).astype(np.float64)
    err = np.abs(got - want)
    assert np.max(err / np.maximum(np.abs(v), 1e-30)) < 3e-5  # absolute, relative to |v|
    m = np.abs(want) > 1e-30
    assert np.max(err[m] / np.abs(want[m])) < 1e-4  # relative, negative tail included
    # small against the 16-bit rounding step of the result (bf16: 2^-8 relative)
    assert np.max(err[m] / np.abs(want[m])) < 2.0 ** -8 / 30


def test_gelu16_special_values():
    got = gelu16_host(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 40.0, -40.0], np.float32))
    assert got[0] == 0 and got[1] == 0
    assert got[2] == np.inf and got[3] == 0
    assert np.isnan(got[4])
    assert got[5] == 40.0 and abs(got[6]) < 1e-30
