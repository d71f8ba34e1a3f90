"""fp64 host oracle for the tiled dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package. The HIP library never calls it, and it never
calls the HIP library: the two share nothing but the seeded inputs of
``synth``.

``gemm_oracle.c`` computes the plain definition C = epi(A x B) in double
(see its header for the passages it follows); this module loads it with
ctypes and adds the element-wise acceptance test:

* reference ``ref`` = exact epilogue of the fp64 sum (unrounded);
* ``s`` = sum_k |a_ik b_kj|;
* tolerance ``tol = c * (1e-4 * |scale| * s + 1e-6)`` with ``c = 1.12891``
  (the supremum of GELU's slope, reached at x = sqrt 2, rounded up) when GELU is on,
  else ``c = 1``; for a 16-bit output, plus half a 16-bit ulp of
  ``|ref| + tol`` (the output itself is rounded once);
* pass iff ``|C - ref| <= tol`` everywhere (NaN fails); for the fp32 SGEMM
  workload additionally ``max |C - ref| <= 1e-3`` (the SGEMM page, section
  4.1, accepts an absolute error within 1e-3);
* exact mode (small-integer inputs): every element equals ``ref`` (fp32 out)
  or ``RNE16(ref)`` (16-bit out) by value.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2
DTYPE_CODE = {"f32": F32, "f16": F16, "bf16": BF16}
BIAS, GELU, RESID, SCALE = 1, 2, 4, 8
# max over x of GELU'(x) = Phi(x) + x phi(x); the maximum is at x = sqrt 2, where it is
# Phi(sqrt 2) + sqrt 2 phi(sqrt 2) = 1.1289041..., rounded up here.
GELU_SLOPE_SUP = 1.12891


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with plain gcc + OpenMP (no HIP headers)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building if needed) the oracle library; returns the ctypes handle."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB
    if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(SRC)):
        build(SRC, p)
    lib = ctypes.CDLL(p)
    i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
    lib.oracle_decode.argtypes = [i32, vp, i64, vp]
    lib.oracle_round16.argtypes = [i32, vp, i64, vp]
    lib.oracle_ulp16.argtypes = [i32, dp]
    lib.oracle_ulp16.restype = dp
    lib.oracle_ulp16_n.argtypes = [i32, vp, i64, vp]
    lib.oracle_gelu.argtypes = [dp]
    lib.oracle_gelu.restype = dp
    lib.oracle_gemm.argtypes = [i64, i64, i64, i32, vp, vp, ctypes.c_uint, dp, vp, i32, vp, vp,
                                vp, i32]
    lib.oracle_gemm_at.argtypes = [i64, i64, i64, i32, vp, vp, ctypes.c_uint, dp, vp, i32, vp,
                                   i64, vp, vp, vp, vp]
    lib.oracle_gemm_f16acc.argtypes = [i64, i64, i64, vp, vp, vp]
    lib.oracle_softmax_rows.argtypes = [i64, i64, vp, i64, dp, vp]
    lib.oracle_threads.restype = i32
    if path is None:
        _lib = lib
    return lib


def _code(dtype) -> int:
    return DTYPE_CODE[dtype] if isinstance(dtype, str) else int(dtype)


def _buf(x, dtype):
    """Contiguous numpy buffer of raw element bits for dtype."""
    code = _code(dtype)
    want = np.float32 if code == F32 else np.uint16
    a = np.ascontiguousarray(x)
    if a.dtype != want:
        raise TypeError(f"expected {want.__name__} bits for dtype {dtype}, got {a.dtype}")
    return a


def decode(dtype, x, lib=None) -> np.ndarray:
    lib = lib or load()
    a = _buf(x, dtype)
    out = np.empty(a.shape, np.float64)
    rc = lib.oracle_decode(_code(dtype), a.ctypes.data, a.size, out.ctypes.data)
    assert rc == 0
    return out


def round16(dtype, x, lib=None) -> np.ndarray:
    """RNE of doubles to bf16/fp16; returns uint16 bit patterns."""
    lib = lib or load()
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    rc = lib.oracle_round16(_code(dtype), a.ctypes.data, a.size, out.ctypes.data)
    assert rc == 0
    return out


def ulp16(dtype, x, lib=None) -> np.ndarray:
    lib = lib or load()
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.float64)
    rc = lib.oracle_ulp16_n(_code(dtype), a.ctypes.data, a.size, out.ctypes.data)
    assert rc == 0
    return out


def gelu(v: float, lib=None) -> float:
    return (lib or load()).oracle_gelu(float(v))


def threads(lib=None) -> int:
    return (lib or load()).oracle_threads()


def gemm(A, B, dtype, flags: int = 0, scale: float = 1.0, bias=None, resid=None,
         resid_dtype="f32", nthreads: int = 0, lib=None):
    """Full fp64 product. A: [M,K] bits, B: [K,N] bits. Returns (ref, s), both [M,N] float64."""
    lib = lib or load()
    A = _buf(A, dtype)
    B = _buf(B, dtype)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2, "inner dimensions differ"
    bias_p = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (N,)
        bias_p = bias.ctypes.data
    resid_p = None
    if resid is not None:
        resid = _buf(resid, resid_dtype)
        assert resid.shape == (M, N)
        resid_p = resid.ctypes.data
    ref = np.empty((M, N), np.float64)
    s = np.empty((M, N), np.float64)
    rc = lib.oracle_gemm(M, N, K, _code(dtype), A.ctypes.data, B.ctypes.data, flags, scale,
                         bias_p, _code(resid_dtype), resid_p, ref.ctypes.data, s.ctypes.data,
                         nthreads)
    if rc != 0:
        raise ValueError(f"oracle_gemm rejected its arguments (code {rc})")
    return ref, s


def gemm_f16acc(A, B, lib=None):
    """fp16 A [M,K], B [K,N] (bit patterns) with every accumulator held in fp16:
    one round-to-nearest-even per k of acc + a*b (DeepGEMM page, section 3.4's
    FP16-accumulation variant). Exact for inputs on the 2^-10 grid in [-1, 1].
    Returns [M,N] float64 (fp16 values)."""
    lib = lib or load()
    A = _buf(A, "f16")
    B = _buf(B, "f16")
    M, K = A.shape
    K2, N = B.shape
    assert K == K2, "inner dimensions differ"
    ref = np.empty((M, N), np.float64)
    rc = lib.oracle_gemm_f16acc(M, N, K, A.ctypes.data, B.ctypes.data, ref.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_gemm_f16acc rejected its arguments (code {rc})")
    return ref


def softmax_rows(S, scale: float = 1.0, lib=None):
    """Row softmax of scale * S in double; S a 2-D float32 array. Returns float64."""
    lib = lib or load()
    S = np.ascontiguousarray(S, dtype=np.float32)
    rows, cols = S.shape
    ref = np.empty((rows, cols), np.float64)
    rc = lib.oracle_softmax_rows(rows, cols, S.ctypes.data, cols, float(scale), ref.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_softmax_rows rejected its arguments (code {rc})")
    return ref


def softmax_tolerance(S, ref, scale: float = 1.0, out_dtype: str = "f32", lib=None):
    """Element-wise bound for an fp32 softmax against the double reference: the
    exponent's argument carries ~2^-24 |scale x| of rounding and exp, the row sum and
    the division a few fp32 ulps, so |P - p| <= p (4e-6 + 2^-22 max_c |scale S|) per
    row; a 16-bit output adds half a 16-bit ulp of the (rounded-once) value."""
    R = np.abs(float(scale) * np.asarray(S, np.float64)).max(axis=1, keepdims=True)
    tol = ref * (4e-6 + 2.0 ** -22 * R)
    if out_dtype != "f32":
        tol = tol + 0.5 * ulp16(out_dtype, np.abs(ref) + tol, lib=lib)
    return tol


def gemm_at(A, B, dtype, rows, cols, flags: int = 0, scale: float = 1.0, bias=None, resid=None,
            resid_dtype="f32", lib=None):
    """Selected elements (rows[t], cols[t]) of the same product: (ref, s), 1-D float64."""
    lib = lib or load()
    A = _buf(A, dtype)
    B = _buf(B, dtype)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.shape == cols.shape
    bias_p = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        bias_p = bias.ctypes.data
    resid_p = None
    if resid is not None:
        resid = _buf(resid, resid_dtype)
        resid_p = resid.ctypes.data
    ref = np.empty(rows.shape, np.float64)
    s = np.empty(rows.shape, np.float64)
    rc = lib.oracle_gemm_at(M, N, K, _code(dtype), A.ctypes.data, B.ctypes.data, flags, scale,
                            bias_p, _code(resid_dtype), resid_p, rows.size, rows.ctypes.data,
                            cols.ctypes.data, ref.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_gemm_at rejected its arguments (code {rc})")
    return ref, s


def tolerance(ref, s, out_dtype="f32", flags: int = 0, scale: float = 1.0, lib=None):
    """Per-element acceptance bound for a result against (ref, s)."""
    c = GELU_SLOPE_SUP if flags & GELU else 1.0
    alpha = abs(scale) if flags & SCALE else 1.0
    tol = c * (1e-4 * alpha * np.asarray(s, np.float64) + 1e-6)
    if _code(out_dtype) != F32:
        tol = tol + 0.5 * ulp16(out_dtype, np.abs(ref) + tol, lib=lib)
    return tol


def check(C, ref, s, out_dtype="f32", flags: int = 0, scale: float = 1.0, abs_max=None,
          exact: bool = False, lib=None) -> dict:
    """Compare a result (raw bits of out_dtype) against the oracle.

    Returns a dict with ``ok``, ``max_ratio`` (max |err|/tol), ``argmax`` (flat
    index), ``max_abs`` (max |err|), ``n_bad`` and ``n``."""
    lib = lib or load()
    Cd = decode(out_dtype, np.asarray(C).reshape(np.shape(ref)), lib=lib)
    ref = np.asarray(ref, np.float64)
    err = np.abs(Cd - ref)
    nan = ~np.isfinite(Cd)
    if exact:
        want = ref if _code(out_dtype) == F32 else decode(out_dtype, round16(out_dtype, ref, lib),
                                                          lib=lib)
        bad = (Cd != want) | nan
        n_bad = int(bad.sum())
        am = int(np.argmax(np.where(bad, 1.0, 0.0).ravel())) if n_bad else -1
        return dict(ok=n_bad == 0, n_bad=n_bad, n=int(ref.size), argmax=am,
                    max_abs=float(np.nanmax(np.abs(Cd - want))) if ref.size else 0.0,
                    max_ratio=float("inf") if n_bad else 0.0)
    tol = tolerance(ref, s, out_dtype, flags, scale, lib=lib)
    ratio = np.where(nan, np.inf, err / tol)
    bad = ratio > 1.0
    max_abs = float(np.max(np.where(nan, np.inf, err))) if ref.size else 0.0
    ok = not bool(bad.any())
    if abs_max is not None and max_abs > abs_max:
        ok = False
    am = int(np.argmax(ratio.ravel())) if ref.size else -1
    return dict(ok=ok, n_bad=int(bad.sum()), n=int(ref.size), argmax=am,
                max_ratio=float(ratio.ravel()[am]) if ref.size else 0.0, max_abs=max_abs)


def flops(M: int, N: int, K: int, batch: int = 1) -> int:
    """Work of the product: one multiply and one add per (i, j, k) (2*M*N*K)."""
    return 2 * M * N * K * batch


def gemm_bytes(M, N, K, in_bytes, out_bytes, batch=1, bias_bytes=0, resid_bytes=0) -> int:
    """Minimal traffic: A, B read once, C written once, plus bias and residual reads."""
    return batch * (M * K * in_bytes + K * N * in_bytes + M * N * out_bytes
                    + N * bias_bytes + M * N * resid_bytes)
