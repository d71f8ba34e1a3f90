"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes a loaded oracle library handle and raises AssertionError
when the oracle disagrees with:

* closed forms (identity, all-ones, rank-1 products);
* exact integer arithmetic (numpy int64 matmul);
* a library routine on tiny shapes (numpy float64 matmul);
* torch's float32 -> bf16 / fp16 conversions and their decodes;
* the normal CDF of scipy (GELU(x) = x Phi(x)), GELU's odd-part identity;
* the figures the pages print (tests/golden).

``test_oracle.py`` runs every pin against the real oracle (all must pass) and
against deliberately broken copies of the oracle source (each copy must fail
at least one pin).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
from scipy.stats import norm

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers --

def _bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values (representable in dtype) -> raw bits via torch."""
    t = torch.from_numpy(np.asarray(x, np.float32))
    if dtype == "f32":
        return t.numpy().copy()
    tt = t.to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return tt.view(torch.int16).numpy().view(np.uint16).copy()


def _rng(seed):
    return np.random.default_rng(seed)


DTYPES = ("f32", "f16", "bf16")


# -------------------------------------------------------------------- codecs --

def pin_decode_all_patterns(lib):
    """Every 16-bit pattern decodes to what torch's widening to float32 gives."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        want = torch.from_numpy(pats.view(np.int16)).view(tdt).to(torch.float32).numpy()
        got = oracle.decode(dt, pats, lib=lib)
        fin = np.isfinite(want)
        assert np.array_equal(got[fin], want[fin].astype(np.float64)), dt
        assert np.array_equal(np.isnan(got), np.isnan(want)), dt
        assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(want) & (want > 0)), dt


def pin_round_trip(lib):
    """Decoding then rounding gives the pattern back (all non-NaN patterns)."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt in ("bf16", "f16"):
        v = oracle.decode(dt, pats, lib=lib)
        keep = ~np.isnan(v)
        back = oracle.round16(dt, v[keep], lib=lib)
        assert np.array_equal(back, pats[keep]), dt


def pin_round_matches_torch(lib):
    """RNE of random fp32 values and of exact halfway cases agrees with torch."""
    r = _rng(7)
    x = np.concatenate([
        r.uniform(-1, 1, 200000),
        r.standard_normal(200000) * 1e3,
        r.standard_normal(50000) * 1e-6,
        np.ldexp(r.uniform(1, 2, 20000), r.integers(-30, 17, 20000)),
    ]).astype(np.float32)
    # exact halfway points between neighbouring 16-bit values
    half_bf = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 3 * 2**-9 + 2**-17], np.float32)
    half_h = np.array([1 + 2**-11, 1 + 3 * 2**-11, 2048 + 1, 2048 + 3, 65519.0, 65520.0,
                       2**-25, 3 * 2**-25, 2**-26], np.float32)
    for dt, tdt, extra in (("bf16", torch.bfloat16, half_bf), ("f16", torch.float16, half_h)):
        xx = np.concatenate([x, extra])
        want = torch.from_numpy(xx).to(tdt).view(torch.int16).numpy().view(np.uint16)
        got = oracle.round16(dt, xx.astype(np.float64), lib=lib)
        assert np.array_equal(got, want), dt
    # ties to even, spelled out
    got = oracle.round16("bf16", np.array([1 + 2**-8, 1 + 3 * 2**-8]), lib=lib)
    assert list(oracle.decode("bf16", got, lib=lib)) == [1.0, 1 + 2**-6]
    got = oracle.round16("f16", np.array([65519.0, 65520.0, 1e6]), lib=lib)
    assert list(oracle.decode("f16", got, lib=lib)) == [65504.0, math.inf, math.inf]


def pin_ulp16(lib):
    """Spacing of bf16 / fp16 at a few known points."""
    assert oracle.ulp16("bf16", np.array([1.0, 1.5, 2.0, 0.75]), lib=lib).tolist() == \
        [2**-7, 2**-7, 2**-6, 2**-8]
    assert oracle.ulp16("f16", np.array([1.0, 1024.0, 2**-14, 2**-20, 0.0]), lib=lib).tolist() == \
        [2**-10, 1.0, 2**-24, 2**-24, 2**-24]


# ---------------------------------------------------------------------- GELU --

def pin_gelu(lib):
    """GELU(x) = x Phi(x) against scipy's normal CDF; GELU(x) - GELU(-x) = x; and full
    relative accuracy in the negative tail, where Phi is tiny (scipy's normal CDF is
    accurate there; a 1 + erf form loses every digit below about x = -8)."""
    xs = np.linspace(-8, 8, 641)
    got = np.array([oracle.gelu(x, lib=lib) for x in xs])
    want = xs * norm.cdf(xs)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-15)
    tail = -np.linspace(1.0, 37.0, 361)
    got = np.array([oracle.gelu(x, lib=lib) for x in tail])
    assert np.allclose(got, tail * norm.cdf(tail), rtol=1e-12, atol=0.0)
    odd = np.array([oracle.gelu(x, lib=lib) - oracle.gelu(-x, lib=lib) for x in xs])
    assert np.allclose(odd, xs, rtol=1e-14, atol=1e-15)
    assert oracle.gelu(0.0, lib=lib) == 0.0
    # textbook table value Phi(1) = 0.841344746...
    assert abs(oracle.gelu(1.0, lib=lib) - 0.8413447460685429) < 1e-15


# -------------------------------------------------------------------- product --

def pin_identity(lib):
    """I x B = B and A x I = A, exactly, in every input type."""
    r = _rng(11)
    for dt in DTYPES:
        B = _bits(r.uniform(-1, 1, (13, 7)), dt)
        I13 = _bits(np.eye(13), dt)
        ref, _ = oracle.gemm(I13, B, dt, lib=lib)
        assert np.array_equal(ref, oracle.decode(dt, B, lib=lib)), dt
        A = _bits(r.uniform(-1, 1, (5, 9)), dt)
        I9 = _bits(np.eye(9), dt)
        ref, _ = oracle.gemm(A, I9, dt, lib=lib)
        assert np.array_equal(ref, oracle.decode(dt, A, lib=lib)), dt


def pin_ones(lib):
    """All-ones left operand gives column sums; all-ones right operand gives row sums."""
    r = _rng(12)
    for dt in DTYPES:
        Bi = r.integers(-8, 9, (17, 6)).astype(np.float64)
        ref, _ = oracle.gemm(_bits(np.ones((4, 17)), dt), _bits(Bi, dt), dt, lib=lib)
        assert np.array_equal(ref, np.broadcast_to(Bi.sum(axis=0), (4, 6))), dt
        Ai = r.integers(-8, 9, (3, 19)).astype(np.float64)
        ref, _ = oracle.gemm(_bits(Ai, dt), _bits(np.ones((19, 5)), dt), dt, lib=lib)
        assert np.array_equal(ref, np.broadcast_to(Ai.sum(axis=1)[:, None], (3, 5))), dt


def pin_rank1(lib):
    """(u v^T)(w x^T) = (v . w) u x^T, exact for small integers."""
    r = _rng(13)
    for dt in DTYPES:
        M, K, N = 6, 11, 4
        u, v = r.integers(-2, 3, M), r.integers(-2, 3, K)
        w, x = r.integers(-2, 3, K), r.integers(-2, 3, N)
        A = _bits(np.outer(u, v), dt)
        B = _bits(np.outer(w, x), dt)
        ref, _ = oracle.gemm(A, B, dt, lib=lib)
        assert np.array_equal(ref, float(np.dot(v, w)) * np.outer(u, x).astype(np.float64)), dt


def pin_integer_exact(lib):
    """Small-integer inputs: every element equals the int64 product; s = |A| |B|."""
    r = _rng(14)
    for dt in DTYPES:
        for (M, N, K) in ((37, 29, 41), (1, 64, 300), (70, 3, 129)):
            Ai = r.integers(-8, 9, (M, K))
            Bi = r.integers(-8, 9, (K, N))
            ref, s = oracle.gemm(_bits(Ai, dt), _bits(Bi, dt), dt, lib=lib)
            assert np.array_equal(ref, (Ai @ Bi).astype(np.float64)), (dt, M, N, K)
            assert np.array_equal(s, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64)), (dt, M, N, K)


def pin_bruteforce_tiny(lib):
    """Every (M,N,K) in {1..9}^3 plus a few prime shapes against numpy's float64 matmul."""
    r = _rng(15)
    shapes = [(m, n, k) for m in range(1, 10) for n in range(1, 10) for k in range(1, 10)]
    shapes += [(37, 31, 29), (2, 37, 23), (31, 3, 37)]
    for idx, (M, N, K) in enumerate(shapes):
        dt = DTYPES[idx % 3]
        A = _bits(r.uniform(-1, 1, (M, K)), dt)
        B = _bits(r.uniform(-1, 1, (K, N)), dt)
        Ad, Bd = oracle.decode(dt, A, lib=lib), oracle.decode(dt, B, lib=lib)
        ref, s = oracle.gemm(A, B, dt, lib=lib)
        want = Ad @ Bd
        sw = np.abs(Ad) @ np.abs(Bd)
        assert np.all(np.abs(ref - want) <= 1e-12 * sw + 1e-300), (dt, M, N, K)
        assert np.allclose(s, sw, rtol=1e-12, atol=0), (dt, M, N, K)


def pin_selected_elements(lib):
    """gemm_at agrees with the full loop on scattered elements (same k order)."""
    r = _rng(16)
    for dt in DTYPES:
        M, N, K = 33, 47, 65
        A = _bits(r.uniform(-1, 1, (M, K)), dt)
        B = _bits(r.uniform(-1, 1, (K, N)), dt)
        bias = r.standard_normal(N).astype(np.float32)
        res = _bits(r.uniform(-1, 1, (M, N)), dt)
        fl = oracle.BIAS | oracle.GELU | oracle.RESID | oracle.SCALE
        ref, s = oracle.gemm(A, B, dt, fl, 0.5, bias, res, dt, lib=lib)
        rows = r.integers(0, M, 200)
        cols = r.integers(0, N, 200)
        ra, sa = oracle.gemm_at(A, B, dt, rows, cols, fl, 0.5, bias, res, dt, lib=lib)
        assert np.array_equal(ra, ref[rows, cols]), dt
        assert np.array_equal(sa, s[rows, cols]), dt


# ------------------------------------------------------------------- epilogue --

def pin_epilogue_plumbing(lib):
    """A = 0: C = bias (broadcast), C = resid; scale by 2^-3 is exact; flag order."""
    r = _rng(17)
    M, N, K = 5, 6, 7
    for dt in DTYPES:
        Z = _bits(np.zeros((M, K)), dt)
        B = _bits(r.uniform(-1, 1, (K, N)), dt)
        bias = r.standard_normal(N).astype(np.float32)
        ref, _ = oracle.gemm(Z, B, dt, oracle.BIAS, 1.0, bias, lib=lib)
        assert np.array_equal(ref, np.broadcast_to(bias.astype(np.float64), (M, N))), dt
        res = _bits(r.uniform(-1, 1, (M, N)), dt)
        ref, _ = oracle.gemm(Z, B, dt, oracle.RESID, 1.0, None, res, dt, lib=lib)
        assert np.array_equal(ref, oracle.decode(dt, res, lib=lib)), dt
        Ai = r.integers(-8, 9, (M, K))
        Bi = r.integers(-8, 9, (K, N))
        ref, s = oracle.gemm(_bits(Ai, dt), _bits(Bi, dt), dt, oracle.SCALE, 0.125, lib=lib)
        assert np.array_equal(ref, (Ai @ Bi) * 0.125), dt
        assert np.array_equal(s, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64)), dt


def pin_epilogue_order(lib):
    """scale, then bias, then GELU, then residual: C = GELU(a*AB + b) + R."""
    r = _rng(18)
    M, N, K = 4, 9, 5
    Ai = r.integers(-3, 4, (M, K))
    Bi = r.integers(-3, 4, (K, N))
    bias = (r.integers(-4, 5, N) * 0.25).astype(np.float32)
    R = r.integers(-2, 3, (M, N)).astype(np.float64)
    acc = (Ai @ Bi).astype(np.float64)
    for fl, want in (
        (oracle.SCALE | oracle.BIAS, 0.5 * acc + bias),
        (oracle.BIAS | oracle.GELU, (acc + bias) * norm.cdf(acc + bias)),
        (oracle.SCALE | oracle.BIAS | oracle.GELU | oracle.RESID,
         (0.5 * acc + bias) * norm.cdf(0.5 * acc + bias) + R),
        (oracle.GELU | oracle.RESID, acc * norm.cdf(acc) + R),
    ):
        ref, _ = oracle.gemm(_bits(Ai, "f32"), _bits(Bi, "f32"), "f32", fl, 0.5, bias,
                             _bits(R, "f32"), "f32", lib=lib)
        assert np.allclose(ref, want, rtol=1e-13, atol=1e-13), fl


# ------------------------------------------------------------ accounting, tol --

def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def pin_page_figures(lib):
    """The work and byte counts the pages print (tests/golden/page_figures.txt)."""
    for row in _golden("page_figures.txt"):
        kind = row[0]
        if kind == "flops":
            M, N, K = map(int, row[1:4])
            want, digits = float(row[4]), int(row[5])
            assert round(oracle.flops(M, N, K) / 1e9, digits) == want, row
        elif kind == "bytes":
            rows_, cols, esize = map(int, row[1:4])
            want_mib = float(row[4])
            got = oracle.gemm_bytes(rows_, 0, cols, esize, 0)  # one M x K operand
            assert got / 2**20 == want_mib, row


def pin_hand_example(lib):
    """A hand-worked 2x3 by 3x2 example with bias and residual (tests/golden)."""
    rows = _golden("hand_2x3x2.txt")
    data = {r[0]: [float(v) for v in r[1:]] for r in rows}
    A = np.array(data["A"]).reshape(2, 3)
    B = np.array(data["B"]).reshape(3, 2)
    bias = np.array(data["bias"], np.float32)
    R = np.array(data["resid"]).reshape(2, 2)
    ref, _ = oracle.gemm(_bits(A, "f32"), _bits(B, "f32"), "f32", lib=lib)
    assert ref.ravel().tolist() == data["C"]
    ref, _ = oracle.gemm(_bits(A, "f32"), _bits(B, "f32"), "f32",
                         oracle.SCALE | oracle.BIAS | oracle.RESID, 0.5, bias, _bits(R, "f32"),
                         "f32", lib=lib)
    assert ref.ravel().tolist() == data["C_epi"]


def pin_check_logic(lib):
    """The acceptance test accepts the reference, rejects 2x the tolerance and NaN."""
    r = _rng(19)
    A = _bits(r.uniform(-1, 1, (8, 16)), "bf16")
    B = _bits(r.uniform(-1, 1, (16, 8)), "bf16")
    ref, s = oracle.gemm(A, B, "bf16", lib=lib)
    tol = oracle.tolerance(ref, s, lib=lib)
    assert np.allclose(tol, 1e-4 * s + 1e-6, rtol=1e-15)
    C = ref.astype(np.float32)
    assert oracle.check(C, ref, s, lib=lib)["ok"]
    bad = (ref + 2 * tol).astype(np.float32)
    assert not oracle.check(bad, ref, s, lib=lib)["ok"]
    nanC = C.copy()
    nanC[3, 4] = np.nan
    out = oracle.check(nanC, ref, s, lib=lib)
    assert not out["ok"] and out["argmax"] == 3 * 8 + 4
    # 16-bit output: the RNE of the reference is accepted
    C16 = oracle.round16("bf16", ref, lib=lib)
    assert oracle.check(C16, ref, s, "bf16", lib=lib)["ok"]
    # exact mode
    Ai = r.integers(-8, 9, (8, 16))
    Bi = r.integers(-8, 9, (16, 8))
    ref, s = oracle.gemm(_bits(Ai, "f16"), _bits(Bi, "f16"), "f16", lib=lib)
    assert oracle.check((Ai @ Bi).astype(np.float32), ref, s, exact=True, lib=lib)["ok"]
    off = (Ai @ Bi).astype(np.float32)
    off[0, 0] += 1
    assert not oracle.check(off, ref, s, exact=True, lib=lib)["ok"]


def pin_f16acc_stepwise(lib):
    """FP16 accumulation (DeepGEMM page, section 3.4) against a step-by-step numpy
    model: the exact acc + a*b in float64, rounded to float16 by numpy's own
    conversion (round to nearest even) at every k. Inputs on the 2^-10 grid, where
    the float64 sum is exact."""
    r = _rng(41)
    for M, N, K in [(3, 4, 1), (5, 7, 33), (2, 3, 257)]:
        A = (r.integers(-1024, 1025, (M, K)) / 1024).astype(np.float16)
        B = (r.integers(-1024, 1025, (K, N)) / 1024).astype(np.float16)
        got = oracle.gemm_f16acc(A.view(np.uint16), B.view(np.uint16), lib=lib)
        want = np.zeros((M, N))
        for i in range(M):
            for j in range(N):
                acc = np.float16(0)
                for k in range(K):
                    acc = np.float16(np.float64(acc) + np.float64(A[i, k]) * np.float64(B[k, j]))
                want[i, j] = acc
        assert np.array_equal(got, want), (M, N, K)


def pin_f16acc_closed_forms(lib):
    """FP16 accumulation: B = I returns A exactly; K = 1 returns RNE16(a b); with
    K = 2048 random products the fp16 accumulator is off the exact sum by far more
    than fp32 accumulation would be (the error the page warns about)."""
    r = _rng(42)
    A = (r.integers(-1024, 1025, (6, 9)) / 1024).astype(np.float16)
    I = np.eye(9, dtype=np.float16)
    assert np.array_equal(oracle.gemm_f16acc(A.view(np.uint16), I.view(np.uint16), lib=lib),
                          A.astype(np.float64))
    a = (r.integers(-1024, 1025, (8, 1)) / 1024).astype(np.float16)
    b = (r.integers(-1024, 1025, (1, 8)) / 1024).astype(np.float16)
    want = (a.astype(np.float64) @ b.astype(np.float64)).astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.gemm_f16acc(a.view(np.uint16), b.view(np.uint16), lib=lib), want)
    A = (r.integers(-1024, 1025, (4, 2048)) / 1024).astype(np.float16)
    B = (r.integers(-1024, 1025, (2048, 4)) / 1024).astype(np.float16)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    err16 = np.abs(oracle.gemm_f16acc(A.view(np.uint16), B.view(np.uint16), lib=lib) - exact).max()
    err32 = np.abs((A.astype(np.float32) @ B.astype(np.float32)).astype(np.float64) - exact).max()
    assert err16 > 1e-3 and err16 > 100 * err32, (err16, err32)


def pin_softmax_library(lib):
    """Row softmax against scipy.special.softmax on random rows (a library routine),
    with a scale; rows sum to 1; a two-element row is the logistic function."""
    from scipy.special import softmax as sp_softmax
    r = _rng(51)
    for rows, cols, scale in [(3, 1, 1.0), (5, 7, 1.0), (4, 513, 0.125), (2, 64, 3.0)]:
        S = (r.standard_normal((rows, cols)) * 4).astype(np.float32)
        got = oracle.softmax_rows(S, scale, lib=lib)
        want = sp_softmax(scale * S.astype(np.float64), axis=1)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-300), (rows, cols, scale)
        assert np.allclose(got.sum(axis=1), 1.0, rtol=0, atol=1e-13 * cols)
    x = np.array([[0.75, -1.5]], np.float32)
    p0 = 1.0 / (1.0 + math.exp(-1.5 - 0.75))
    got = oracle.softmax_rows(x, lib=lib)
    assert abs(got[0, 0] - p0) <= 1e-15 and abs(got[0, 1] - (1 - p0)) <= 1e-15


def pin_softmax_invariants(lib):
    """Shift invariance, equal entries give 1/cols exactly, and scores of 1e4 do not
    overflow (the row maximum gets all of the weight)."""
    r = _rng(52)
    S = (r.integers(-3072, 3073, (6, 40)) / 1024).astype(np.float32)
    a = oracle.softmax_rows(S, lib=lib)
    b = oracle.softmax_rows(S + np.float32(64.0), lib=lib)  # exact: S is on the 2^-10 grid
    assert np.allclose(a, b, rtol=1e-12, atol=0)
    eq = oracle.softmax_rows(np.full((2, 8), 3.5, np.float32), lib=lib)
    assert np.array_equal(eq, np.full((2, 8), 0.125))
    big = np.zeros((1, 5), np.float32)
    big[0, 2] = 1e4
    got = oracle.softmax_rows(big, lib=lib)
    assert np.all(np.isfinite(got)) and got[0, 2] == 1.0 and got[0, 0] == 0.0


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
