"""Attention continuation through the C ABI (GPU): the row softmax
(gemm_softmax_rows) against the fp64 oracle, and the chain S = Q K^T,
P = softmax(S), O = P V checked stage by stage (each stage fed the GPU's own
output of the stage before, against the oracle).

Softmax tolerance (oracle.softmax_tolerance): |P - p| <= p (4e-6 + 2^-22
max_c |scale S|) per row, plus half a 16-bit ulp for a 16-bit P.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_15_amd as g
    return g


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check_softmax(P, S, scale, out_dtype):
    ref = oracle.softmax_rows(S, scale)
    tol = oracle.softmax_tolerance(S, ref, scale, out_dtype)
    Pd = P.double().numpy() if out_dtype == "f32" else P.float().double().numpy()
    err = np.abs(Pd - ref)
    bad = ~(err <= tol)
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], tol[bad][:5])
    return (err / np.maximum(tol, 1e-300)).max()


@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_softmax_rows_shapes(g, out_dtype):
    """Rows of 1 to 4097 columns: register-held rows (multiples of 4 up to 1024,
    with partly filled chunks), the two-pass vector and scalar paths; scales 1, 1/8,
    2 and a negative one; scores up to |40|."""
    dev = torch.device("cuda")
    for i, (rows, cols, scale, std) in enumerate([(37, 1, 1.0, 1.0), (37, 3, 1.0, 3.0),
                                                  (64, 512, 1.0, 8.0), (5, 1000, 0.125, 8.0),
                                                  (7, 1024, -0.5, 4.0), (11, 4, 2.0, 1.0),
                                                  (6, 260, 1.0, 3.0), (3, 4097, 1.0, 2.0),
                                                  (9, 4096, 0.125, 40.0)]):
        S = synth.normal(600 + i, (rows, cols), std, "f32")
        P = g.softmax_rows(S.to(dev), scale, out_dtype).cpu()
        torch.cuda.synchronize()
        r = _check_softmax(P, S.numpy(), scale, out_dtype)
        say(f"[softmax] {rows}x{cols} scale {scale} {out_dtype}: max err/tol {r:.3f}")


def test_softmax_strides_and_errors(g):
    """Row strides larger than the row (through the C ABI directly), a 4-byte-offset
    S (scalar path), and the argument errors."""
    dev = torch.device("cuda")
    rows, cols, lds, ldp = 7, 100, 130, 111
    Sfull = synth.normal(610, (rows, lds), 2.0, "f32").to(dev)
    Pfull = torch.full((rows, ldp), -7.0, dtype=torch.float32, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = g.lib.gemm_softmax_rows(ctypes.c_void_p(Sfull.data_ptr()), rows, cols, lds, 1.0,
                                 ctypes.c_void_p(Pfull.data_ptr()), ldp, g.F32, s)
    torch.cuda.synchronize()
    assert rc == 0
    Pc = Pfull.cpu()
    _check_softmax(Pc[:, :cols], Sfull.cpu()[:, :cols].numpy(), 1.0, "f32")
    assert torch.all(Pc[:, cols:] == -7.0)  # columns past cols untouched
    # S starting 4 bytes past a 16-byte boundary: scalar loads
    buf = synth.normal(611, (1 + 6 * 64,), 1.0, "f32").to(dev)
    S = buf[1:].view(6, 64)
    P = g.softmax_rows(S, 1.0, "bf16").cpu()
    _check_softmax(P, S.cpu().numpy(), 1.0, "bf16")
    p = ctypes.c_void_p(Pfull.data_ptr())
    sp = ctypes.c_void_p(Sfull.data_ptr())
    assert g.lib.gemm_softmax_rows(sp, 0, cols, lds, 1.0, p, ldp, g.F32, s) == -1
    assert g.lib.gemm_softmax_rows(sp, rows, cols, cols - 1, 1.0, p, ldp, g.F32, s) == -10
    assert g.lib.gemm_softmax_rows(sp, rows, cols, lds, float("inf"), p, ldp, g.F32, s) == -10
    assert g.lib.gemm_softmax_rows(sp, rows, cols, lds, 1.0, p, ldp, 7, s) == -2
    assert g.lib.gemm_softmax_rows(None, rows, cols, lds, 1.0, p, ldp, g.F32, s) == -3


def _chain(g, Q, Kt, V):
    """S = Q Kt (fp32), P = softmax(S) (bf16), O = P V (fp32), batched over heads."""
    dev = torch.device("cuda")
    nb, Sq, D = Q.shape
    qk = g.Plan(Sq, Sq, D, "bf16", batch_hint=nb)
    pv = g.Plan(Sq, D, Sq, "bf16", batch_hint=nb)
    S = qk.run_batched(Q.to(dev), Kt.to(dev))
    P = g.softmax_rows(S, 1.0, "bf16")
    O = pv.run_batched(P, V.to(dev))
    torch.cuda.synchronize()
    return S.cpu(), P.cpu(), O.cpu(), qk, pv


def test_attention_chain_small(g):
    """3 heads of sequence 130 (ragged against every tile), head dimension 64: every
    element of S, P and O, stage by stage."""
    nb, Sq, D = 3, 130, 64
    Q = synth.normal(620, (nb, Sq, D), 1.0, "bf16")
    Kt = synth.normal(621, (nb, Sq, D), 1.0, "bf16").transpose(1, 2).contiguous()
    V = synth.normal(622, (nb, Sq, D), 1.0, "bf16")
    S, P, O, qk, pv = _chain(g, Q, Kt, V)
    say("[attention] qk", qk.describe(), "| pv", pv.describe())
    for b in range(nb):
        ref, s = oracle.gemm(synth.bits(Q[b]), synth.bits(Kt[b]), "bf16")
        assert oracle.check(synth.bits(S[b]), ref, s)["ok"], b
        _check_softmax(P[b], S[b].numpy(), 1.0, "bf16")
        ref, s = oracle.gemm(synth.bits(P[b]), synth.bits(V[b]), "bf16")
        r = oracle.check(synth.bits(O[b]), ref, s)
        assert r["ok"], (b, r)


def test_attention_workload_sampled(g):
    """The attention workload (96 heads, sequence 512, dimension 64) in the launch
    configuration the benchmark times: every head's S spot-checked, P checked on 4
    rows per head against the oracle softmax of the GPU's S, O on 64 elements per
    head against the oracle product of the GPU's P."""
    Q, Kt, V = synth.attention_inputs()
    S, P, O, _, _ = _chain(g, Q, Kt, V)
    nb, Sq, D = Q.shape
    rng = np.random.default_rng(630)
    for b in range(nb):
        rows = rng.integers(0, Sq, 4)
        _check_softmax(P[b][rows], S[b][rows].numpy(), 1.0, "bf16")
        ii, jj = rng.integers(0, Sq, 64), rng.integers(0, D, 64)
        ref, s = oracle.gemm_at(synth.bits(P[b]), synth.bits(V[b]), "bf16", ii, jj)
        r = oracle.check(O[b].numpy()[ii, jj], ref, s)
        assert r["ok"], (b, r)
        ii, jj = rng.integers(0, Sq, 64), rng.integers(0, Sq, 64)
        ref, s = oracle.gemm_at(synth.bits(Q[b]), synth.bits(Kt[b]), "bf16", ii, jj)
        assert oracle.check(S[b].numpy()[ii, jj], ref, s)["ok"], b
