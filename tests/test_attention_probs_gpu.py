"""The attention probabilities in one kernel (gemm_attention_probs: P =
softmax(scale Q K^T) with the scores kept in registers) against the fp64 oracle,
through the C ABI: both storages of the keys, every P type, head dimensions 8 to 64,
ragged query counts, 1 to 512 keys, and the 96-head launch the benchmark times.

Tolerance: the kernel's scores are the fp32 product, within the product bound t_S =
1e-4 sum|q k| + 1e-6 of the exact ones; a softmax moves by at most p (|d_i| + max
|d|) when its inputs move by d, so the bound is the oracle's fp32-softmax bound
(oracle.softmax_tolerance, on the exact scores rounded to fp32) plus p (2 |scale|
max_row t_S + 2^-23 max_row |scale S|) for the two roundings of the scores, plus
2^-126: a probability below the smallest normal fp32 number may come out as 0 (the
exact value of exp(-60) / sum is not an fp32 number at all).
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


def _keys_t(Kmat, layout):
    """K^T [D x N] of one item, as the oracle takes B."""
    return Kmat if layout == "kn" else Kmat.transpose(0, 1).contiguous()


def _check_rows(P, S_ref, s_abs, scale, out_dtype):
    """P rows against the softmax of the exact scores S_ref (float64, with sum|qk|
    s_abs); returns the largest error / bound."""
    S32 = S_ref.astype(np.float32)
    ref = oracle.softmax_rows(S32, scale)
    tS = oracle.tolerance(S_ref, s_abs)
    R = np.abs(scale * S_ref).max(axis=1, keepdims=True)
    tol = (oracle.softmax_tolerance(S32, ref, scale, out_dtype)
           + ref * (2 * abs(scale) * tS.max(axis=1, keepdims=True) + 2.0 ** -23 * R)
           + 2.0 ** -126)
    Pd = P.double().numpy() if out_dtype == "f32" else P.float().double().numpy()
    err = np.abs(Pd - ref)
    bad = ~(err <= tol)
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], tol[bad][:5])
    return float((err / np.maximum(tol, 1e-300)).max())


def _check_item(P, Q, Kmat, layout, scale, out_dtype, dtype):
    ref, s = oracle.gemm(synth.bits(Q), synth.bits(_keys_t(Kmat, layout)), dtype)
    return _check_rows(P, ref, s, scale, out_dtype)


CASES = [  # (batch, M, N, D, layout, scale, input std)
    (3, 130, 136, 64, "kn", 0.125, 1.0),
    (2, 64, 512, 64, "kn", 0.125, 1.0),
    (2, 65, 512, 64, "nk", 1.0, 1.0),
    (9, 200, 200, 40, "nk", 0.25, 1.0),
    (1, 1, 8, 8, "kn", 1.0, 1.0),
    (1, 3, 1, 64, "nk", 1.0, 1.0),
    (17, 70, 96, 16, "kn", -0.5, 2.0),
    (2, 129, 264, 64, "kn", 1.0, 2.0),  # scores of std ~16: many exp underflow to 0
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_m{}_n{}_d{}_{}".format(*c[:5]))
def test_attention_probs(g, case, dtype):
    """Every element of P for each P type, against the oracle."""
    nb, M, N, D, layout, scale, std = case
    dev = torch.device("cuda")
    seed = 2000 + 7 * CASES.index(case) + (0 if dtype == "bf16" else 3)
    Q = synth.normal(seed, (nb, M, D), std, dtype)
    Kmat = synth.normal(seed + 1, (nb, D, N) if layout == "kn" else (nb, N, D), std, dtype)
    Qd, Kd = Q.to(dev), Kmat.to(dev)
    for out_dtype in ("f32", "bf16", "f16"):
        say(f"[attention_probs] {dtype} {case} -> {out_dtype}")
        out = torch.full((nb, M, N), float("nan"), dtype=synth.DTYPES[out_dtype], device=dev)
        P = g.attention_probs(Qd, Kd, scale, layout, out_dtype, out=out)
        torch.cuda.synchronize()
        P = P.cpu()
        worst = max(_check_item(P[b], Q[b], Kmat[b], layout, scale, out_dtype, dtype)
                    for b in range(nb))
        say(f"    max err/bound {worst:.3f}")


@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_attention_probs_heads(g, layout):
    """The benchmark's launch: 96 heads, 512 queries and keys, dimension 64, scale
    1/8, bf16 P. Four heads (first, last, either side of an XCD boundary) in full,
    eight whole rows of every other head."""
    Q, Kt = synth.qk_inputs()
    nb, S, D = Q.shape
    Kmat = Kt if layout == "kn" else Kt.transpose(1, 2).contiguous()
    dev = torch.device("cuda")
    P = g.attention_probs(Q.to(dev), Kmat.to(dev), 0.125, layout, "bf16")
    torch.cuda.synchronize()
    P = P.cpu()
    rng = np.random.default_rng(2100)
    worst = 0.0
    for b in range(nb):
        if b in (0, 7, 8, nb - 1):
            worst = max(worst, _check_item(P[b], Q[b], Kt[b], "kn", 0.125, "bf16", "bf16"))
            continue
        rows = rng.choice(S, 8, replace=False)
        ii = np.repeat(rows, S)
        jj = np.tile(np.arange(S), 8)
        ref, s = oracle.gemm_at(synth.bits(Q[b]), synth.bits(Kt[b]), "bf16", ii, jj)
        worst = max(worst, _check_rows(P[b][torch.as_tensor(rows)], ref.reshape(8, S),
                                       s.reshape(8, S), 0.125, "bf16"))
    say(f"[attention_probs] 96 heads {layout}: max err/bound {worst:.3f}")


@pytest.mark.parametrize("nb,M,N,layout", [(80, 250, 136, "kn"), (70, 256, 512, "nk")])
def test_attention_probs_runs_cross_items(g, nb, M, N, layout):
    """More 32-row tiles than resident workgroups (640 and 560 against 512), so
    workgroups walk runs of one or two tiles and many runs cross into the next item
    (keys reloaded mid-run); N = 512 with whole tiles takes the unchecked store
    path. Every element of every item."""
    dev = torch.device("cuda")
    seed = 2300 + nb
    Q = synth.normal(seed, (nb, M, 64), 1.0, "bf16")
    Kmat = synth.normal(seed + 1, (nb, 64, N) if layout == "kn" else (nb, N, 64), 1.0, "bf16")
    P = g.attention_probs(Q.to(dev), Kmat.to(dev), 0.125, layout, "bf16")
    torch.cuda.synchronize()
    P = P.cpu()
    worst = max(_check_item(P[b], Q[b], Kmat[b], layout, 0.125, "bf16", "bf16") for b in range(nb))
    say(f"[attention_probs] {nb} x {M}x{N} {layout}: max err/bound {worst:.3f}")


def test_attention_probs_errors(g):
    """Argument errors come back as status codes and launch nothing."""
    dev = torch.device("cuda")
    Q = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device=dev)
    Kt = torch.zeros((2, 64, 520), dtype=torch.bfloat16, device=dev)
    P = torch.zeros((2, 64, 520), dtype=torch.float32, device=dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    q, k, p = (ctypes.c_void_p(t.data_ptr()) for t in (Q, Kt, P))
    call = g.lib.gemm_attention_probs
    assert call(q, k, 2, 64, 512, 64, g.BF16, 0, 1.0, p, g.F32, s) == 0
    assert call(q, k, 2, 64, 520, 64, g.BF16, 0, 1.0, p, g.F32, s) == -1   # N > 512
    assert call(q, k, 2, 64, 500, 72, g.BF16, 0, 1.0, p, g.F32, s) == -1   # D > 64
    assert call(q, k, 2, 64, 500, 12, g.BF16, 0, 1.0, p, g.F32, s) == -1   # D % 8
    assert call(q, k, 2, 64, 12, 64, g.BF16, 0, 1.0, p, g.F32, s) == -1    # kn needs N % 8
    assert call(q, k, 0, 64, 64, 64, g.BF16, 0, 1.0, p, g.F32, s) == -1
    assert call(q, k, 2, 64, 64, 64, g.BF16, 2, 1.0, p, g.F32, s) == -10   # layout
    assert call(q, k, 2, 64, 64, 64, g.BF16, 0, float("nan"), p, g.F32, s) == -10
    assert call(q, k, 2, 64, 64, 64, g.F32, 0, 1.0, p, g.F32, s) == -2
    assert call(q, k, 2, 64, 64, 64, g.BF16, 0, 1.0, p, 9, s) == -2
    assert call(None, k, 2, 64, 64, 64, g.BF16, 0, 1.0, p, g.F32, s) == -3
    q8 = ctypes.c_void_p(Q.data_ptr() + 8)
    assert call(q8, k, 2, 64, 64, 64, g.BF16, 0, 1.0, p, g.F32, s) == -4
    torch.cuda.synchronize()


def test_attention_probs_graph_replay(g):
    """The fused kernel captured in a HIP graph and replayed with new Q between
    replays and eager work in between: every replay equals the eager result bit for
    bit."""
    nb, M, N, D = 9, 130, 200, 64
    dev = torch.device("cuda")
    Qs = [synth.normal(2200 + i, (nb, M, D), 1.0, "bf16").to(dev) for i in range(2)]
    Kmat = synth.normal(2202, (nb, N, D), 1.0, "bf16").to(dev)
    eager = [g.attention_probs(Q, Kmat, 0.125, "nk", "bf16").clone() for Q in Qs]
    torch.cuda.synchronize()
    Q0 = Qs[0].clone()
    out = torch.empty((nb, M, N), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.attention_probs(Q0, Kmat, 0.125, "nk", "bf16", out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.attention_probs(Q0, Kmat, 0.125, "nk", "bf16", out=out)
    junk = torch.randn(1 << 20, device=dev)
    for rep, i in enumerate((0, 1, 1, 0)):
        Q0.copy_(Qs[i])
        out.fill_(float("nan"))
        graph.replay()
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[i].view(torch.int16)), (rep, i)
