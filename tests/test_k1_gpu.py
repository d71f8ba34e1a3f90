"""Parity of the one-slice streaming kernels (m16s_*: K <= 64, each workgroup looping
over tiles and batch items with the next tile's operands loading; *_nk with B given
transposed) against the fp64
oracle, through the C ABI: ragged shapes with K below, at and well under 64, more
tiles than resident workgroups and fewer, batches split by item over the XCDs (8 or
more items, an uneven number per XCD) and not (fewer items), every epilogue and
output type, and the 96-head attention-scores launch the benchmark times."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import synth
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_15_amd as g
    return g


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _configs():
    try:
        import dense_gemm_15_amd as g
        return [c for c in g.config_names() if c.startswith("m16s")]
    except Exception:
        return []


K1 = _configs()


def _tile(name):
    bm, bn, _ = (int(x) for x in name.split("_")[2].split("x"))
    return bm, bn


def _dtype(name):
    return "bf16" if "_bf16_" in name else "f16"


def _nk(name):
    """Configurations for B given transposed (Bt [N x K]) carry _nk."""
    return "_nk" in name


def _unaligned(name):
    """The register-load forms (_u) take rows of any 2-byte alignment."""
    return name.endswith("_u")


def _plan(g, name, M, N, K, **kw):
    return g.Plan(M, N, K, _dtype(name), config=name, b_layout="nk" if _nk(name) else "kn", **kw)


def _given(name, B):
    """B as the configuration takes it (the oracle always gets B [.., K, N])."""
    return B.transpose(-1, -2).contiguous() if _nk(name) else B


@pytest.mark.parametrize("name", K1)
def test_k1_ragged(g, name):
    """Ragged shapes with K = 64, 40, 16 and 8, each element against the oracle; a
    shape of more tiles than resident workgroups checked on its edges and a sample."""
    dtype = _dtype(name)
    bm, bn = _tile(name)
    for si, (M, N, K) in enumerate([(2 * bm + 3, bn + 8, 64), (bm, 2 * bn + 8, 40), (1, 8, 8),
                                    (3 * bm + 5, 5 * bn + 24, 16)]):
        say(f"[{name}] M={M} N={N} K={K}")
        plan = _plan(g, name, M, N, K)
        assert plan.config_name == name
        for kind in ("uniform", "int"):
            A, B = gc.inputs(M, N, K, dtype, 1300 + 11 * si, kind)
            C = gc.run_gpu(plan, A, _given(name, B))
            r = gc.check_full(C, A, B, dtype, exact=(kind == "int"))
            assert r["ok"], (name, M, N, K, kind, r)
    M, N, K = 4096 + 5, 4096 + 8, 64
    say(f"[{name}] M={M} N={N} K={K} (more tiles than workgroups)")
    plan = _plan(g, name, M, N, K)
    A, B = gc.inputs(M, N, K, dtype, 1350, "uniform")
    C = gc.run_gpu(plan, A, _given(name, B))
    rows, cols = gc.sample_indices(M, N, 400, 1351)
    r = gc.check_sampled(C, A, B, dtype, rows, cols)
    assert r["ok"], (name, r)


@pytest.mark.parametrize("name", K1)
def test_k1_epilogues(g, name):
    """Bias + GELU into 16-bit C, scale + residual into fp32 and 16-bit C (the 16-bit
    forms store straight from the registers), every element."""
    dtype = _dtype(name)
    bm, bn = _tile(name)
    M, N, K = 2 * bm + 3, bn + 8, 64
    cases = [dict(out_dtype="bf16", bias=True, gelu=True),
             dict(out_dtype="f16", bias=True, gelu=True),
             dict(out_dtype="f32", resid=True, scale=0.125),
             dict(out_dtype=dtype, resid=True, scale=-2.0, bias=True)]
    for ci, epi in enumerate(cases):
        say(f"[{name}] epilogue {epi}")
        plan = _plan(g, name, M, N, K, **epi)
        assert plan.config_name == name
        A, B = gc.inputs(M, N, K, dtype, 1400 + ci)
        bias = synth.normal(1410 + ci, (N,), 0.5, "f32") if epi.get("bias") else None
        resid = (synth.normal(1420 + ci, (M, N), 1.0, epi["out_dtype"])
                 if epi.get("resid") else None)
        C = gc.run_gpu(plan, A, _given(name, B), bias, resid)
        r = gc.check_full(C, A, B, dtype, epi["out_dtype"], bias, resid, epi.get("scale"),
                          epi.get("gelu", False))
        assert r["ok"], (name, epi, r)


@pytest.mark.parametrize("nb,M,N", [(5, 130, 136), (9, 300, 264), (17, 129, 128)])
def test_k1_batched_ragged(g, nb, M, N):
    """Batches of ragged products with K = 64: fewer than 8 items (tiles strided over
    the workgroups), 9 and 17 items (split by item over the XCDs, uneven per XCD);
    every element of every item, on every bf16 configuration (both B layouts)."""
    K = 64
    for name in [c for c in K1 if "_bf16_" in c]:
        say(f"[{name}] batch {nb} M={M} N={N} K={K}")
        plan = _plan(g, name, M, N, K, batch_hint=nb)
        A = synth.uniform(1500 + nb, (nb, M, K), "bf16")
        B = synth.uniform(1501 + nb, (nb, K, N), "bf16")
        dev = torch.device("cuda")
        C = plan.run_batched(A.to(dev), _given(name, B).to(dev))
        torch.cuda.synchronize()
        C = C.cpu()
        for b in range(nb):
            r = gc.check_full(C[b], A[b], B[b], "bf16")
            assert r["ok"], (name, nb, b, r)


def test_k1_attention_scores(g):
    """The 96 heads of Q K^T (sequence 512, dimension 64) through each bf16 m16s
    configuration, the launch the benchmark times: four heads (first, last, the two
    either side of an XCD boundary) in full, 64 elements of every other head."""
    Q, Kt = synth.qk_inputs()
    nb, S, D = Q.shape
    dev = torch.device("cuda")
    Qd = Q.to(dev)
    rng = np.random.default_rng(1600)
    for name in [c for c in K1 if "_bf16_" in c]:
        say(f"[{name}] 96 x 512x512x64")
        plan = _plan(g, name, S, S, D, batch_hint=nb)
        out = plan.run_batched(Qd, _given(name, Kt).to(dev))
        torch.cuda.synchronize()
        out = out.cpu()
        for b in range(nb):
            if b in (0, 7, 8, nb - 1):
                r = gc.check_full(out[b], Q[b], Kt[b], "bf16")
            else:
                ii, jj = rng.integers(0, S, 64), rng.integers(0, S, 64)
                r = gc.check_sampled(out[b], Q[b], Kt[b], "bf16", ii, jj)
            assert r["ok"], (name, b, r)


UNALIGNED = [
    # (M, N, K): K and N not multiples of 8 (rows of odd element counts; the last
    # chunk of a row holds 1 to 7 elements, each count at least once for K and N),
    # thin last tile column and row, K below 8 (element loads), K of one element, a
    # product smaller than one tile
    (517, 261, 63),
    (300, 1001, 57),
    (1029, 387, 7),
    (260, 130, 1),
    (37, 19, 33),
    (300, 1020, 46),
    (70, 1022, 12),
]


@pytest.mark.parametrize("name", [c for c in K1 if _unaligned(c)])
def test_k1_unaligned_rows(g, name):
    """The register-load form on rows that are not 16-byte multiples (odd K, odd N,
    both), with thin last tile strips, float and small-integer inputs, fp32 C and an
    epilogue into 16-bit C: every element against the oracle."""
    dtype = _dtype(name)
    for si, (M, N, K) in enumerate(UNALIGNED):
        for kind in ("uniform", "int"):
            say(f"[{name}] M={M} N={N} K={K} {kind}")
            plan = _plan(g, name, M, N, K)
            assert plan.config_name == name
            A, B = gc.inputs(M, N, K, dtype, 1800 + 7 * si, kind)
            C = gc.run_gpu(plan, A, _given(name, B))
            r = gc.check_full(C, A, B, dtype, exact=(kind == "int"))
            assert r["ok"], (name, M, N, K, kind, r)
        epi = dict(out_dtype=dtype, bias=True, gelu=True, resid=True)
        plan = _plan(g, name, M, N, K, **epi)
        A, B = gc.inputs(M, N, K, dtype, 1850 + si)
        bias = synth.normal(1860 + si, (N,), 0.5, "f32")
        resid = synth.normal(1870 + si, (M, N), 1.0, dtype)
        C = gc.run_gpu(plan, A, _given(name, B), bias, resid)
        r = gc.check_full(C, A, B, dtype, dtype, bias, resid, None, True)
        assert r["ok"], (name, M, N, K, "epilogue", r)


@pytest.mark.parametrize("nk", [False, True])
def test_k1_unaligned_selected(g, nk):
    """4095 x 4097 x 63 (fp16, the odd-shape benchmark product) is planned on the
    register-load streaming kernel without copies or workspace; a batch of unaligned
    products and an operand off a 16-byte boundary inside a larger buffer run on the
    same configuration. Every element of the big product against the oracle."""
    M, N, K = 4095, 4097, 63
    plan = g.Plan(M, N, K, "f16", b_layout="nk" if nk else "kn")
    want = "m16s_f16_256x128x64_w4x2" + ("_nk" if nk else "") + "_u"
    say(f"[unaligned] {plan.describe()}")
    assert plan.config_name == want and plan.workspace_bytes == 0
    A, B = gc.inputs(M, N, K, "f16", 1880 + nk)
    Bg = B.t().contiguous() if nk else B
    C = gc.run_gpu(plan, A, Bg)
    r = gc.check_full(C, A, B, "f16")
    assert r["ok"], r
    # A two bytes past a 16-byte boundary: the same kernel, the same bits
    dev = torch.device("cuda")
    buf = torch.empty(M * K + 1, dtype=torch.float16, device=dev)
    Av = buf[1:].view(M, K)
    Av.copy_(A.to(dev))
    assert Av.data_ptr() % 16 == 2
    C2 = plan.run(Av, Bg.to(dev), out=torch.full((M, N), float("nan"), device=dev))
    torch.cuda.synchronize()
    assert torch.equal(C2.cpu().view(torch.int32), C.view(torch.int32))
    # a batch of 2 items with strides of odd element counts
    nb, M, N, K = 2, 2100, 2003, 45
    plan = g.Plan(M, N, K, "bf16", batch_hint=nb, b_layout="nk" if nk else "kn")
    assert plan.config_name == "m16s_bf16_256x128x64_w4x2" + ("_nk" if nk else "") + "_u"
    A = synth.uniform(1890, (nb, M, K), "bf16")
    B = synth.uniform(1891, (nb, K, N), "bf16")
    dev = torch.device("cuda")
    out = plan.run_batched(A.to(dev), (B.transpose(1, 2).contiguous() if nk else B).to(dev))
    torch.cuda.synchronize()
    out = out.cpu()
    for b in range(nb):
        r = gc.check_full(out[b], A[b], B[b], "bf16")
        assert r["ok"], (nk, b, r)


def test_k1_needs_one_slice(g):
    """K above 64 cannot run on a one-slice configuration: plan creation refuses it."""
    with pytest.raises(g.GemmError):
        g.Plan(128, 128, 72, "bf16", config=K1[0])
    with pytest.raises(g.GemmError):
        g.Plan(128, 128, 72, "bf16", config=[c for c in K1 if _nk(c)][0], b_layout="nk")


def test_k1_graph_replay(g):
    """The streaming kernel captured in a HIP graph and replayed, with eager work and
    a changed A between replays: every replay equals the eager result bit for bit."""
    name = [c for c in K1 if "_bf16_" in c and not _nk(c)][0]
    nb, M, N, K = 9, 300, 264, 64
    plan = g.Plan(M, N, K, "bf16", config=name, batch_hint=nb)
    dev = torch.device("cuda")
    As = [synth.uniform(1700 + i, (nb, M, K), "bf16").to(dev) for i in range(2)]
    B = synth.uniform(1702, (nb, K, N), "bf16").to(dev)
    eager = [plan.run_batched(A, B).clone() for A in As]
    torch.cuda.synchronize()
    A0 = As[0].clone()
    out = torch.empty((nb, M, N), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run_batched(A0, B, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run_batched(A0, B, out=out)
    junk = torch.randn(1 << 20, device=dev)
    for rep, i in enumerate((0, 1, 1, 0)):
        A0.copy_(As[i])
        out.fill_(float("nan"))
        graph.replay()
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager[i].view(torch.int32)), (rep, i)
