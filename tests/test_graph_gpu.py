"""Plans captured in a HIP graph (through torch's graph capture on the stream the
binding passes to gemm_run) and replayed: every replay must equal the eager
result bit for bit, including the split-K few-row path whose partial sums go
through the plan's workspace. Eager work and synchronisation run between the
replays, and the inputs change in place between them."""
from __future__ import annotations

import sys

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


CASES = [
    # (M, N, K, dtype, epilogue)
    (300, 264, 200, "bf16", dict(bias=True, gelu=True, out_dtype="bf16")),
    (1024, 1024, 512, "f32", dict()),
    (2, 1000, 3000, "bf16", dict(bias=True, out_dtype="f32")),  # few-row kernel, split K
    (1, 4096, 4096, "f16", dict()),
    (300, 261, 203, "f16", dict()),                     # padded copies of A and B, element-wise C
    (512, 512, 256, "bf16", dict(b_layout="nk")),       # B given transposed
    (200, 136, 77, "bf16", dict(b_layout="nk")),        # transposed B with padded copies
    (256, 256, 4096, "bf16", dict(bias=True, gelu=True, out_dtype="bf16",
                                  config="m16d_bf16_64x128x64_w2x2_a4_b4_r2")),  # split along K
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_graph_replay_matches_eager(g, case):
    M, N, K, dtype, epi = CASES[case]
    print(f"[graph] {M}x{N}x{K} {dtype} {epi}", file=sys.stderr, flush=True)
    plan = g.Plan(M, N, K, dtype, **epi)
    nk = epi.get("b_layout") == "nk"
    dev = torch.device("cuda")
    sets, Bref = [], []
    for seed in (901, 905, 909):
        A, B = gc.inputs(M, N, K, dtype, seed)
        Bref.append(B)
        bias = synth.normal(seed + 2, (N,), 0.5, "f32").to(dev) if epi.get("bias") else None
        sets.append((A.to(dev), (B.t().contiguous() if nk else B).to(dev), bias))
    eager = [plan.run(A, B, bias=b).clone() for A, B, b in sets]
    torch.cuda.synchronize()

    A0, B0, b0 = (t.clone() if t is not None else None for t in sets[0])
    out = torch.empty_like(eager[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run(A0, B0, bias=b0, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run(A0, B0, bias=b0, out=out)

    junk = torch.randn(1 << 20, device=dev)
    for rep, i in enumerate((0, 1, 2, 0, 2)):
        A, B, b = sets[i]
        A0.copy_(A)
        B0.copy_(B)
        if b is not None:
            b0.copy_(b)
        out.fill_(float("nan"))
        graph.replay()
        junk.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16 if out.element_size() == 2 else torch.int32),
                           eager[i].view(torch.int16 if out.element_size() == 2 else torch.int32)), \
            (case, rep, i, plan.describe())
    # the eager results themselves are right
    A, _, b = sets[0]
    r = gc.check_full(eager[0].cpu(), A.cpu(), Bref[0], dtype, epi.get("out_dtype", "f32"),
                      None if b is None else b.cpu(), gelu=epi.get("gelu", False))
    assert r["ok"], r


def test_graph_replay_attention_chain(g):
    """S = Q K^T, P = softmax(S), O = P V captured as one graph (three kernels on one
    stream, the softmax through gemm_softmax_rows) and replayed with Q changed in
    place between replays: every replay equals the eager chain bit for bit."""
    nb, Sq, D = 4, 256, 64
    dev = torch.device("cuda")
    Qs = [synth.normal(960 + i, (nb, Sq, D), 1.0, "bf16").to(dev) for i in range(3)]
    Kt = synth.normal(964, (nb, Sq, D), 1.0, "bf16").transpose(1, 2).contiguous().to(dev)
    V = synth.normal(965, (nb, Sq, D), 1.0, "bf16").to(dev)
    qk = g.Plan(Sq, Sq, D, "bf16", batch_hint=nb)
    pv = g.Plan(Sq, D, Sq, "bf16", batch_hint=nb)
    S = torch.empty((nb, Sq, Sq), dtype=torch.float32, device=dev)
    P = torch.empty((nb, Sq, Sq), dtype=torch.bfloat16, device=dev)
    O = torch.empty((nb, Sq, D), dtype=torch.float32, device=dev)
    Q = Qs[0].clone()

    def chain():
        qk.run_batched(Q, Kt, out=S)
        g.softmax_rows(S, 1.0, "bf16", out=P)
        pv.run_batched(P, V, out=O)

    eager = []
    for q in Qs:
        Q.copy_(q)
        chain()
        eager.append(O.clone())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    for rep in range(5):
        Q.copy_(Qs[rep % 3])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, eager[rep % 3]), rep
