"""The allocation-free entry point gemm_run_noalloc (the library's own per-GPU scratch
instead of a caller workspace), through the C ABI: two calls in a row, the second with a
smaller input, each equal bit for bit to gemm_run_ws on the same plan and within the
oracle's bound; a plan that needs more scratch than the array holds is refused."""
from __future__ import annotations

import ctypes

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


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _case(g, M, N, K, dtype, epi, seed):
    dev = torch.device("cuda")
    plan = g.Plan(M, N, K, dtype, **epi)
    od = epi.get("out_dtype", "f32")
    A, B = gc.inputs(M, N, K, dtype, seed)
    bias = synth.normal(seed + 3, (N,), 0.5, "f32") if epi.get("bias") else None
    return dict(plan=plan, od=od, A=A, B=B, bias=bias, dA=A.to(dev), dB=B.to(dev),
                db=None if bias is None else bias.to(dev), epi=epi, dtype=dtype)


def _run_ws(g, c):
    ws = torch.empty(c["plan"].workspace_bytes, dtype=torch.uint8, device="cuda")
    C = gc.nan_out((c["plan"].M, c["plan"].N), c["od"])
    rc = g.lib.gemm_run_ws(c["plan"]._h, _vp(c["dA"]), _vp(c["dB"]), _vp(c["db"]), None, _vp(C),
                           _vp(ws), ws.numel(), None)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return C.cpu()


def _run_noalloc(g, c):
    C = gc.nan_out((c["plan"].M, c["plan"].N), c["od"])
    rc = g.lib.gemm_run_noalloc(c["plan"]._h, 1, _vp(c["dA"]), 0, _vp(c["dB"]), 0, _vp(c["db"]),
                                None, 0, _vp(C), 0, None)
    assert rc == 0, rc
    return C


PAIRS = [
    # plans split along K (fp32 partial sums in the scratch)
    ((256, 256, 4096, "bf16", dict(bias=True, gelu=True, out_dtype="bf16")),
     (130, 136, 4096, "f16", dict(bias=True, out_dtype="f16"))),
    # padded operand copies in the scratch (both operands, then A only)
    ((2000, 1003, 77, "f16", dict()), (300, 264, 203, "bf16", dict(bias=True))),
    # few rows, K split
    ((1, 4096, 4096, "f16", dict()), (3, 1000, 3000, "f16", dict(bias=True))),
]


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_workspace_run(g, pair):
    big, small = (_case(g, *spec, 1800 + 10 * pair + i) for i, spec in enumerate(PAIRS[pair]))
    for c in (big, small):
        assert 0 < c["plan"].workspace_bytes <= g.lib.gemm_noalloc_scratch_bytes()
        print(f"[noalloc] {c['plan'].describe()}", flush=True)
    got = [_run_noalloc(g, big), _run_noalloc(g, small)]  # two calls in a row, second smaller
    torch.cuda.synchronize()
    for c, C in zip((big, small), got):
        C = C.cpu()
        ref = _run_ws(g, c)
        assert torch.equal(C.view(torch.int16 if c["od"] != "f32" else torch.int32),
                           ref.view(torch.int16 if c["od"] != "f32" else torch.int32))
        r = gc.check_full(C, c["A"], c["B"], c["dtype"], c["od"], c["bias"], None, None,
                          c["epi"].get("gelu", False))
        assert r["ok"], r


def test_noalloc_refuses_oversized_plan(g):
    """A padded copy of a 16384 x 1008 bf16 A (33 MB) exceeds the 16 MiB array."""
    plan = g.Plan(16384, 512, 1001, "bf16")
    assert plan.workspace_bytes > g.lib.gemm_noalloc_scratch_bytes(), plan.describe()
    dev = torch.device("cuda")
    A = torch.zeros(16384, 1001, dtype=torch.bfloat16, device=dev)
    B = torch.zeros(1001, 512, dtype=torch.bfloat16, device=dev)
    C = torch.empty(16384, 512, device=dev)
    rc = g.lib.gemm_run_noalloc(plan._h, 1, _vp(A), 0, _vp(B), 0, None, None, 0, _vp(C), 0, None)
    assert rc == -11
    assert "workspace" in g.strerror(rc)
