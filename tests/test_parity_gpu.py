"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (see ``oracle.check``): |C - ref| <= c (1e-4 |scale| s + 1e-6) per
element, plus half a 16-bit ulp for 16-bit outputs; small-integer inputs must
match exactly; the fp32 4096^3 SGEMM must also stay within 1e-3 absolute
(the SGEMM page, section 4.1).
"""
from __future__ import annotations

import re
import sys

import numpy as np
import pytest
import torch

import oracle
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
    # configuration names without importing the library at collection time
    try:
        import dense_gemm_15_amd as g
        return g.config_names()
    except Exception:
        return []


def _dtype_of(name):
    """Input type a configuration reads, from its name (f32 kernels start with f32)."""
    if "bf16" in name:
        return "bf16"
    if "_f16" in name:
        return "f16"
    if name.startswith("f32") or "_f32" in name:
        return "f32"
    raise ValueError(f"no input type in configuration name {name}")


CONFIGS = _configs()
TILE_CONFIGS = [c for c in CONFIGS if not c.startswith(("gemv", "m16n", "m16s"))
                and not c.endswith("_nk") and "acc16" not in c]
NT_CONFIGS = [c for c in CONFIGS if c.startswith("m16n") or (c.startswith(("m16w", "f32d")) and c.endswith("_nk"))]
GEMV_CONFIGS = [c for c in CONFIGS if c.startswith("gemv")]


@pytest.mark.parametrize("name", TILE_CONFIGS)
def test_each_config_ragged(g, name):
    """Every compiled configuration on shapes spanning several tiles with ragged tails."""
    dtype = _dtype_of(name)
    idx = g.config_index(name)
    vec = "scalar" not in name and not name.startswith(("simple", "ladder"))
    parts = name.split("_")
    tile = [p for p in parts if "x" in p and p[0].isdigit()][0] if not name.startswith("simple") \
        else "64x64"
    dims = list(map(int, tile.split("x")))
    bm, bn = dims[0], dims[1]
    bk = dims[2] if len(dims) > 2 else (32 if dtype == "f32" and not name.startswith("simple")
                                        else 64)
    align = 4 if dtype == "f32" else 8
    shapes = [(2 * bm + 3, bn + align, 2 * bk + align), (bm, bn, bk), (1, align, align)]
    if not vec:
        shapes += [(2 * bm + 3, bn + 5, 2 * bk + 7), (1, 1, 1), (5, 3, 2)]
    for si, (M, N, K) in enumerate(shapes):
        say(f"[{name}] M={M} N={N} K={K}")
        plan = g.Plan(M, N, K, dtype, config=idx)
        assert plan.config_name == name
        for kind in ("uniform", "int"):
            A, B = gc.inputs(M, N, K, dtype, 1000 + 17 * si, kind)
            C = gc.run_gpu(plan, A, B)
            r = gc.check_full(C, A, B, dtype, exact=(kind == "int"))
            assert r["ok"], (name, M, N, K, kind, r)


def _describe(plan):
    return dict(kv.split("=", 1) for kv in plan.describe().split())


@pytest.mark.parametrize("name", GEMV_CONFIGS)
def test_gemv_config(g, name):
    """Few-row split-K kernel: M from 1 to its row limit, N with a ragged last
    strip of 128 columns, K from 1 to several K slices (split 1 and split > 1).
    Every plan runs twice: the second run reuses the plan's workspace."""
    dtype = _dtype_of(name)
    mr = int(re.search(r"_m(\d+)", name).group(1))
    idx = g.config_index(name)
    align = 4 if dtype == "f32" else 8
    kmax = {1: 4096, 4: 1024, 8: 512}[mr]
    cases = [(1, align, 1), (mr, 128 + 3 * align, 200), (max(1, mr - 1), 1000, 3 * kmax + 5),
             (mr, 136, 40000 if mr == 1 else 9000)]
    splits = set()
    for si, (M, N, K) in enumerate(cases):
        say(f"[{name}] M={M} N={N} K={K}")
        plan = g.Plan(M, N, K, dtype, config=idx)
        d = _describe(plan)
        assert d["config"] == name
        splits.add(int(d["split"]) > 1)
        for kind in ("uniform", "int"):
            A, B = gc.inputs(M, N, K, dtype, 2000 + 31 * si, kind)
            for rep in range(2):
                C = gc.run_gpu(plan, A, B)
                r = gc.check_full(C, A, B, dtype, exact=(kind == "int"))
                assert r["ok"], (name, M, N, K, kind, rep, d, r)
    assert splits == {False, True}


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_gemv_epilogue_and_batch(g, dtype):
    """Few-row kernel with every epilogue stage and 16-bit output, then a
    strided batch (batch items reuse the plan's workspace in stream order)."""
    M, N, K = 3, 264, 2500
    plan = g.Plan(M, N, K, dtype, bias=True, gelu=True, resid=True, scale=0.5,
                  out_dtype="bf16")
    d = _describe(plan)
    say(f"[gemv-epi] {dtype} {plan.describe()}")
    assert d["config"].startswith("gemv") and int(d["split"]) > 1
    A, B = gc.inputs(M, N, K, dtype, 611)
    bias = synth.normal(612, (N,), 0.5, "f32")
    resid = synth.uniform(613, (M, N), "bf16")
    C = gc.run_gpu(plan, A, B, bias, resid)
    r = gc.check_full(C, A, B, dtype, "bf16", bias, resid, 0.5, True)
    assert r["ok"], r

    nb = 3
    bplan = g.Plan(M, N, K, dtype, batch_hint=nb)
    assert _describe(bplan)["config"].startswith("gemv")
    As = torch.stack([gc.inputs(M, N, K, dtype, 620 + 2 * b)[0] for b in range(nb)])
    Bs = torch.stack([gc.inputs(M, N, K, dtype, 620 + 2 * b)[1] for b in range(nb)])
    dev = torch.device("cuda")
    Cs = bplan.run_batched(As.to(dev), Bs.to(dev))
    torch.cuda.synchronize()
    Cs = Cs.cpu()
    for b in range(nb):
        r = gc.check_full(Cs[b], As[b], Bs[b], dtype)
        assert r["ok"], (b, r)


def test_ladder_fp16_accumulation_exact(g):
    """The fp16-accumulating rung of the optimisation ladder equals the oracle's
    fp16-accumulation mode bit for bit (one RNE to fp16 per k of acc + a*b) on
    inputs of the 2^-10 grid, on shapes spanning several 64x64 tiles with ragged
    edges, also strided-batched."""
    name = "ladder_v3acc16_f16_64x64x16"
    for si, (M, N, K) in enumerate([(130, 70, 300), (64, 64, 16), (1, 3, 1000)]):
        say(f"[{name}] M={M} N={N} K={K}")
        A = synth.grid(900 + si, (M, K), "f16")
        B = synth.grid(910 + si, (K, N), "f16")
        plan = g.Plan(M, N, K, "f16", config=name)
        C = gc.run_gpu(plan, A, B).double().numpy()
        ref = oracle.gemm_f16acc(synth.bits(A), synth.bits(B))
        assert np.array_equal(C, ref), (M, N, K, np.abs(C - ref).max())
    M, N, K, nb = 70, 90, 130, 3
    As = torch.stack([synth.grid(920 + b, (M, K), "f16") for b in range(nb)])
    Bs = torch.stack([synth.grid(930 + b, (K, N), "f16") for b in range(nb)])
    plan = g.Plan(M, N, K, "f16", config=name, batch_hint=nb)
    dev = torch.device("cuda")
    Cs = plan.run_batched(As.to(dev), Bs.to(dev))
    torch.cuda.synchronize()
    for b in range(nb):
        ref = oracle.gemm_f16acc(synth.bits(As[b]), synth.bits(Bs[b]))
        assert np.array_equal(Cs[b].cpu().double().numpy(), ref), b


def test_accumulation_error_study(g):
    """DeepGEMM page, section 3.4: the same random fp16 inputs through the fp32- and
    the fp16-accumulating rung; against the fp64 product the fp16 accumulator's
    maximum absolute error is orders of magnitude larger (here: > 100x), while the
    fp32 one is within the parity tolerance."""
    M, N, K = 256, 192, 4096
    A, B = gc.inputs(M, N, K, "f16", 940)
    ref, s = oracle.gemm(synth.bits(A), synth.bits(B), "f16")
    errs = {}
    for name in ("ladder_v3_f16_64x64x16", "ladder_v3acc16_f16_64x64x16"):
        C = gc.run_gpu(g.Plan(M, N, K, "f16", config=name), A, B).double().numpy()
        errs[name] = np.abs(C - ref).max()
        if "acc16" not in name:
            r = oracle.check(C.astype(np.float32), ref, s, "f32")
            assert r["ok"], r
    say(f"[accumulation] max abs error fp32-acc {errs['ladder_v3_f16_64x64x16']:.3e}, "
        f"fp16-acc {errs['ladder_v3acc16_f16_64x64x16']:.3e}")
    assert errs["ladder_v3acc16_f16_64x64x16"] > 100 * errs["ladder_v3_f16_64x64x16"]


def test_ladder_never_chosen_automatically(g):
    """The ladder rungs run only when forced by name."""
    for M, N, K in [(4096, 4096, 4096), (127, 1000, 771), (1, 3, 5), (300, 264, 200)]:
        for dt in ("f16", "bf16", "f32"):
            assert not g.Plan(M, N, K, dt).config_name.startswith("ladder")


EPI_CASES = [
    dict(bias=True),
    dict(bias=True, gelu=True),
    dict(bias=True, resid=True),
    dict(scale=0.125),
    dict(scale=0.5, bias=True, gelu=True, resid=True),
    dict(gelu=True, resid=True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("epi", range(len(EPI_CASES)))
def test_epilogues(g, dtype, out_dtype, epi):
    """Fused epilogues on the automatically chosen kernel, every output type."""
    e = EPI_CASES[epi]
    M, N, K = 300, 264, 200
    say(f"[epi] {dtype}->{out_dtype} {e}")
    plan = g.Plan(M, N, K, dtype, out_dtype=out_dtype, **e)
    A, B = gc.inputs(M, N, K, dtype, 77)
    bias = synth.normal(78, (N,), 0.5, "f32") if e.get("bias") else None
    resid = synth.uniform(79, (M, N), out_dtype) if e.get("resid") else None
    C = gc.run_gpu(plan, A, B, bias, resid)
    r = gc.check_full(C, A, B, dtype, out_dtype, bias, resid, e.get("scale"), e.get("gelu", False))
    assert r["ok"], (dtype, out_dtype, e, plan.describe(), r)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gelu_accuracy(g, dtype):
    """The device GELU against the oracle's exact-erf GELU: C = gelu(A x 1) with
    K = 1 puts every value of A through the epilogue unchanged. The device uses a
    published erfc approximation (relative error below 1.2e-7); the bound allows
    1.5e-7 |v| plus four fp32 ulps of the result."""
    import oracle
    vals = np.concatenate([np.linspace(-12, 12, 4001), [0.0, 1e-30, -1e-30, 1e-6, -1e-6, 0.5,
                                                       -0.5, 3.0, -3.0, 5.5, -5.5, 9.0, -9.0]])
    M, N, K = len(vals), 8, 1
    A = torch.tensor(vals, dtype=torch.float32).reshape(M, 1).to(gc.TORCH[dtype])
    B = torch.ones(K, N, dtype=gc.TORCH[dtype])
    plan = g.Plan(M, N, K, dtype, gelu=True)
    say(f"[gelu] {dtype} {plan.describe()}")
    C = gc.run_gpu(plan, A, B).double().numpy()
    v = A.double().numpy()[:, 0]
    ref = np.array([oracle.gelu(x) for x in v])
    bound = 1.5e-7 * np.abs(v) + 4 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    err = np.abs(C - ref[:, None])
    worst = int(np.argmax((err - bound[:, None]).max(axis=1)))
    assert (err <= bound[:, None]).all(), (v[worst], C[worst, 0], ref[worst], bound[worst])


def test_workload_fp16_512(g):
    """FP16 512^3, fp32 out: every element against the oracle."""
    A, B = synth.gemm_inputs("fp16_512")
    plan = g.Plan(512, 512, 512, "f16")
    say("[fp16_512]", plan.describe())
    C = gc.run_gpu(plan, A, B)
    r = gc.check_full(C, A, B, "f16")
    assert r["ok"], r


@pytest.mark.parametrize("name", ["bf16_4096", "fp16_4096", "fp32_4096"])
def test_workload_square_4096(g, name):
    """4096^3 at the benchmark's launch configuration: every one of the 16.8M outputs
    against the oracle's fp64 product; the fp32 SGEMM also within 1e-3 absolute over
    all outputs (the SGEMM page, section 4.1)."""
    w = synth.WORKLOADS[name]
    A, B = synth.gemm_inputs(name)
    plan = g.Plan(4096, 4096, 4096, w["dtype"])
    say(f"[{name}]", plan.describe())
    C = gc.run_gpu(plan, A, B)
    r = gc.check_full(C, A, B, w["dtype"], abs_max=1e-3 if w["dtype"] == "f32" else None)
    say(f"[{name}] max err/tol {r['max_ratio']:.3f} max abs {r['max_abs']:.3e}")
    assert r["ok"], r

@pytest.mark.parametrize("shape,dtype,config", [
    ((3000, 3000, 9000), "bf16", "m16w_bf16_256x256x32_r4"),
    ((3072, 3072, 5000), "f16", "m16w_f16_256x256x32_r4"),
    ((4000, 3000, 2056), "f16", "m16t_f16_256x256x64_w2x4_a3_b2"),
])
def test_cost_model_choices(g, shape, dtype, config):
    """Large products outside the shape table, on the configuration the cost model
    picks (the one-wave-per-SIMD kernel for a long K, m16t's 256 x 256 tile below K of
    about 4096), with ragged M, N or K: sampled outputs (random, corners, tile edges)
    against the oracle, for uniform inputs and, bit-exact, small integers."""
    M, N, K = shape
    plan = g.Plan(M, N, K, dtype)
    say(f"[{shape} {dtype}]", plan.describe())
    assert plan.config_name == config
    rows, cols = gc.sample_indices(M, N, 2000, 11)
    for kind in ("uniform", "int"):
        A, B = gc.inputs(M, N, K, dtype, 4100 + K, kind)
        C = gc.run_gpu(plan, A, B)
        r = gc.check_sampled(C, A, B, dtype, rows, cols, exact=(kind == "int"))
        assert r["ok"], (shape, dtype, kind, r)


@pytest.mark.parametrize("name", ["longk_256x256x4096", "longk_64x4096x4096"])
def test_workload_long_k(g, name):
    """The long-K benchmark workloads at their launch configuration (split along K):
    256 x 256 x 4096 every element, 64 x 4096 x 4096 sampled elements (random,
    corners, tile edges), against the oracle."""
    w = synth.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    A, B = synth.gemm_inputs(name)
    plan = g.Plan(M, N, K, w["dtype"])
    say(f"[{name}]", plan.describe())
    assert int(_describe(plan)["split"]) > 1
    C = gc.run_gpu(plan, A, B)
    if M * N <= 65536:
        r = gc.check_full(C, A, B, w["dtype"])
    else:
        rows, cols = gc.sample_indices(M, N, 2000, 7)
        r = gc.check_sampled(C, A, B, w["dtype"], rows, cols)
    assert r["ok"], r


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_square_4096_integer_rowsums(g, dtype):
    """Small-integer 4096^3: sampled elements exact, and every row sum of C equals
    A (B 1) computed by the oracle (a property covering all 16.7M outputs)."""
    import oracle
    M = N = K = 4096
    A = synth.small_int(61, (M, K), dtype)
    B = synth.small_int(62, (K, N), dtype)
    plan = g.Plan(M, N, K, dtype)
    C = gc.run_gpu(plan, A, B)
    rows, cols = gc.sample_indices(M, N, 2000, 6)
    r = gc.check_sampled(C, A, B, dtype, rows, cols, exact=True)
    assert r["ok"], r
    Bones = synth.bits(B).astype(np.float64) if dtype == "f32" else oracle.decode(dtype, synth.bits(B))
    bsum = Bones.sum(axis=1)  # exact: integers below 2^53
    # A (B 1) through the oracle: a K x 1 right operand of the row sums
    bcol = torch.from_numpy(bsum.astype(np.float32)).reshape(K, 1)
    ref, _ = oracle.gemm(synth.bits(A.float()), synth.bits(bcol), "f32")
    got = C.double().numpy().sum(axis=1)
    assert np.array_equal(got, ref[:, 0]), np.abs(got - ref[:, 0]).max()


def test_workload_ffn(g):
    """Encoder FFN: H = GELU(X W1 + b1) in bf16, Y = H W2 + b2 + X in bf16, every
    element. Stage-wise: GEMM1 against the oracle, GEMM2 against the oracle fed the
    GPU's own H. End to end: against the all-oracle chain (the oracle's H rounded to
    bf16, then GEMM2), Y within the GEMM2 bound plus sum_k |dH_mk w2_kn| for the
    differences dH between the GPU's H and the oracle's (each within GEMM1's bound,
    checked above; near zero that is many bf16 ulps of H, so no ulp count is
    assumed)."""
    import oracle
    X, W1, b1, W2, b2 = synth.ffn_inputs()
    T, Hd, F = X.shape[0], X.shape[1], W1.shape[1]
    p1 = g.Plan(T, F, Hd, "bf16", bias=True, gelu=True, out_dtype="bf16")
    p2 = g.Plan(T, Hd, F, "bf16", bias=True, resid=True, out_dtype="bf16")
    say("[ffn1]", p1.describe())
    say("[ffn2]", p2.describe())
    dev = torch.device("cuda")
    Xd = X.to(dev)
    H = gc.nan_out((T, F), "bf16")
    Y = gc.nan_out((T, Hd), "bf16")
    p1.run(Xd, W1.to(dev), bias=b1.to(dev), out=H)
    p2.run(H, W2.to(dev), bias=b2.to(dev), resid=Xd, out=Y)
    torch.cuda.synchronize()
    H, Y = H.cpu(), Y.cpu()
    fl1 = oracle.BIAS | oracle.GELU
    ref1, s1 = oracle.gemm(synth.bits(X), synth.bits(W1), "bf16", fl1, 1.0, b1.numpy())
    r = oracle.check(synth.bits(H), ref1, s1, "bf16", fl1)
    say(f"[ffn1] max err/tol {r['max_ratio']:.3f}")
    assert r["ok"], ("ffn1", r)
    r = gc.check_full(Y, H, W2, "bf16", "bf16", bias=b2, resid=X)
    say(f"[ffn2 stage] max err/tol {r['max_ratio']:.3f}")
    assert r["ok"], ("ffn2", r)
    # the all-oracle chain
    h_ref_bits = oracle.round16("bf16", ref1)
    h_ref = oracle.decode("bf16", h_ref_bits)
    h_gpu = oracle.decode("bf16", synth.bits(H))
    dh = np.abs(h_gpu - h_ref)
    ulps = dh / oracle.ulp16("bf16", np.abs(h_ref))
    fl2 = oracle.BIAS | oracle.RESID
    ref2, s2 = oracle.gemm(h_ref_bits, synth.bits(W2), "bf16", fl2, 1.0, b2.numpy(),
                           synth.bits(X), "bf16")
    w2 = np.abs(oracle.decode("bf16", synth.bits(W2)))
    carry = dh @ w2  # sum_k |dH_mk| |w2_kn|, exact enough in fp64 for a bound
    tol = 1e-4 * s2 + 1e-6 + carry
    tol = tol + 0.5 * oracle.ulp16("bf16", np.abs(ref2) + tol)
    y = oracle.decode("bf16", synth.bits(Y))
    ratio = np.abs(y - ref2) / tol
    say(f"[ffn chain] max err/tol {ratio.max():.3f}, H elements differing "
        f"{int((dh > 0).sum())} of {dh.size}, {int((ulps > 1).sum())} by more than one ulp "
        f"(at most {ulps.max():.0f})")
    assert np.isfinite(y).all() and (ratio <= 1.0).all(), float(ratio.max())


def test_workload_qk_batched(g):
    """96 attention-score GEMMs 512 x 512 x 64 in one strided-batched call; every
    element of every head against the oracle."""
    import oracle
    Q, Kt = synth.qk_inputs()
    nb, S, D = Q.shape
    plan = g.Plan(S, S, D, "bf16", batch_hint=nb)
    say("[qk]", plan.describe())
    dev = torch.device("cuda")
    Sc = plan.run_batched(Q.to(dev), Kt.to(dev))
    torch.cuda.synchronize()
    Sc = Sc.cpu()
    for b in range(nb):
        ref, s = oracle.gemm(synth.bits(Q[b]), synth.bits(Kt[b]), "bf16")
        r = oracle.check(synth.bits(Sc[b]), ref, s)
        assert r["ok"], (b, r)


@pytest.mark.parametrize("name", ["gemv_1x4096x4096", "odd_127x1000x771", "odd_4095x4097x63"])
def test_workload_odd_shapes(g, name):
    """M = 1, and shapes with ragged, unaligned rows: every element."""
    w = synth.WORKLOADS[name]
    A, B = synth.gemm_inputs(name)
    plan = g.Plan(w["M"], w["N"], w["K"], w["dtype"])
    say(f"[{name}]", plan.describe())
    C = gc.run_gpu(plan, A, B)
    r = gc.check_full(C, A, B, w["dtype"])
    assert r["ok"], r


def _run_nt(plan, A, B, bias=None, resid=None, batched=False):
    """Run a transposed-B plan: the kernel gets Bt = B^T (contiguous); the oracle
    keeps using B."""
    dev = torch.device("cuda")
    Bt = B.transpose(-1, -2).contiguous()
    fn = plan.run_batched if batched else plan.run
    out = fn(A.to(dev), Bt.to(dev), None if bias is None else bias.to(dev),
             None if resid is None else resid.to(dev))
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("name", NT_CONFIGS)
def test_each_nt_config_ragged(g, name):
    """Every transposed-B configuration (B given as Bt [N x K]) on shapes spanning
    several tiles with ragged M/N/K tails, the exact tile size and one row."""
    dtype = _dtype_of(name)
    idx = g.config_index(name)
    dims = list(map(int, [p for p in name.split("_") if "x" in p and p[0].isdigit()][0].split("x")))
    bm, bn, bk = dims
    shapes = [(2 * bm + 3, bn + 8, 2 * bk + 8), (bm, bn, bk), (1, 8, 8), (bm + 5, 2 * bn + 3, 3 * bk)]
    for si, (M, N, K) in enumerate(shapes):
        say(f"[{name}] M={M} N={N} K={K}")
        plan = g.Plan(M, N, K, dtype, config=idx, b_layout="nk")
        assert plan.config_name == name
        for kind in ("uniform", "int"):
            A, B = gc.inputs(M, N, K, dtype, 3000 + 17 * si, kind)
            C = _run_nt(plan, A, B)
            r = gc.check_full(C, A, B, dtype, exact=(kind == "int"))
            assert r["ok"], (name, M, N, K, kind, r)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_nt_epilogue_packed_and_errors(g, dtype):
    """Transposed B with bias + GELU to 16-bit output, with residual, with K not a
    multiple of 8 (A and Bt copied into padded rows), and the alignment error."""
    cases = [(300, 264, 200, dict(bias=True, gelu=True, out_dtype="bf16"), 0),
             (257, 130, 192, dict(bias=True, resid=True, out_dtype=dtype), 0),
             (200, 136, 77, dict(), 3)]
    for ci, (M, N, K, epi, packed) in enumerate(cases):
        plan = g.Plan(M, N, K, dtype, b_layout="nk", **epi)
        d = _describe(plan)
        say(f"[nt] {plan.describe()}")
        assert d["b"] == "nk" and int(d["packed"]) == packed
        A, B = gc.inputs(M, N, K, dtype, 810 + ci)
        od = epi.get("out_dtype", "f32")
        bias = synth.normal(820 + ci, (N,), 0.5, "f32") if epi.get("bias") else None
        resid = synth.uniform(830 + ci, (M, N), od) if epi.get("resid") else None
        C = _run_nt(plan, A, B, bias, resid)
        r = gc.check_full(C, A, B, dtype, od, bias, resid, None, epi.get("gelu", False))
        assert r["ok"], (ci, r)
    # an operand off a 16-byte boundary: transposed B has no scalar-load kernel
    import ctypes
    M, N, K = 64, 64, 64
    plan = g.Plan(M, N, K, dtype, b_layout="nk")
    dev = torch.device("cuda")
    buf = torch.zeros(M * K + 8, dtype=gc.TORCH[dtype], device=dev)
    C = torch.empty(M, N, device=dev)
    rc = g.lib.gemm_run(plan._h, ctypes.c_void_p(buf.data_ptr() + 2), ctypes.c_void_p(buf.data_ptr()),
                        None, None, ctypes.c_void_p(C.data_ptr()), None)
    assert rc == -4


def test_workload_qk_nt(g):
    """96 attention-score GEMMs with K as stored ([S x D] per head, no transposed
    copy): C = Q K^T through a transposed-B plan, every element of every head."""
    import oracle
    Q, Kt = synth.qk_inputs()
    Kmat = Kt.transpose(1, 2).contiguous()  # [96 x 512 x 64]
    nb, S, D = Q.shape
    plan = g.Plan(S, S, D, "bf16", batch_hint=nb, b_layout="nk")
    say("[qk-nt]", plan.describe())
    dev = torch.device("cuda")
    Sc = plan.run_batched(Q.to(dev), Kmat.to(dev))
    torch.cuda.synchronize()
    Sc = Sc.cpu()
    for b in range(nb):
        ref, s = oracle.gemm(synth.bits(Q[b]), synth.bits(Kt[b]), "bf16")
        r = oracle.check(synth.bits(Sc[b]), ref, s)
        assert r["ok"], (b, r)


PACKED_CASES = [
    # (M, N, K, dtype, out_dtype, epilogue, expected packed bits)
    (300, 264, 203, "bf16", "f32", dict(), 1),                        # A rows unaligned
    (300, 261, 200, "f16", "f32", dict(), 2),                         # B (and C) rows unaligned
    (517, 1003, 77, "bf16", "bf16", dict(bias=True, resid=True), 3),  # both, 16-bit C, residual
    (257, 777, 130, "f16", "f16", dict(bias=True, gelu=True), 3),
    # even N that is not a multiple of 8: 16-bit C stored two columns per lane
    (300, 266, 200, "bf16", "bf16", dict(bias=True, resid=True), 2),
    (129, 1002, 64, "f16", "f16", dict(), 2),
]


@pytest.mark.parametrize("case", range(len(PACKED_CASES)))
def test_packed_operands(g, case):
    """16-bit operands whose rows are not 16-byte multiples are copied into
    zero-padded rows and run through a 16-byte-load kernel; C rows that are not
    16-byte multiples are stored one or two elements per lane. Every element, float and
    small-integer inputs, two runs of the same plan."""
    M, N, K, dtype, out_dtype, epi, bits = PACKED_CASES[case]
    plan = g.Plan(M, N, K, dtype, out_dtype=out_dtype, **epi)
    d = _describe(plan)
    say(f"[packed] {plan.describe()}")
    assert int(d["packed"]) == bits and d["config"].startswith(("m16d", "m16t"))
    for kind in ("uniform", "int"):
        A, B = gc.inputs(M, N, K, dtype, 700 + case, kind)
        bias = synth.normal(710 + case, (N,), 0.5, "f32") if epi.get("bias") else None
        resid = synth.uniform(720 + case, (M, N), out_dtype) if epi.get("resid") else None
        for rep in range(2):
            C = gc.run_gpu(plan, A, B, bias, resid)
            # integer inputs are exact only without the non-integer epilogue terms
            r = gc.check_full(C, A, B, dtype, out_dtype, bias, resid, None, epi.get("gelu", False),
                              exact=(kind == "int" and not epi))
            assert r["ok"], (kind, rep, plan.describe(), r)


@pytest.mark.parametrize("name", ["m16t_bf16_64x128x64_w2x2_a3_b3", "m16t_bf16_128x128x64_w2x2_a2_b2",
                                  "m16d_bf16_64x128x64_w2x2_a4_b4_r2", "m16n_bf16_64x128x64_w2x2_a3_b3"])
@pytest.mark.parametrize("shape,nb", [((200, 136, 96), 8), ((200, 136, 96), 12), ((130, 120, 72), 5),
                                      ((130, 120, 72), 8), ((70, 248, 40), 17)])
def test_batched_grid_order(g, name, shape, nb):
    """Batched grids in both workgroup orders: item by item with a contiguous share per
    XCD when the workgroups divide by 8 (8 and 12 items of 8 tiles, 8 items of 3 tiles
    on 64 x 128), tile-major otherwise (5 items of 3 tiles); ragged M, N and K; every
    element of every item against the oracle."""
    M, N, K = shape
    nk = name.startswith("m16n")
    plan = g.Plan(M, N, K, "bf16", config=name, batch_hint=nb, b_layout="nk" if nk else "kn")
    say(f"[{name}] {nb} x {M}x{N}x{K}")
    As = torch.stack([gc.inputs(M, N, K, "bf16", 1800 + 2 * b)[0] for b in range(nb)])
    Bs = torch.stack([gc.inputs(M, N, K, "bf16", 1800 + 2 * b)[1] for b in range(nb)])
    if nk:
        Cs = _run_nt(plan, As, Bs, batched=True)
    else:
        dev = torch.device("cuda")
        Cs = plan.run_batched(As.to(dev), Bs.to(dev))
        torch.cuda.synchronize()
        Cs = Cs.cpu()
    for b in range(nb):
        r = gc.check_full(Cs[b], As[b], Bs[b], "bf16")
        assert r["ok"], (name, shape, nb, b, r)


def test_packed_batched_and_misaligned(g):
    """A strided batch through the padded copies (one item at a time), and an
    operand that is not copied but starts off a 16-byte boundary: the plan then
    takes its scalar fallback."""
    M, N, K, nb = 200, 136, 77, 3
    plan = g.Plan(M, N, K, "bf16", batch_hint=nb)
    assert int(_describe(plan)["packed"]) == 1
    As = torch.stack([gc.inputs(M, N, K, "bf16", 730 + 2 * b)[0] for b in range(nb)])
    Bs = torch.stack([gc.inputs(M, N, K, "bf16", 730 + 2 * b)[1] for b in range(nb)])
    dev = torch.device("cuda")
    Cs = plan.run_batched(As.to(dev), Bs.to(dev))
    torch.cuda.synchronize()
    for b in range(nb):
        r = gc.check_full(Cs[b].cpu(), As[b], Bs[b], "bf16")
        assert r["ok"], (b, r)
    # B (rows aligned, not copied) one element past a 16-byte boundary
    A, B = As[0], Bs[0]
    Bbuf = torch.empty(K * N + 1, dtype=torch.bfloat16, device=dev)
    Bbuf[1:] = B.reshape(-1).to(dev)
    C = plan.run(A.to(dev), Bbuf[1:].view(K, N))
    torch.cuda.synchronize()
    r = gc.check_full(C.cpu(), A, B, "bf16")
    assert r["ok"], r


def test_operands_past_2gib(g):
    """Maximum sizes: an A of exactly 2 GiB (bf16, 2^20 x 1024) and an fp32 C of 2 GiB
    (65536 x 8192) leave the kernels that address operands with 32-bit offsets; the
    64-bit-addressed ones must produce the same products. Sampled rows, including the
    last ones (past the 2 GiB mark), against the oracle."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(950)
    # A of 2^31 bytes
    M, N, K = 1 << 20, 64, 1024
    A = synth.device_uniform(951, (M, K), "bf16")
    B = synth.uniform(952, (K, N), "bf16")
    plan = g.Plan(M, N, K, "bf16")
    say(f"[2GiB A] {plan.describe()}")
    assert not plan.config_name.startswith(("m16d", "m16n", "m16t", "m16w", "f32d", "gemv"))
    C = plan.run(A, B.to(dev))
    torch.cuda.synchronize()
    rows = np.concatenate([rng.integers(0, M, 24), [M - 2, M - 1]])
    Ar = A[torch.from_numpy(rows).to(dev)].cpu()
    Cr = C[torch.from_numpy(rows).to(dev)].cpu()
    r = gc.check_full(Cr, Ar, B, "bf16")
    assert r["ok"], r
    del A, C
    torch.cuda.empty_cache()
    # fp32 C of 2^31 bytes
    M, N, K = 1 << 16, 1 << 13, 16
    A = synth.uniform(953, (M, K), "f32")
    B = synth.uniform(954, (K, N), "f32")
    plan = g.Plan(M, N, K, "f32")
    say(f"[2GiB C] {plan.describe()}")
    C = plan.run(A.to(dev), B.to(dev))
    torch.cuda.synchronize()
    rows = np.concatenate([rng.integers(0, M, 8), [M - 1]])
    Cr = C[torch.from_numpy(rows).to(dev)].cpu()
    r = gc.check_full(Cr, A[torch.from_numpy(rows)], B, "f32")
    assert r["ok"], r
    del C
    torch.cuda.empty_cache()


def test_wide_b_rows(g):
    """Row-major B rows of 2^24 - 8 and 2^24 bf16 elements with a short K: the first
    stays on the 32-bit-offset kernel (a 64-row slice of B spans just under 2 GiB of
    offsets, rows past K still out of range), the second goes to a 64-bit-addressed
    one. Sampled columns, including the last ones, against the oracle."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(960)
    M, K = 16, 16
    for N, fast in (((1 << 24) - 8, True), (1 << 24, False)):
        A = synth.uniform(961, (M, K), "bf16")
        B = synth.device_uniform(962, (K, N), "bf16")
        plan = g.Plan(M, N, K, "bf16")
        say(f"[wide B N={N}] {plan.describe()}")
        assert plan.config_name.startswith(("m16d", "m16t")) == fast, plan.config_name
        C = plan.run(A.to(dev), B)
        torch.cuda.synchronize()
        cols = torch.from_numpy(np.concatenate([rng.integers(0, N, 56), np.arange(N - 8, N)])).to(dev)
        r = gc.check_full(C[:, cols].cpu(), A, B[:, cols].cpu(), "bf16")
        assert r["ok"], (N, r)
        del B, C
        torch.cuda.empty_cache()


SPLIT_CASES = [
    # (M, N, K, dtype, epilogue, batch, expected split), on m16d_{t}_64x128x64_w2x2_a4_b4_r2
    (256, 256, 4096, "f16", dict(), 1, 8),
    (256, 256, 4096, "bf16", dict(bias=True, gelu=True, out_dtype="bf16"), 1, 8),
    (200, 296, 8192, "bf16", dict(resid=True, scale=0.5), 1, 16),
    (130, 136, 4096, "f16", dict(bias=True, out_dtype="f16"), 1, 8),
    (256, 256, 4096, "bf16", dict(bias=True), 3, 8),
    (512, 512, 512, "bf16", dict(), 1, 1),  # 8 K slices: faster whole
]


@pytest.mark.parametrize("case", range(len(SPLIT_CASES)))
def test_split_k_tiles(g, case):
    """Tile products with few tiles and a long K run split along K (the slices as
    the items of one strided batch into fp32 partials, then the reduction kernel
    adds them in slice order and applies the epilogue): every element against the
    oracle, float and small-integer inputs, batch items in turn on one workspace,
    each plan run twice; a short K stays whole."""
    M, N, K, dtype, epi, nb, split = SPLIT_CASES[case]
    cfg = f"m16d_{dtype}_64x128x64_w2x2_a4_b4_r2"
    out_dtype = epi.get("out_dtype", "f32")
    exact = not any(epi.get(f) for f in ("bias", "gelu", "resid"))  # integer sums stay exact
    plan = g.Plan(M, N, K, dtype, batch_hint=nb, config=cfg, **epi)
    d = _describe(plan)
    say(f"[split-K] {plan.describe()}")
    assert int(d["split"]) == split and d["config"].startswith("m16d"), d
    dev = torch.device("cuda")
    for kind in ("uniform", "int"):
        A = torch.stack([gc.inputs(M, N, K, dtype, 1800 + 10 * case + b, kind)[0] for b in range(nb)])
        B = torch.stack([gc.inputs(M, N, K, dtype, 1800 + 10 * case + b, kind)[1] for b in range(nb)])
        bias = synth.normal(1890 + case, (N,), 0.5, "f32") if epi.get("bias") else None
        resid = synth.normal(1895 + case, (nb, M, N), 1.0, out_dtype) if epi.get("resid") else None
        for rep in range(2):
            C = plan.run_batched(A.to(dev), B.to(dev), None if bias is None else bias.to(dev),
                                 None if resid is None else resid.to(dev))
            torch.cuda.synchronize()
            C = C.cpu()
            for b in range(nb):
                r = gc.check_full(C[b], A[b], B[b], dtype, out_dtype, bias,
                                  None if resid is None else resid[b], epi.get("scale"),
                                  epi.get("gelu", False), exact=exact and kind == "int")
                assert r["ok"], (case, kind, rep, b, r)


def test_repeat_shape_hits_cache(g):
    """A repeated shape is served from the exact-shape cache."""
    h0, m0, _ = g.cache_stats()
    g.Plan(333, 444, 555, "bf16")
    h1, m1, _ = g.cache_stats()
    g.Plan(333, 444, 555, "bf16")
    h2, m2, _ = g.cache_stats()
    assert m2 == m1 and h2 == h1 + 1


def test_unaligned_pointer_fallback(g):
    """A 16-bit operand offset by one element is not 16-byte aligned: the plan
    takes its scalar fallback and the result is still right."""
    M, N, K = 200, 136, 72
    A, B = gc.inputs(M, N, K, "bf16", 91)
    dev = torch.device("cuda")
    Abuf = torch.empty(M * K + 1, dtype=torch.bfloat16, device=dev)
    Abuf[1:] = A.reshape(-1).to(dev)
    Aoff = Abuf[1:].view(M, K)
    plan = g.Plan(M, N, K, "bf16")
    C = plan.run(Aoff, B.to(dev))
    torch.cuda.synchronize()
    r = gc.check_full(C.cpu(), A, B, "bf16")
    assert r["ok"], r


def test_errors_on_device(g):
    """Error paths that need a live device: NULL pointers and misalignment."""
    import ctypes
    plan = g.Plan(64, 64, 64, "f32", bias=True)
    dev = torch.device("cuda")
    A = torch.zeros(64, 64, device=dev)
    rc = g.lib.gemm_run(plan._h, ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(A.data_ptr()),
                        None, None, ctypes.c_void_p(A.data_ptr()), None)
    assert rc == -3  # bias flag set, bias NULL
    rc = g.lib.gemm_run(plan._h, ctypes.c_void_p(A.data_ptr() + 2), ctypes.c_void_p(A.data_ptr()),
                        ctypes.c_void_p(A.data_ptr()), None, ctypes.c_void_p(A.data_ptr()), None)
    assert rc == -4  # fp32 A not 4-byte aligned
    rc = g.lib.gemm_run(None, None, None, None, None, None, None)
    assert rc == -7


W_CONFIGS = [c for c in CONFIGS if c.startswith("m16w")]


@pytest.mark.parametrize("name", W_CONFIGS)
def test_epilogues_each_m16w(g, name):
    """The one-wave-per-SIMD kernels with every epilogue stage and output type:
    16-byte-aligned C rows with N % 8 == 0 (a lane's four columns in one vector
    store), and for B given transposed also N even but not a multiple of 8 and N odd
    (one element at a time); K with a ragged 32-deep tail. Every element."""
    dtype = _dtype_of(name)
    nk = name.endswith("_nk")
    cases = [(300, 264, 200, dict(bias=True, gelu=True, out_dtype="bf16")),
             (257, 136, 96, dict(bias=True, resid=True, out_dtype=dtype)),
             (130, 264, 64, dict(scale=0.5, resid=True, out_dtype="f32")),
             (70, 520, 40, dict(bias=True, out_dtype="f16"))]
    if nk:
        cases += [(130, 262, 64, dict(scale=0.5, resid=True, out_dtype="bf16")),
                  (70, 263, 40, dict(bias=True, gelu=True, out_dtype="f16")),
                  (99, 261, 72, dict(resid=True, out_dtype="f32"))]
    for ci, (M, N, K, epi) in enumerate(cases):
        plan = g.Plan(M, N, K, dtype, config=name, b_layout="nk" if nk else "kn", **epi)
        say(f"[{name}] {M}x{N}x{K} {epi}")
        A, B = gc.inputs(M, N, K, dtype, 1500 + ci)
        od = epi.get("out_dtype", "f32")
        bias = synth.normal(1510 + ci, (N,), 0.5, "f32") if epi.get("bias") else None
        resid = synth.uniform(1520 + ci, (M, N), od) if epi.get("resid") else None
        C = _run_nt(plan, A, B, bias, resid) if nk else gc.run_gpu(plan, A, B, bias, resid)
        r = gc.check_full(C, A, B, dtype, od, bias, resid, epi.get("scale"), epi.get("gelu", False))
        assert r["ok"], (name, M, N, K, epi, r)


WS_CASES = [
    # (M, N, K, dtype, epilogue): a tile product split along K (fp32 partial sums), A rows
    # not 16-byte multiples (padded copy of A), few rows with K split (partial sums)
    (256, 256, 4096, "bf16", dict(bias=True, gelu=True, out_dtype="bf16")),
    (300, 264, 203, "bf16", dict()),
    (3, 1000, 3000, "f16", dict(bias=True)),
]


@pytest.mark.parametrize("case", range(len(WS_CASES)))
def test_workspace_contract(g, case):
    """Plans own no device memory: a plan whose configuration needs scratch reports its
    size (gemm_plan_workspace_bytes) and runs on a caller-provided workspace
    (gemm_run_ws); without one it runs its workspace-free configuration. Both every
    element against the oracle; a workspace too small or off a 256-byte boundary is
    refused."""
    import ctypes
    M, N, K, dtype, epi = WS_CASES[case]
    plan = g.Plan(M, N, K, dtype, **epi)
    d = _describe(plan)
    n = plan.workspace_bytes
    say(f"[ws] {plan.describe()}")
    assert n > 0 and int(d["workspace"]) == n and d["nows"] != "none"
    od = epi.get("out_dtype", "f32")
    A, B = gc.inputs(M, N, K, dtype, 1600 + case)
    bias = synth.normal(1610 + case, (N,), 0.5, "f32") if epi.get("bias") else None
    for ws in (None, False):  # a torch-allocated workspace, then none
        C = gc.run_gpu(plan, A, B, bias, workspace=ws)
        r = gc.check_full(C, A, B, dtype, od, bias, None, None, epi.get("gelu", False))
        assert r["ok"], (ws, r)
    dev = torch.device("cuda")
    Ad, Bd = A.to(dev), B.to(dev)
    C = gc.nan_out((M, N), od)
    buf = torch.empty(n + 512, dtype=torch.uint8, device=dev)
    bp = ctypes.c_void_p(bias.to(dev).data_ptr()) if bias is not None else None
    small = g.lib.gemm_run_ws(plan._h, ctypes.c_void_p(Ad.data_ptr()), ctypes.c_void_p(Bd.data_ptr()),
                              bp, None, ctypes.c_void_p(C.data_ptr()), ctypes.c_void_p(buf.data_ptr()),
                              n - 1, None)
    off = g.lib.gemm_run_ws(plan._h, ctypes.c_void_p(Ad.data_ptr()), ctypes.c_void_p(Bd.data_ptr()),
                            bp, None, ctypes.c_void_p(C.data_ptr()),
                            ctypes.c_void_p(buf.data_ptr() + 16), n, None)
    torch.cuda.synchronize()
    assert (small, off) == (-11, -4)


def test_workspace_required_transposed_padded(g):
    """A transposed-B plan with padded operands has no workspace-free configuration."""
    plan = g.Plan(200, 136, 77, "bf16", b_layout="nk")
    assert plan.workspace_bytes > 0 and _describe(plan)["nows"] == "none"
    A, B = gc.inputs(200, 136, 77, "bf16", 1620)
    dev = torch.device("cuda")
    with pytest.raises(g.GemmError) as e:
        plan.run(A.to(dev), B.t().contiguous().to(dev), workspace=False)
    assert e.value.status == -11
    C = _run_nt(plan, A, B)
    r = gc.check_full(C, A, B, "bf16")
    assert r["ok"], r


F32_PADDED = [
    # (M, N, K, packed bits): fp32 rows that are not 16-byte multiples, products large
    # enough (2^27 multiply-adds, tiles for every CU) for the copies to repay
    (2050, 2051, 135, 3),
    (2048, 2051, 260, 2),
    (2050, 2048, 150, 1),
]


@pytest.mark.parametrize("case", range(len(F32_PADDED)))
def test_fp32_padded_copies(g, case):
    """fp32 operands whose rows are not 16-byte multiples (K or N not a multiple of 4)
    copied into zero-padded rows and run on f32d: float and small-integer inputs, every
    element, two runs of the plan; then bias + GELU + residual into bf16 C."""
    M, N, K, bits = F32_PADDED[case]
    plan = g.Plan(M, N, K, "f32")
    d = _describe(plan)
    say(f"[f32 padded] {plan.describe()}")
    assert d["config"].startswith("f32d_") and int(d["packed"]) == bits
    for kind in ("uniform", "int"):
        A, B = gc.inputs(M, N, K, "f32", 2300 + case, kind)
        for rep in range(2):
            C = gc.run_gpu(plan, A, B)
            r = gc.check_full(C, A, B, "f32", exact=(kind == "int"))
            assert r["ok"], (kind, rep, r)
    plan = g.Plan(M, N, K, "f32", bias=True, gelu=True, resid=True, out_dtype="bf16")
    assert int(_describe(plan)["packed"]) == bits
    A, B = gc.inputs(M, N, K, "f32", 2310 + case)
    bias = synth.normal(2320 + case, (N,), 0.5, "f32")
    resid = synth.uniform(2330 + case, (M, N), "bf16")
    C = gc.run_gpu(plan, A, B, bias, resid)
    r = gc.check_full(C, A, B, "f32", "bf16", bias, resid, None, True)
    assert r["ok"], r


def test_fp32_4097_cube(g):
    """4097^3 fp32 (no row a 16-byte multiple): both operands copied into padded rows
    and an f32d kernel on them; every one of the 16.8M outputs against the oracle,
    within 1e-3 absolute over all of them (the SGEMM page, section 4.1)."""
    n = 4097
    plan = g.Plan(n, n, n, "f32")
    d = _describe(plan)
    say(f"[f32 4097] {plan.describe()}")
    # the 4096 x 4096 block on the 256 x 256 kernel, the last row and column apart
    assert d["config"] == "f32d_256x256x16_w4x2_a3" and int(d["packed"]) == 3
    assert d["edge"] == "1,1"
    A = synth.uniform(2340, (n, n), "f32")
    B = synth.uniform(2341, (n, n), "f32")
    C = gc.run_gpu(plan, A, B)
    r = gc.check_full(C, A, B, "f32", abs_max=1e-3)
    say(f"[f32 4097] max err/tol {r['max_ratio']:.3f} max abs {r['max_abs']:.3e}")
    assert r["ok"], r


EDGES = [
    # (dtype, M, N, K, batch, epilogue, out, edge, packed): products a few rows / columns
    # past multiples of 256, the whole-tile block in full rounds of 256 x 256 tiles
    ("f32", 4100, 4100, 4100, 1, dict(), "f32", "4,4", 0),
    ("f32", 4096, 4097, 1024, 1, dict(bias=True, gelu=True, resid=True), "bf16", "0,1", 2),
    ("f32", 4099, 4096, 600, 2, dict(scale=0.5, bias=True), "f32", "3,0", 0),
    ("bf16", 4097, 4097, 4097, 1, dict(), "f32", "1,1", 3),
    ("f16", 4104, 4104, 1024, 1, dict(bias=True, gelu=True, resid=True), "f16", "8,8", 0),
    ("bf16", 4096, 4097, 2048, 2, dict(scale=0.5), "bf16", "0,1", 2),
    ("f16", 4099, 4096, 600, 1, dict(resid=True), "f32", "3,0", 0),
]


@pytest.mark.parametrize("case", range(len(EDGES)))
def test_thin_edges(g, case):
    """Thin edges split off: the whole-tile block on the 256 x 256 kernel of the input
    type (f32d, m16t), the last rows on the few-row kernel (partial sums in the
    workspace), the last columns on the few-column kernel; aligned and padded operands,
    every epilogue stage into 16-bit C (staged and register store forms), strided
    batches, and the same plan without a workspace (the whole product on a plain
    configuration). Every element against the oracle (fp32 also within 1e-3 absolute)."""
    dt, M, N, K, nb, epi, od, edge, bits = EDGES[case]
    plan = g.Plan(M, N, K, dt, out_dtype=od, batch_hint=nb, **epi)
    d = _describe(plan)
    say(f"[edges] {plan.describe()}")
    main = "f32d_256x256x16_w4x2_a3" if dt == "f32" else f"m16t_{dt}_256x256x64_w2x4_a3_b2"
    assert d["config"] == main and d["edge"] == edge
    assert int(d["packed"]) == bits
    dev = torch.device("cuda")
    As = torch.stack([synth.uniform(2400 + 2 * b, (M, K), dt) for b in range(nb)])
    Bs = torch.stack([synth.uniform(2401 + 2 * b, (K, N), dt) for b in range(nb)])
    bias = synth.normal(2420, (N,), 0.5, "f32") if epi.get("bias") else None
    resid = synth.uniform(2421, (M, N), od) if epi.get("resid") else None
    for ws in (None, False):
        if nb == 1:
            C = gc.run_gpu(plan, As[0], Bs[0], bias, resid, workspace=ws)[None]
        else:
            C = plan.run_batched(As.to(dev), Bs.to(dev), None if bias is None else bias.to(dev),
                                 out=gc.nan_out((nb, M, N), od), workspace=ws)
            torch.cuda.synchronize()
            C = C.cpu()
        for b in range(nb):
            r = gc.check_full(C[b], As[b], Bs[b], dt, od, bias, resid, epi.get("scale"),
                              epi.get("gelu", False),
                              abs_max=1e-3 if (dt, od) == ("f32", "f32") else None)
            assert r["ok"], (ws, b, r)


def test_fp32_transposed_b(g):
    """fp32 with B given transposed (Y = X W^T + b with fp32 weights [out, in]): the
    selected f32d *_nk plan on an aligned shape with bias + GELU, K not a multiple of
    4 (A and Bt copied into padded rows), a residual into fp32 C; every element."""
    cases = [(300, 264, 200, dict(bias=True, gelu=True), 0),
             (127, 1000, 771, dict(), 3),
             (257, 130, 203, dict(resid=True, scale=0.5), 3)]
    for ci, (M, N, K, epi, bits) in enumerate(cases):
        plan = g.Plan(M, N, K, "f32", b_layout="nk", **epi)
        d = _describe(plan)
        say(f"[f32 nt] {plan.describe()}")
        assert d["b"] == "nk" and d["config"].startswith("f32d_") and int(d["packed"]) == bits
        A, B = gc.inputs(M, N, K, "f32", 2350 + ci)
        bias = synth.normal(2360 + ci, (N,), 0.5, "f32") if epi.get("bias") else None
        resid = synth.uniform(2370 + ci, (M, N), "f32") if epi.get("resid") else None
        C = _run_nt(plan, A, B, bias, resid)
        r = gc.check_full(C, A, B, "f32", "f32", bias, resid, epi.get("scale"),
                          epi.get("gelu", False))
        assert r["ok"], (ci, r)


def test_workspace_two_streams(g):
    """One plan split along K and one with padded operand copies, each run on two
    streams at the same time with a workspace per stream, four rounds queued before any
    wait: every element of every output against the oracle."""
    dev = torch.device("cuda")
    specs = [(256, 256, 4096, "bf16", dict(bias=True, out_dtype="bf16")),
             (517, 1003, 77, "bf16", dict(bias=True, resid=True, out_dtype="bf16"))]
    plans = [g.Plan(M, N, K, dt, **e) for (M, N, K, dt, e) in specs]
    for p in plans:
        say(f"[ws2] {p.describe()}")
    assert int(_describe(plans[0])["split"]) > 1 and int(_describe(plans[1])["packed"]) == 3
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [[torch.empty(p.workspace_bytes, dtype=torch.uint8, device=dev) for _ in streams]
           for p in plans]
    jobs = []
    for rnd in range(4):
        for pi, (M, N, K, dt, e) in enumerate(specs):
            for si in range(2):
                seed = 1700 + 100 * pi + 10 * rnd + si
                A, B = gc.inputs(M, N, K, dt, seed)
                bias = synth.normal(seed + 5, (N,), 0.5, "f32")
                resid = synth.uniform(seed + 6, (M, N), "bf16") if e.get("resid") else None
                dA, dB, db = A.to(dev), B.to(dev), bias.to(dev)
                dr = resid.to(dev) if resid is not None else None
                C = gc.nan_out((M, N), "bf16")
                jobs.append((pi, si, A, B, bias, resid, dA, dB, db, dr, C))
    torch.cuda.synchronize()  # inputs in place before the streams start
    for (pi, si, A, B, bias, resid, dA, dB, db, dr, C) in jobs:
        s = streams[si]
        with torch.cuda.stream(s):
            plans[pi].run(dA, dB, bias=db, resid=dr, out=C, stream=s, workspace=wss[pi][si])
    torch.cuda.synchronize()
    for (pi, si, A, B, bias, resid, dA, dB, db, dr, C) in jobs:
        r = gc.check_full(C.cpu(), A, B, "bf16", "bf16", bias, resid)
        assert r["ok"], (pi, si, r)


M16S_UNALIGNED = [
    # (M, N, K, out_dtype, epilogue): K within one slice, rows not 16-byte multiples, large C
    (4099, 2048, 57, "bf16", dict(bias=True, resid=True)),   # A rows unaligned, 16-bit C
    (4099, 2050, 57, "bf16", dict(bias=True, gelu=True)),    # both, even N not % 8
    (4100, 2051, 60, "f32", dict(scale=0.5)),                # both, odd N, fp32 C
]


@pytest.mark.parametrize("case", range(len(M16S_UNALIGNED)))
def test_unaligned_streaming_kernel(g, case):
    """Rows that are not 16-byte multiples with K within one 64-deep slice and a large
    C: the streaming kernel's register-load form, no copies and no workspace (the
    configuration is asserted); bf16 inputs, 16-bit and fp32 C, every epilogue stage.
    Every element."""
    M, N, K, od, epi = M16S_UNALIGNED[case]
    plan = g.Plan(M, N, K, "bf16", out_dtype=od, **epi)
    d = _describe(plan)
    say(f"[m16s unaligned] {plan.describe()}")
    assert d["config"] == "m16s_bf16_256x128x64_w4x2_u" and int(d["packed"]) == 0
    assert plan.workspace_bytes == 0
    A, B = gc.inputs(M, N, K, "bf16", 1900 + case)
    bias = synth.normal(1910 + case, (N,), 0.5, "f32") if epi.get("bias") else None
    resid = synth.uniform(1920 + case, (M, N), od) if epi.get("resid") else None
    C = gc.run_gpu(plan, A, B, bias, resid)
    r = gc.check_full(C, A, B, "bf16", od, bias, resid, epi.get("scale"), epi.get("gelu", False))
    assert r["ok"], r


def test_poison_mode(g, monkeypatch):
    """GEMM15_POISON: every run first fills C with NaN (a debug aid for unwritten
    elements). Tile, split-K, few-row, padded-copy, streaming and batched runs with it on
    still produce every element, against the oracle; C starts as zeros here, so an
    element left as NaN can only come from the poison fill."""
    monkeypatch.setenv("GEMM15_POISON", "1")
    dev = torch.device("cuda")
    cases = [(300, 264, 200, "bf16", dict(bias=True, out_dtype="bf16")),
             (256, 256, 4096, "f16", dict()),
             (3, 1000, 3000, "bf16", dict(bias=True)),
             (300, 264, 203, "f16", dict(out_dtype="f16")),
             (4099, 2048, 57, "bf16", dict(out_dtype="f32"))]
    for ci, (M, N, K, dt, epi) in enumerate(cases):
        plan = g.Plan(M, N, K, dt, **epi)
        od = epi.get("out_dtype", "f32")
        A, B = gc.inputs(M, N, K, dt, 2000 + ci)
        bias = synth.normal(2010 + ci, (N,), 0.5, "f32") if epi.get("bias") else None
        C = torch.zeros((M, N), dtype=gc.TORCH[od], device=dev)
        plan.run(A.to(dev), B.to(dev), None if bias is None else bias.to(dev), out=C)
        torch.cuda.synchronize()
        r = gc.check_full(C.cpu(), A, B, dt, od, bias)
        assert r["ok"], (plan.describe(), r)
    Q, Kt = synth.qk_inputs()
    Q, Kt = Q[:5], Kt[:5]
    plan = g.Plan(512, 512, 64, "bf16", batch_hint=5)
    S = torch.zeros((5, 512, 512), device=dev)
    plan.run_batched(Q.to(dev), Kt.to(dev), out=S)
    torch.cuda.synchronize()
    for b in range(5):
        r = gc.check_full(S[b].cpu(), Q[b], Kt[b], "bf16")
        assert r["ok"], (b, r)


GELU_RANGE_CONFIGS = ["m16t_bf16_128x128x64_w2x2_a2_b2", "m16w_bf16_256x128x32_r6",
                      "m16d_bf16_64x128x64_w2x2_a4_b4_r2", "m16s_bf16_128x128x64_w2x2"]


@pytest.mark.parametrize("name", GELU_RANGE_CONFIGS)
@pytest.mark.parametrize("od", ["f32", "bf16", "f16"])
def test_gelu_epilogue_range(g, name, od):
    """The GELU epilogue over its whole range, on each epilogue form (per-launch variants
    with the 16-bit GELU, the one-wave-per-SIMD form, the one-body form): A and B carry
    one non-zero k column / row, so each pre-activation A[i,0] B[0,j] + bias[j] is exact
    in fp32 and they span about -19 .. 19 (far negative tail included). fp32 results
    within 5e-7 (|v| + |GELU|) of the oracle; 16-bit results equal to the oracle's
    rounded value in nearly every element and never more than one unit in the last
    place away from it (where that value is well inside the normal range)."""
    if name not in CONFIGS:
        pytest.skip(f"{name} not built")
    M, N, K = 300, 264, 16
    A = torch.zeros(M, K, dtype=torch.float32)
    A[:, 0] = 0.25 + (torch.arange(M) % 64).float() / 16
    B = torch.zeros(K, N, dtype=torch.float32)
    B[0, :] = torch.linspace(-4.5, 4.5, N)
    A, B = A.to(torch.bfloat16), B.to(torch.bfloat16)
    bias = synth.normal(1530, (N,), 0.1, "f32")
    plan = g.Plan(M, N, K, "bf16", config=name, bias=True, gelu=True, out_dtype=od)
    say(f"[{name}] GELU range -> {od}")
    C = gc.run_gpu(plan, A, B, bias)
    ref, _ = oracle.gemm(gc.to_bits(A), gc.to_bits(B), "bf16", oracle.BIAS | oracle.GELU, 1.0,
                         bias.numpy(), None, od)
    pre = A.float()[:, :1].double().numpy() * B.float()[:1, :].double().numpy() + bias.double().numpy()
    assert pre.min() < -15 and pre.max() > 15
    got = oracle.decode(od, gc.to_bits(C))
    assert np.all(np.isfinite(got)), name
    if od == "f32":
        err = np.abs(got - ref)
        assert np.all(err <= 5e-7 * (np.abs(pre) + np.abs(ref)) + 1e-37), (name, float(err.max()))
        return
    want = oracle.decode(od, oracle.round16(od, ref))
    # results near or below the output type's smallest normal come from fp32 intermediates
    # (Phi ~ |GELU| / |v|, the exponential) in or near fp32's subnormal range, which the
    # kernels' arithmetic does not keep: there, the result must be that tiny too
    tiny = 2.0 ** (-120 if od == "bf16" else -14)
    normal = np.abs(want) >= tiny
    assert np.all(np.abs(got[~normal]) <= tiny), (name, od)
    ulps = np.abs(got - want)[normal] / oracle.ulp16(od, np.abs(want[normal]))
    assert ulps.max() <= 1.0, (name, od, float(ulps.max()))
    exact = float(np.mean(got[normal] == want[normal]))
    assert exact >= (0.95 if od == "bf16" else 0.80), (name, od, exact)
