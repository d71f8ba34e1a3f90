"""The C ABI on the host: exports, argument checking and configuration choice.

CPU only: nothing here launches a kernel. ``gemm_select`` runs the same
shape-bucket rules and exact-shape cache as plan creation against a described
device, so the dispatch logic is testable without a GPU.
"""
import ctypes
import os
import re

import pytest
import torch

import dense_gemm_15_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm15.h")
MI355X = dict(cu_count=256, lds_bytes=163840)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(g.lib, n), n
    assert set(names) == set(g.SIGNATURES), "binding and header disagree"


def test_library_is_the_in_tree_build():
    maps = open("/proc/self/maps").read()
    assert g.LIB_PATH in maps


def test_strerror_every_status():
    for code in list(g.STATUS) + [-99, 5]:
        s = g.strerror(code)
        assert isinstance(s, str) and s
    assert g.strerror(0) == "success"


def test_config_names_unique():
    names = g.config_names()
    assert len(names) == len(set(names)) == g.lib.gemm_config_count()
    assert g.lib.gemm_config_name(-1) is None
    assert g.lib.gemm_config_name(len(names)) is None


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_plan_create_without_device():
    with pytest.raises(g.GemmError) as e:
        g.Plan(64, 64, 64, "bf16")
    assert e.value.status == -5


def test_layout_plan_errors_without_device():
    """gemm_plan_create_layout validates its layout before looking for a device."""
    e = g.Epilogue(0, 1.0, g.F32)
    assert not g.lib.gemm_plan_create_layout(64, 64, 64, g.BF16, ctypes.byref(e), 1, -1, 7)
    assert g.lib.gemm_last_error() == -10  # GEMM_ERR_ARG
    assert not g.lib.gemm_plan_create_layout(64, 64, 64, g.F32, ctypes.byref(e), 1, -1, 1)
    assert g.lib.gemm_last_error() == -5  # fp32 with a transposed B is valid: no device here


def test_attention_probs_argument_errors_without_device():
    """gemm_attention_probs checks shapes, layout, scale, types, pointers and
    alignment before it looks for a device (the pointers here are never touched)."""
    q, k, p = (ctypes.c_void_p(0x10000 * (i + 1)) for i in range(3))
    call = g.lib.gemm_attention_probs
    assert call(q, k, 1, 64, 513, 64, g.BF16, 0, 1.0, p, g.F32, None) == -1   # N > 512
    assert call(q, k, 1, 64, 0, 64, g.BF16, 0, 1.0, p, g.F32, None) == -1
    assert call(q, k, 1, 0, 64, 64, g.BF16, 0, 1.0, p, g.F32, None) == -1
    assert call(q, k, 0, 64, 64, 64, g.BF16, 0, 1.0, p, g.F32, None) == -1
    assert call(q, k, 1, 64, 64, 4, g.BF16, 0, 1.0, p, g.F32, None) == -1     # D < 8
    assert call(q, k, 1, 64, 64, 72, g.BF16, 0, 1.0, p, g.F32, None) == -1    # D > 64
    assert call(q, k, 1, 64, 64, 20, g.BF16, 1, 1.0, p, g.F32, None) == -1    # D % 8
    assert call(q, k, 1, 64, 20, 64, g.BF16, 0, 1.0, p, g.F32, None) == -1    # K^T: N % 8
    assert call(q, k, 1, 1 << 26, 64, 64, g.BF16, 0, 1.0, p, g.F32, None) == -1  # > 2 GiB
    assert call(q, k, 1, 64, 64, 64, g.BF16, 3, 1.0, p, g.F32, None) == -10   # layout
    assert call(q, k, 1, 64, 64, 64, g.BF16, 0, float("inf"), p, g.F32, None) == -10
    assert call(q, k, 1, 64, 64, 64, g.F32, 0, 1.0, p, g.F32, None) == -2
    assert call(q, k, 1, 64, 64, 64, g.BF16, 0, 1.0, p, 5, None) == -2
    assert call(q, None, 1, 64, 64, 64, g.BF16, 0, 1.0, p, g.F32, None) == -3
    assert call(q, k, 1, 64, 64, 64, g.BF16, 0, 1.0, None, g.F32, None) == -3
    q8 = ctypes.c_void_p(0x10008)
    assert call(q8, k, 1, 64, 64, 64, g.BF16, 0, 1.0, p, g.F32, None) == -4
    p1 = ctypes.c_void_p(0x30001)
    assert call(q, k, 1, 64, 64, 64, g.BF16, 0, 1.0, p1, g.BF16, None) == -4
    if not torch.cuda.is_available():  # every argument valid: the device is missing
        assert call(q, k, 1, 64, 64, 64, g.BF16, 1, 1.0, p, g.F32, None) == -5


def test_null_plan_rejected():
    assert g.lib.gemm_run(None, None, None, None, None, None, None) == -7
    assert g.lib.gemm_run_ws(None, None, None, None, None, None, None, 0, None) == -7
    assert g.lib.gemm_plan_workspace_bytes(None) == -7
    assert g.lib.gemm_plan_describe(None, None, 0) == -7
    g.lib.gemm_plan_destroy(None)  # no-op


@pytest.mark.parametrize("shape,code", [((0, 4, 4), -1), ((4, -1, 4), -1), ((4, 4, 0), -1),
                                        ((1 << 32, 4, 4), -1)])
def test_select_rejects_bad_shapes(shape, code):
    with pytest.raises(g.GemmError) as e:
        g.select(*shape, "bf16", **MI355X)
    assert e.value.status == code


def test_select_rejects_bad_dtype_and_args():
    ch = g.Choice()
    dev = g.DeviceDesc(256, 163840)
    e = g.Epilogue(0, 1.0, 0)
    assert g.lib.gemm_select(ctypes.byref(dev), 8, 8, 8, 7, ctypes.byref(e), 1, 1,
                             ctypes.byref(ch)) == -2
    bad = g.Epilogue(0, 1.0, 9)
    assert g.lib.gemm_select(ctypes.byref(dev), 8, 8, 8, 0, ctypes.byref(bad), 1, 1,
                             ctypes.byref(ch)) == -2
    bad = g.Epilogue(64, 1.0, 0)
    assert g.lib.gemm_select(ctypes.byref(dev), 8, 8, 8, 0, ctypes.byref(bad), 1, 1,
                             ctypes.byref(ch)) == -2
    assert g.lib.gemm_select(ctypes.byref(dev), 8, 8, 8, 0, ctypes.byref(e), 0, 1,
                             ctypes.byref(ch)) == -10
    assert g.lib.gemm_select(None, 8, 8, 8, 0, ctypes.byref(e), 1, 1, ctypes.byref(ch)) == -3


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [(4096, 4096, 4096), (8192, 3072, 768), (8192, 768, 3072),
                                   (512, 512, 512), (1, 4096, 4096), (127, 1000, 771),
                                   (4095, 4097, 63), (1, 1, 1), (33, 65, 17)])
def test_select_fits_budget_and_type(dtype, shape):
    ch = g.select(*shape, dtype, **MI355X)
    name = g.config_names()[ch.config]
    assert ch.lds_bytes <= MI355X["lds_bytes"]
    assert dtype in name
    es = 4 if dtype == "f32" else 2
    M, N, K = shape
    pa, pb = (K * es) % 16 != 0, (N * es) % 16 != 0
    if pa or pb:
        # rows that are not 16-byte multiples take a scalar-load kernel, or (16-bit
        # inputs) a 16-byte-load kernel on copies of exactly those operands in padded rows
        if dtype != "f32" and K <= 64 and M * N >= 1 << 22:
            # K within one 64-deep slice and a large C: the streaming kernel's
            # register-load form, which reads the rows as they are
            assert name == f"m16s_{dtype}_256x128x64_w4x2_u" and ch.packed == 0, name
        elif ch.packed:
            # fp32: only where the copies repay (2^27 multiply-adds and more)
            assert dtype != "f32" or (M > 8 and M * N * K >= 1 << 27)
            assert name.startswith("f32d" if dtype == "f32" else ("m16d", "m16t")), name
            assert ch.packed == (1 if pa else 0) | (2 if pb else 0)
        else:
            assert not (dtype == "f32" and M > 8 and M * N * K >= 1 << 27)
            assert "scalar" in name or name.startswith("simple")
    else:
        assert ch.packed == 0


def test_select_small_lds_device():
    ch = g.select(4096, 4096, 4096, "bf16", cu_count=64, lds_bytes=65536)
    assert ch.lds_bytes <= 65536


def test_select_large_square_uses_big_tiles():
    ch = g.select(4096, 4096, 4096, "bf16", **MI355X)
    assert ch.bm * ch.bn >= 128 * 128
    assert ch.workgroups >= 256  # at least one workgroup per CU


def test_select_small_problem_uses_small_tiles():
    big = g.select(4096, 4096, 4096, "f16", **MI355X)
    small = g.select(1, 4096, 4096, "f16", **MI355X)
    assert small.bm * small.bn < big.bm * big.bn


def test_select_batch_hint_changes_tiles():
    one = g.select(512, 512, 64, "bf16", batch_hint=1, **MI355X)
    many = g.select(512, 512, 64, "bf16", batch_hint=96, **MI355X)
    assert many.bm * many.bn >= one.bm * one.bn
    assert many.workgroups >= 256


def test_select_keeps_slice_offsets_32bit():
    """A 32-bit-offset tiled kernel reads a K slice of row-major B at offsets up to
    bk row lengths: a B row of 2^24 16-bit elements (64 rows = 2 GiB) goes to the
    64-bit kernels, one row shorter stays on the fast ones; the few-row kernels
    address B from its start and keep any width under the 2 GiB total."""
    wide = g.select(16, 1 << 24, 16, "bf16", **MI355X)
    assert not g.config_names()[wide.config].startswith(("m16d", "m16t", "m16n", "m16w", "f32d"))
    fits = g.select(16, (1 << 24) - 8, 16, "bf16", **MI355X)
    assert g.config_names()[fits.config].startswith(("m16d", "m16t"))
    few = g.select(1, 1 << 24, 16, "bf16", **MI355X)
    assert g.config_names()[few.config].startswith("gemv")


TUNED = [
    ((4096, 4096, 4096), 1, "bf16", "m16w_bf16_256x256x32_r4"),
    ((4096, 4096, 4096), 1, "f16", "m16w_f16_256x256x32_r4"),
    ((8192, 8192, 8192), 1, "bf16", "m16w_bf16_256x256x32_r4"),
    ((8192, 8192, 8192), 1, "f16", "m16w_f16_256x256x32_r4"),
    ((8192, 3072, 768), 1, "bf16", "m16t_bf16_128x128x64_w2x2_a2_b2"),
    ((8192, 768, 3072), 1, "bf16", "m16t_bf16_128x256x64_w2x4_a3_b3"),
    ((512, 512, 64), 96, "bf16", "m16s_bf16_256x128x64_w4x2"),
    ((2048, 2048, 2048), 1, "bf16", "m16t_bf16_64x128x64_w2x2_a3_b3"),
    ((512, 64, 512), 96, "bf16", "m16t_bf16_128x128x64_w2x2_a2_b2"),
    ((512, 512, 512), 1, "f16", "m16t_f16_64x128x64_w2x2_a3_b3"),
    ((4096, 4096, 4096), 1, "f32", "f32d_256x256x16_w4x2_a3"),
]


def test_select_tuned_transposed_b():
    """The shape table keeps the two B layouts apart: 4096^3 and the 96-head scores
    product with B given transposed take their own measured configurations."""
    nk = dict(b_layout="nk", **MI355X)
    assert g.config_names()[g.select(4096, 4096, 4096, "bf16", **nk).config] == \
        "m16n_bf16_256x256x64_w2x4_a3_b2"
    assert g.config_names()[g.select(512, 512, 64, "bf16", batch_hint=96, **nk).config] == \
        "m16s_bf16_128x128x64_w2x2_nk"
    c = g.select(512, 512, 64, "bf16", batch_hint=96, **MI355X)
    assert g.config_names()[c.config] == "m16s_bf16_256x128x64_w4x2"
    # the streaming kernel splits nothing and keeps every CU full (one 96 KB workgroup each)
    assert c.split == 1 and c.workgroups == 256 and c.kind == 5


@pytest.mark.parametrize("shape,batch,dtype,name", TUNED)
def test_select_uses_tuned_shapes(shape, batch, dtype, name):
    """Workload shapes take their measured configuration, on the device they were
    measured on; the same shape on a smaller device goes to the cost model."""
    ch = g.select(*shape, dtype, batch_hint=batch, **MI355X)
    assert g.config_names()[ch.config] == name
    small = g.select(*shape, dtype, batch_hint=batch, cu_count=80, lds_bytes=65536)
    assert small.lds_bytes <= 65536


def test_select_split_k_tiles():
    """Few tiles and a long K take the smallest splitting m16d tile, split along K;
    short K stays whole (on the 64 x 128 direct-to-LDS tile, measured faster there)."""
    for (M, N, K), split in [((256, 256, 4096), 8), ((64, 4096, 4096), 8),
                             ((128, 128, 65536), 32), ((512, 512, 512), 1), ((1024, 1024, 1024), 1)]:
        c = g.select(M, N, K, "bf16", **MI355X)
        want = "m16d_bf16_64x128" if split > 1 else "m16t_bf16_64x128"
        assert g.config_names()[c.config].startswith(want), (M, N, K)
        assert c.split == split, (M, N, K, c.split)
        tiles = -(-M // 64) * -(-N // 128)
        assert c.workgroups == tiles * split


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_select_few_rows_split_k(dtype, M):
    """M <= 8 takes the split-K few-row kernel with the fewest rows covering M,
    enough workgroups to fill the device and at most its K rows per workgroup."""
    ch = g.select(M, 4096, 4096, dtype, **MI355X)
    name = g.config_names()[ch.config]
    mr = 1 if M == 1 else (4 if M <= 4 else 8)
    assert name == f"gemv_{dtype}_m{mr}"
    assert ch.split > 1 and ch.workgroups >= MI355X["cu_count"]
    assert (4096 + ch.split - 1) // ch.split <= ch.bk
    # a ninth row leaves the few-row kernel
    assert not g.config_names()[g.select(9, 4096, 4096, dtype, **MI355X).config].startswith("gemv")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_select_transposed_b(dtype):
    """A transposed B (Bt [N x K]) takes the both-operands-K-contiguous kernels;
    K not a multiple of 8 (4 for fp32) copies both operands."""
    for M, N, K in [(4096, 4096, 4096), (512, 512, 64), (1, 4096, 4096), (300, 264, 200)]:
        ch = g.select(M, N, K, dtype, b_layout="nk", **MI355X)
        assert g.config_names()[ch.config].startswith(f"m16n_{dtype}_") and ch.packed == 0
    ch = g.select(127, 1000, 771, dtype, b_layout="nk", **MI355X)
    assert g.config_names()[ch.config].startswith("m16n") and ch.packed == 3
    # the plain layout never takes a transposed-B kernel
    assert not g.config_names()[g.select(4096, 4096, 4096, dtype, **MI355X).config].startswith("m16n")
    # fp32: the f32d kernels with Bt slices loaded like A's; K not a multiple of 4
    # copies both operands, and few rows take them too (no few-row kernel for Bt)
    for M, N, K in [(4096, 4096, 4096), (300, 264, 200), (1, 4096, 4096)]:
        ch = g.select(M, N, K, "f32", b_layout="nk", **MI355X)
        assert g.config_names()[ch.config].startswith("f32d_") and ch.packed == 0
        assert g.config_names()[ch.config].endswith("_nk")
    ch = g.select(127, 1000, 771, "f32", b_layout="nk", **MI355X)
    assert g.config_names()[ch.config].startswith("f32d_") and ch.packed == 3


def test_exact_shape_cache_hit():
    h0, m0, e0 = g.cache_stats()
    g.select(777, 555, 333, "bf16", **MI355X)
    h1, m1, e1 = g.cache_stats()
    g.select(777, 555, 333, "bf16", **MI355X)
    h2, m2, e2 = g.cache_stats()
    assert (m1, e1) == (m0 + 1, e0 + 1)
    assert (h2, m2, e2) == (h1 + 1, m1, e1)


def test_package_never_touches_oracle():
    pkg = os.path.join(ROOT, "dense_gemm_15_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_selection_and_cache_under_threads():
    """Plans may be created from several threads at once: the exact-shape cache is
    process-global and guarded by a lock. Eight threads choose configurations for a
    mix of fresh and repeated shapes at the same time (ctypes releases the GIL during
    the call); every answer equals the one-thread answer, and the cache counts one
    miss and one entry per distinct shape, hits for every other call."""
    from concurrent.futures import ThreadPoolExecutor

    fields = [f for f, _ in g.Choice._fields_]
    shapes = [(64 + 37 * i, 96 + 53 * (i % 7), 48 + 29 * (i % 5), ("bf16", "f16", "f32")[i % 3])
              for i in range(48)]
    shapes = [(m + 90001, n, k, dt) for m, n, k, dt in shapes]  # not chosen before in this process
    h0, m0, e0 = g.cache_stats()
    calls = [s for s in shapes for _ in range(6)]

    def pick(s):
        ch = g.select(*s, **MI355X)
        return s, tuple(getattr(ch, f) for f in fields)

    with ThreadPoolExecutor(max_workers=8) as ex:
        got = list(ex.map(pick, calls))
    h1, m1, e1 = g.cache_stats()
    assert m1 - m0 == len(shapes) and e1 - e0 == len(shapes)
    assert h1 - h0 == len(calls) - len(shapes)
    serial = {s: tuple(getattr(g.select(*s, **MI355X), f) for f in fields) for s in shapes}
    for s, c in got:
        assert c == serial[s], s


def test_select_tuned_every_output_type():
    """The 4096^3 and 8192^3 rows hold for every output type (the one-wave-per-SIMD
    kernel was measured fastest with fp32 and 16-bit output alike); a B given
    transposed keeps rows of its own."""
    names = g.config_names()
    for M in (4096, 8192):
        for dt, outs in (("bf16", ("f32", "bf16")), ("f16", ("f32", "f16"))):
            for od in outs:
                assert names[g.select(M, M, M, dt, out_dtype=od, **MI355X).config] == \
                    f"m16w_{dt}_256x256x32_r4", (M, dt, od)
    nk = dict(b_layout="nk", **MI355X)
    assert names[g.select(4096, 4096, 4096, "bf16", **nk).config] == \
        "m16n_bf16_256x256x64_w2x4_a3_b2"
    assert names[g.select(8192, 8192, 8192, "f16", **nk).config] == "m16w_f16_256x256x32_r5_nk"


@pytest.mark.parametrize("shape,prefix", [
    ((3072, 3072, 3072), "m16t_{t}_256x256x64_w2x4"),
    ((4096, 4096, 2048), "m16t_{t}_256x256x64_w2x4"),
    ((8192, 8192, 2048), "m16t_{t}_256x256x64_w2x4"),
    ((6144, 6144, 6144), "m16t_{t}_128x256x64_w2x4"),
    ((4096, 4096, 16384), "m16w_{t}_256x256x32_r4"),
    ((2048, 8192, 8192), "m16w_{t}_256x256x32_r4"),
])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_cost_model_large_shapes(shape, prefix, dtype):
    """Large shapes outside the shape table: the cost model takes m16t's 256 x 256 tile
    up to K of about 4096 and the one-wave-per-SIMD kernel beyond, as measured on
    MI355X (its longer prologue and epilogue only pay off over a long K); where 256 x
    256 tiles leave a partial last round (6144^2: 2.25 rounds) m16t's 128 x 256 tile,
    measured 1-3% faster there (6144^2 x 3072 213.9 against 219.4 us)."""
    ch = g.select(*shape, dtype, **MI355X)
    assert g.config_names()[ch.config].startswith(prefix.format(t=dtype)), shape


@pytest.mark.parametrize("shape", [(256, 512, 1024), (127, 1000, 768), (4096, 256, 1024),
                                   (256, 256, 64), (512, 2048, 768)])
def test_small_products_take_direct_lds_tiles(shape):
    """Products of a few dozen tiles go to a direct-to-LDS 64 x 128 tile, not to the
    register-staged kernels (measured on MI355X: those take 1.3-2x its time even with
    twice as many tiles)."""
    ch = g.select(*shape, "bf16", **MI355X)
    assert g.config_names()[ch.config].startswith(("m16t_bf16_64x128", "m16d_bf16_64x128")), shape


@pytest.mark.parametrize("shape,layout,prefix", [
    ((3072, 3072, 128), "kn", "m16t_bf16_256x256"),
    ((4096, 3072, 128), "kn", "m16t_bf16_256x256"),
    ((1536, 4096, 128), "nk", "m16n_bf16_128x256"),
    ((3072, 3072, 64), "nk", "m16n_bf16_256x256"),
])
def test_cost_model_counts_rounds(shape, layout, prefix):
    """A short K leaves each round of workgroups mostly fixed latency (launch, first
    loads, last stores): the cost model charges it per round, so the fewer, larger
    tiles win there (measured on MI355X: 3072^2 x 128 13.3 us on 256 x 256 tiles
    against 18.9 us on 128 x 128, B transposed 1536 x 4096 x 128 9.8 against 15.4 us
    on 64 x 128)."""
    ch = g.select(*shape, "bf16", b_layout=layout, **MI355X)
    assert g.config_names()[ch.config].startswith(prefix), (shape, layout)


@pytest.mark.parametrize("shape", [(512, 512, 512), (1024, 1024, 1024), (768, 4096, 128)])
def test_small_transposed_products_take_three_slot_tile(shape):
    """With B given transposed, small products take the 64 x 128 tile with the 3-slot
    ring (measured 3-9% faster than the 4-slot one and than 128 x 128 tiles)."""
    ch = g.select(*shape, "bf16", b_layout="nk", **MI355X)
    assert g.config_names()[ch.config] == "m16n_bf16_64x128x64_w2x2_a3_b3", shape
