"""Host-side logic of bench.py (CPU only): kernel-symbol mapping, the committed
HBM-traffic figures, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_symbol_to_config():
    s = bench.symbol_to_config
    assert s("void g15::(anonymous namespace)::gemm_m16d_kernel<g15::bf16_t, 256, 256, 4, 2, 3, 4,"
             " 1>(g15::LaunchArgs)") == "m16d_bf16_256x256x64_w4x2_a3_b4_r1"
    assert s("void g15::(anonymous namespace)::gemm_m16n_kernel<g15::f16_t, 128, 128, 2, 2, 2, 2,"
             " false>(g15::LaunchArgs)") == "m16n_f16_128x128x64_w2x2_a2_b2"
    assert s("void g15::(anonymous namespace)::gemm_m16n_kernel<g15::bf16_t, 128, 128, 2, 2, 2, 2,"
             " true>(g15::LaunchArgs)") == "m16t_bf16_128x128x64_w2x2_a2_b2"
    assert s("void g15::(anonymous namespace)::gemm_f32d_kernel<256, 256, 4, 2, 3, false>"
             "(g15::LaunchArgs)") == "f32d_256x256x16_w4x2_a3"
    assert s("void g15::(anonymous namespace)::gemm_f32d_kernel<128, 128, 2, 2, 3, true>"
             "(g15::LaunchArgs)") == "f32d_128x128x16_w2x2_a3_nk"
    assert s("void g15::(anonymous namespace)::gemm_m16w_kernel<g15::bf16_t, 256, 256, 4, true>"
             "(g15::LaunchArgs)") == "m16w_bf16_256x256x32_r4"
    assert s("void g15::(anonymous namespace)::gemm_m16w_kernel<g15::f16_t, 256, 128, 6, false>"
             "(g15::LaunchArgs)") == "m16w_f16_256x128x32_r6_nk"
    assert s("void g15::(anonymous namespace)::gemv_kernel<g15::f16_t, 1, 4096, 8>"
             "(g15::LaunchArgs, long)") == "gemv_f16_m1"
    assert s("void g15::(anonymous namespace)::gemm_m16s_kernel<g15::bf16_t, 128, 128, 2, 2, true,"
             " false>(g15::LaunchArgs)") == "m16s_bf16_128x128x64_w2x2"
    assert s("void g15::(anonymous namespace)::gemm_m16s_kernel<g15::f16_t, 256, 128, 4, 2, false,"
             " true>(g15::LaunchArgs)") == "m16s_f16_256x128x64_w4x2_nk_u"
    assert s("__amd_rocclr_copyBuffer") is None


def test_committed_traffic_matches_sources():
    """The committed FETCH_SIZE / WRITE_SIZE figures belong to the current sources of
    the headline kernels (re-collect them after changing those kernels)."""
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    for cfg in ("m16w_bf16_256x256x32_r4", "f32d_256x256x16_w4x2_a3"):
        assert t["kernels"][cfg]["source_hash"] == bench.kernel_source_hash(cfg), cfg
        v = bench.measured_traffic(cfg)
        assert v is not None and v > 134e6, (cfg, v)  # at least A + B + C once
    # a family's hash ignores files the kernel does not include
    assert bench.kernel_source_hash("m16d_x") != bench.kernel_source_hash("f32d_x")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
