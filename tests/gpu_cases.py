"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
get the oracle's verdict on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def flags_of(bias=False, gelu=False, resid=False, scale=None):
    return ((oracle.BIAS if bias else 0) | (oracle.GELU if gelu else 0)
            | (oracle.RESID if resid else 0) | (oracle.SCALE if scale is not None else 0))


def to_bits(t: torch.Tensor) -> np.ndarray:
    return synth.bits(t.cpu())


def sample_indices(M, N, count, seed):
    """Random (row, col) pairs plus every corner and tile-edge neighbourhood."""
    r = np.random.default_rng(seed)
    rows = list(r.integers(0, M, count))
    cols = list(r.integers(0, N, count))
    edge_r = sorted({0, 1, M - 1, M - 2, M // 2} | {x for b in (32, 64, 128, 256)
                                                    for x in (b - 1, b, M - b) if 0 <= x < M})
    edge_c = sorted({0, 1, N - 1, N - 2, N // 2} | {x for b in (32, 64, 128, 256)
                                                    for x in (b - 1, b, N - b) if 0 <= x < N})
    for i in edge_r:
        for j in edge_c:
            rows.append(i)
            cols.append(j)
    rows = np.clip(np.array(rows, np.int64), 0, M - 1)
    cols = np.clip(np.array(cols, np.int64), 0, N - 1)
    return rows, cols


def nan_out(shape, out_dtype, dev="cuda"):
    """An output buffer filled with NaN, so an element the kernel never writes fails the
    comparison instead of passing on a stale value from an earlier run."""
    return torch.full(shape, float("nan"), dtype=TORCH[out_dtype], device=dev)


def run_gpu(plan, A, B, bias=None, resid=None, workspace=None):
    dev = torch.device("cuda")
    out = nan_out((plan.M, plan.N), plan.out_dtype)
    plan.run(A.to(dev), B.to(dev), None if bias is None else bias.to(dev),
             None if resid is None else resid.to(dev), out=out, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu()


def check_full(C, A, B, dtype, out_dtype="f32", bias=None, resid=None, scale=None, gelu=False,
               exact=False, abs_max=None):
    fl = flags_of(bias is not None, gelu, resid is not None, scale)
    ref, s = oracle.gemm(to_bits(A), to_bits(B), dtype, fl, 1.0 if scale is None else scale,
                         None if bias is None else bias.numpy(),
                         None if resid is None else to_bits(resid), out_dtype)
    return oracle.check(to_bits(C), ref, s, out_dtype, fl, 1.0 if scale is None else scale,
                        abs_max=abs_max, exact=exact)


def check_sampled(C, A, B, dtype, rows, cols, out_dtype="f32", bias=None, resid=None, scale=None,
                  gelu=False, exact=False, abs_max=None):
    fl = flags_of(bias is not None, gelu, resid is not None, scale)
    ref, s = oracle.gemm_at(to_bits(A), to_bits(B), dtype, rows, cols, fl,
                            1.0 if scale is None else scale,
                            None if bias is None else bias.numpy(),
                            None if resid is None else to_bits(resid), out_dtype)
    got = to_bits(C)[rows, cols]
    return oracle.check(got, ref, s, out_dtype, fl, 1.0 if scale is None else scale,
                        abs_max=abs_max, exact=exact)


def inputs(M, N, K, dtype, seed, kind="uniform"):
    if kind == "int":
        A = synth.small_int(seed, (M, K), dtype)
        B = synth.small_int(seed + 1, (K, N), dtype)
    else:
        A = synth.uniform(seed, (M, K), dtype)
        B = synth.uniform(seed + 1, (K, N), dtype)
    return A, B
