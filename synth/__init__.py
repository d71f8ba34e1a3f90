"""Seeded synthetic inputs for the dense GEMM workloads.

This module only draws numbers. It holds none of the GEMM's arithmetic: no
products, no sums, no epilogue. Both the CPU oracle and the HIP library are
fed from it, and neither is imported here.

Recipe (one ``numpy.random.default_rng(seed)`` stream per tensor):

* ``uniform``: float64 U[-1, 1) draws -> float32 -> the requested element type.
  The float32 -> bf16 / fp16 step is torch's conversion (round to nearest,
  ties to even), so the 16-bit matrices are "uniform[-1,1] rounded to 16-bit".
* ``normal``:  float64 standard normal draws times ``std`` -> float32 -> type.
* ``small_int``: integers in [lo, hi] (exactly representable in every type),
  used for the bit-exact cases.

The shapes and seeds of the benchmark workloads (square 4096 GEMMs, the BERT
encoder FFN with hidden 768 / FFN 3072 over 16 x 512 tokens, 96 attention-score
heads of 512 x 64, and three odd fp16 shapes) live in ``WORKLOADS``.
"""
from __future__ import annotations

import numpy as np
import torch

DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
}


def _cast(x64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return t.to(DTYPES[dtype]).contiguous()


def uniform(seed: int, shape, dtype: str, lo: float = -1.0, hi: float = 1.0) -> torch.Tensor:
    """U[lo, hi) drawn in float64 from ``seed``, rounded to ``dtype`` (CPU tensor)."""
    rng = np.random.default_rng(seed)
    return _cast(rng.uniform(lo, hi, size=tuple(shape)), dtype)


def normal(seed: int, shape, std: float, dtype: str) -> torch.Tensor:
    """N(0, std^2) drawn in float64 from ``seed``, rounded to ``dtype`` (CPU tensor)."""
    rng = np.random.default_rng(seed)
    return _cast(rng.standard_normal(size=tuple(shape)) * std, dtype)


def small_int(seed: int, shape, dtype: str, lo: int = -8, hi: int = 8) -> torch.Tensor:
    """Integers uniform in [lo, hi], held in ``dtype`` (exact in bf16/fp16/fp32)."""
    rng = np.random.default_rng(seed)
    return _cast(rng.integers(lo, hi + 1, size=tuple(shape)).astype(np.float64), dtype)


def grid(seed: int, shape, dtype: str, step: float = 2.0 ** -10) -> torch.Tensor:
    """Multiples of ``step`` uniform in [-1, 1] (exact in fp16 for step 2^-10)."""
    rng = np.random.default_rng(seed)
    n = int(round(1.0 / step))
    return _cast(rng.integers(-n, n + 1, size=tuple(shape)).astype(np.float64) * step, dtype)


def device_uniform(seed: int, shape, dtype: str, device="cuda") -> torch.Tensor:
    """U[-1, 1) drawn on the GPU by torch's generator seeded with ``seed``, in
    ``dtype``: for operands too large to draw on the host."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.rand(tuple(shape), generator=gen, device=device, dtype=torch.float32) * 2 - 1
    return x.to(DTYPES[dtype])


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw element bits of a CPU tensor as a numpy array.

    16-bit types come back as ``uint16``; float32 comes back as ``float32``
    (its bits are its value)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


# Workloads: every tensor with its shape, distribution, type and seed.
# ("gemm", M, N, K, dtype, seedA, seedB) entries are plain C = A x B with fp32 C.
WORKLOADS = {
    "fp16_512": dict(kind="gemm", M=512, N=512, K=512, dtype="f16", seeds=(101, 102)),
    "fp32_4096": dict(kind="gemm", M=4096, N=4096, K=4096, dtype="f32", seeds=(201, 202)),
    "bf16_4096": dict(kind="gemm", M=4096, N=4096, K=4096, dtype="bf16", seeds=(301, 302)),
    "fp16_4096": dict(kind="gemm", M=4096, N=4096, K=4096, dtype="f16", seeds=(301, 302)),
    # Encoder FFN: X [16*512 x 768] ~N(0,1); W1 [768 x 3072], W2 [3072 x 768] ~N(0, 0.02);
    # fp32 biases ~N(0, 0.02); seeds X 401, W1 402, b1 403, W2 404, b2 405.
    "ffn": dict(kind="ffn", tokens=8192, hidden=768, ffn=3072, seeds=(401, 402, 403, 404, 405)),
    # Attention scores: Q, K [96 x 512 x 64] bf16 ~N(0,1) (index = batch*12 + head); seeds 501, 502.
    "qk": dict(kind="qk", batch=96, seq=512, head_dim=64, seeds=(501, 502)),
    # Attention continuation: V [96 x 512 x 64] bf16 ~N(0,1), seed 503; P = softmax(Q K^T)
    # row by row (the tutorial page's Softmax(QK^T)V, no 1/sqrt(D) factor), O = P V.
    "attention": dict(kind="attention", batch=96, seq=512, head_dim=64, seeds=(501, 502, 503)),
    "gemv_1x4096x4096": dict(kind="gemm", M=1, N=4096, K=4096, dtype="f16", seeds=(511, 512)),
    "odd_127x1000x771": dict(kind="gemm", M=127, N=1000, K=771, dtype="f16", seeds=(521, 522)),
    "odd_4095x4097x63": dict(kind="gemm", M=4095, N=4097, K=63, dtype="f16", seeds=(531, 532)),
    # Few tiles, long K (the small-M x N, large-K shapes run split along K).
    "longk_256x256x4096": dict(kind="gemm", M=256, N=256, K=4096, dtype="bf16", seeds=(541, 542)),
    "longk_64x4096x4096": dict(kind="gemm", M=64, N=4096, K=4096, dtype="bf16", seeds=(543, 544)),
}


def gemm_inputs(name: str):
    """(A, B) CPU tensors of a plain GEMM workload."""
    w = WORKLOADS[name]
    assert w["kind"] == "gemm"
    sa, sb = w["seeds"]
    A = uniform(sa, (w["M"], w["K"]), w["dtype"])
    B = uniform(sb, (w["K"], w["N"]), w["dtype"])
    return A, B


def ffn_inputs():
    """X, W1, b1, W2, b2 of the encoder FFN workload (CPU tensors)."""
    w = WORKLOADS["ffn"]
    sx, s1, sb1, s2, sb2 = w["seeds"]
    T, H, F = w["tokens"], w["hidden"], w["ffn"]
    X = normal(sx, (T, H), 1.0, "bf16")
    W1 = normal(s1, (H, F), 0.02, "bf16")
    b1 = normal(sb1, (F,), 0.02, "f32")
    W2 = normal(s2, (F, H), 0.02, "bf16")
    b2 = normal(sb2, (H,), 0.02, "f32")
    return X, W1, b1, W2, b2


def attention_inputs():
    """Q [96 x 512 x 64], K^T [96 x 64 x 512] (as qk_inputs) and V [96 x 512 x 64], bf16."""
    w = WORKLOADS["attention"]
    Q, Kt = qk_inputs()
    V = normal(w["seeds"][2], (w["batch"], w["seq"], w["head_dim"]), 1.0, "bf16")
    return Q, Kt, V


def qk_inputs():
    """Q [96 x 512 x 64] and K^T [96 x 64 x 512] bf16 (CPU tensors).

    K is drawn as [96 x 512 x 64] and transposed per head into a contiguous
    row-major [64 x 512] right operand."""
    w = WORKLOADS["qk"]
    sq, sk = w["seeds"]
    b, s, d = w["batch"], w["seq"], w["head_dim"]
    Q = normal(sq, (b, s, d), 1.0, "bf16")
    Kmat = normal(sk, (b, s, d), 1.0, "bf16")
    Kt = Kmat.transpose(1, 2).contiguous()
    return Q, Kt
