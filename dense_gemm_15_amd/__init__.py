"""gemm15: tiled dense GEMM for AMD MI355X (gfx950) -- Python binding.

Thin ctypes marshalling over the C ABI in ``include/gemm15.h`` (the library
``libgemm15.so`` built in-tree from ``csrc/``). Every step of the product runs
in the library's HIP kernels; torch supplies device memory and the stream
only. If the library is missing this import fails: there is no other path.

    import torch, dense_gemm_15_amd as g
    plan = g.Plan(M, N, K, "bf16")                # C = A x B, fp32 out
    C = plan.run(A, B)                              # A [M,K], B [K,N] on cuda
    ffn1 = g.Plan(8192, 3072, 768, "bf16", bias=True, gelu=True, out_dtype="bf16")
    H = ffn1.run(X, W1, bias=b1)
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library binds to; must precede the CDLL

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgemm15.so")

F32, F16, BF16 = 0, 1, 2
B_LAYOUT = {"kn": 0, "nk": 1}
EPI_BIAS, EPI_GELU, EPI_RESID, EPI_SCALE = 1, 2, 4, 8
_CODE = {"f32": F32, "f16": F16, "bf16": BF16}
_TORCH = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}
_NAME = {v: k for k, v in _CODE.items()}

STATUS = {
    0: "GEMM_OK", -1: "GEMM_ERR_SHAPE", -2: "GEMM_ERR_DTYPE", -3: "GEMM_ERR_NULL",
    -4: "GEMM_ERR_ALIGN", -5: "GEMM_ERR_NO_DEVICE", -6: "GEMM_ERR_HIP", -7: "GEMM_ERR_PLAN",
    -8: "GEMM_ERR_NOMEM", -9: "GEMM_ERR_CONFIG", -10: "GEMM_ERR_ARG", -11: "GEMM_ERR_WORKSPACE",
}


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({strerror(status)})")


class Epilogue(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("scale", ctypes.c_float), ("out_dtype", ctypes.c_int32)]


class DeviceDesc(ctypes.Structure):
    _fields_ = [("cu_count", ctypes.c_int32), ("lds_bytes", ctypes.c_int32)]


class Choice(ctypes.Structure):
    _fields_ = [("config", ctypes.c_int32), ("kind", ctypes.c_int32), ("bm", ctypes.c_int32),
                ("bn", ctypes.c_int32), ("bk", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("split", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("packed", ctypes.c_int32)]


# Every symbol include/gemm15.h declares, with its ctypes signature.
_I64, _I32, _VP = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
SIGNATURES = {
    "gemm_plan_create": (_VP, [_I64, _I64, _I64, _I32, ctypes.POINTER(Epilogue)]),
    "gemm_plan_create_ex": (_VP, [_I64, _I64, _I64, _I32, ctypes.POINTER(Epilogue), _I64, _I32]),
    "gemm_plan_create_layout": (_VP, [_I64, _I64, _I64, _I32, ctypes.POINTER(Epilogue), _I64, _I32,
                                      _I32]),
    "gemm_run": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "gemm_run_strided_batched": (ctypes.c_int, [_VP, _I64, _VP, _I64, _VP, _I64, _VP, _VP, _I64,
                                                _VP, _I64, _VP]),
    "gemm_run_ws": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _VP]),
    "gemm_run_strided_batched_ws": (ctypes.c_int, [_VP, _I64, _VP, _I64, _VP, _I64, _VP, _VP,
                                                   _I64, _VP, _I64, _VP, _I64, _VP]),
    "gemm_plan_workspace_bytes": (_I64, [_VP]),
    "gemm_run_noalloc": (ctypes.c_int, [_VP, _I64, _VP, _I64, _VP, _I64, _VP, _VP, _I64, _VP,
                                        _I64, _VP]),
    "gemm_noalloc_scratch_bytes": (_I64, []),
    "gemm_plan_destroy": (None, [_VP]),
    "gemm_softmax_rows": (ctypes.c_int, [_VP, _I64, _I64, _I64, ctypes.c_float, _VP, _I64, _I32,
                                         _VP]),
    "gemm_attention_probs": (ctypes.c_int, [_VP, _VP, _I64, _I64, _I64, _I64, _I32, _I32,
                                            ctypes.c_float, _VP, _I32, _VP]),
    "gemm_last_error": (ctypes.c_int, []),
    "gemm_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "gemm_plan_describe": (ctypes.c_int, [_VP, ctypes.c_char_p, ctypes.c_size_t]),
    "gemm_select": (ctypes.c_int, [ctypes.POINTER(DeviceDesc), _I64, _I64, _I64, _I32,
                                   ctypes.POINTER(Epilogue), _I64, _I32, ctypes.POINTER(Choice)]),
    "gemm_select_layout": (ctypes.c_int, [ctypes.POINTER(DeviceDesc), _I64, _I64, _I64, _I32,
                                          ctypes.POINTER(Epilogue), _I64, _I32, _I32,
                                          ctypes.POINTER(Choice)]),
    "gemm_config_count": (ctypes.c_int, []),
    "gemm_config_name": (ctypes.c_char_p, [_I32]),
    "gemm_cache_stats": (None, [ctypes.POINTER(ctypes.c_int64)] * 3),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python dense_gemm_15_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.gemm_strerror(status).decode()


def config_names() -> list[str]:
    return [lib.gemm_config_name(i).decode() for i in range(lib.gemm_config_count())]


def config_index(name: str) -> int:
    names = config_names()
    if name not in names:
        raise KeyError(name)
    return names.index(name)


def cache_stats() -> tuple[int, int, int]:
    h, m, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    lib.gemm_cache_stats(ctypes.byref(h), ctypes.byref(m), ctypes.byref(e))
    return h.value, m.value, e.value


def _epi(bias=False, gelu=False, resid=False, scale=None, out_dtype="f32") -> Epilogue:
    flags = (EPI_BIAS if bias else 0) | (EPI_GELU if gelu else 0) | (EPI_RESID if resid else 0)
    if scale is not None:
        flags |= EPI_SCALE
    return Epilogue(flags, 1.0 if scale is None else float(scale), _CODE[out_dtype])


def select(M, N, K, dtype, *, cu_count=256, lds_bytes=163840, batch_hint=1, aligned16=True,
           b_layout="kn", **epi) -> Choice:
    """Configuration the library would choose on a described device (no GPU needed)."""
    ch = Choice()
    e = _epi(**epi)
    rc = lib.gemm_select_layout(ctypes.byref(DeviceDesc(cu_count, lds_bytes)), M, N, K,
                                _CODE[dtype], ctypes.byref(e), batch_hint, int(bool(aligned16)),
                                B_LAYOUT[b_layout], ctypes.byref(ch))
    if rc != 0:
        raise GemmError(rc, "gemm_select")
    return ch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class Plan:
    """A plan for C = epi(A x B); wraps gemm_plan_create_layout / gemm_run.

    b_layout="kn": B is [K, N]; b_layout="nk": the B passed to run() is Bt [N, K]
    and C = epi(A Bt^T)."""

    def __init__(self, M: int, N: int, K: int, dtype: str, *, bias: bool = False,
                 gelu: bool = False, resid: bool = False, scale: float | None = None,
                 out_dtype: str = "f32", batch_hint: int = 1, config: int | str = -1,
                 b_layout: str = "kn"):
        if isinstance(config, str):
            config = config_index(config)
        self.M, self.N, self.K = M, N, K
        self.dtype, self.out_dtype = dtype, out_dtype
        self.b_layout = b_layout
        self.flags = _epi(bias, gelu, resid, scale, out_dtype)
        self._h = lib.gemm_plan_create_layout(M, N, K, _CODE[dtype], ctypes.byref(self.flags),
                                              batch_hint, config, B_LAYOUT[b_layout])
        if not self._h:
            raise GemmError(lib.gemm_last_error(), "gemm_plan_create_layout")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and lib is not None:  # at interpreter exit the module globals may be gone
            lib.gemm_plan_destroy(h)
            self._h = None

    @property
    def workspace_bytes(self) -> int:
        """Device scratch the plan's runs use (0 for most plans)."""
        n = lib.gemm_plan_workspace_bytes(self._h)
        if n < 0:
            raise GemmError(n, "gemm_plan_workspace_bytes")
        return n

    def _workspace(self, workspace, device, stream):
        """(pointer, bytes) of the scratch for one run: None allocates it through torch
        when the plan needs some; False runs the plan's workspace-free configuration; a
        uint8 cuda tensor is used as given."""
        if workspace is False:
            return None, 0, None
        n = self.workspace_bytes
        if workspace is None:
            if n == 0:
                return None, 0, None
            workspace = torch.empty(n, dtype=torch.uint8, device=device)
        if workspace.device.type != "cuda" or workspace.dtype != torch.uint8:
            raise TypeError("workspace must be a uint8 cuda tensor")
        if stream is not None and stream != torch.cuda.current_stream(workspace.device):
            workspace.record_stream(stream)  # freed memory is not reused before the run ends
        return ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), workspace

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(512)
        rc = lib.gemm_plan_describe(self._h, buf, len(buf))
        if rc < 0:
            raise GemmError(rc, "gemm_plan_describe")
        return buf.value.decode()

    @property
    def config_name(self) -> str:
        return dict(kv.split("=", 1) for kv in self.describe().split())["config"]

    def _check(self, t, shape, dt, what):
        if t.device.type != "cuda":
            raise ValueError(f"{what} must be a cuda tensor")
        if t.dtype != _TORCH[_CODE[dt]]:
            raise TypeError(f"{what} must be {_TORCH[_CODE[dt]]}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous with shape {tuple(shape)}")

    def _stream(self, stream):
        s = stream if stream is not None else torch.cuda.current_stream()
        return ctypes.c_void_p(s.cuda_stream)

    def run(self, A, B, bias=None, resid=None, out=None, stream=None, workspace=None):
        """C = epi(A x B) on the current (or given) stream; returns C. workspace: None
        (scratch allocated through torch when the plan needs some), False (the plan's
        workspace-free configuration) or a uint8 cuda tensor of at least
        workspace_bytes."""
        M, N, K = self.M, self.N, self.K
        self._check(A, (M, K), self.dtype, "A")
        self._check(B, (K, N) if self.b_layout == "kn" else (N, K), self.dtype, "B")
        if out is None:
            out = torch.empty((M, N), dtype=_TORCH[_CODE[self.out_dtype]], device=A.device)
        self._check(out, (M, N), self.out_dtype, "C")
        if self.flags.flags & EPI_BIAS:
            self._check(bias, (N,), "f32", "bias")
        if self.flags.flags & EPI_RESID:
            self._check(resid, (M, N), self.out_dtype, "resid")
        wp, wn, _keep = self._workspace(workspace, A.device, stream)
        rc = lib.gemm_run_ws(self._h, _ptr(A), _ptr(B), _ptr(bias), _ptr(resid), _ptr(out),
                             wp, wn, self._stream(stream))
        if rc != 0:
            raise GemmError(rc, "gemm_run_ws")
        return out

    def run_batched(self, A, B, bias=None, resid=None, out=None, stream=None, workspace=None):
        """C[b] = epi(A[b] x B[b]) for 3-D contiguous A [b,M,K], B [b,K,N]; returns C
        (workspace as for run)."""
        M, N, K = self.M, self.N, self.K
        nb = A.shape[0]
        self._check(A, (nb, M, K), self.dtype, "A")
        self._check(B, (nb, K, N) if self.b_layout == "kn" else (nb, N, K), self.dtype, "B")
        if out is None:
            out = torch.empty((nb, M, N), dtype=_TORCH[_CODE[self.out_dtype]], device=A.device)
        self._check(out, (nb, M, N), self.out_dtype, "C")
        if self.flags.flags & EPI_BIAS:
            self._check(bias, (N,), "f32", "bias")
        if self.flags.flags & EPI_RESID:
            self._check(resid, (nb, M, N), self.out_dtype, "resid")
        wp, wn, _keep = self._workspace(workspace, A.device, stream)
        rc = lib.gemm_run_strided_batched_ws(self._h, nb, _ptr(A), M * K, _ptr(B), K * N,
                                             _ptr(bias), _ptr(resid), M * N, _ptr(out), M * N,
                                             wp, wn, self._stream(stream))
        if rc != 0:
            raise GemmError(rc, "gemm_run_strided_batched_ws")
        return out


def softmax_rows(S, scale: float = 1.0, out_dtype: str = "bf16", out=None, stream=None):
    """P = softmax(scale * S) over the last dimension of a contiguous fp32 cuda tensor
    (gemm_softmax_rows); P has S's shape and type out_dtype."""
    if S.device.type != "cuda" or S.dtype != torch.float32 or not S.is_contiguous():
        raise ValueError("S must be a contiguous float32 cuda tensor")
    cols = S.shape[-1]
    rows = S.numel() // cols
    if out is None:
        out = torch.empty(S.shape, dtype=_TORCH[_CODE[out_dtype]], device=S.device)
    elif (out.shape != S.shape or out.dtype != _TORCH[_CODE[out_dtype]] or not out.is_contiguous()
          or out.device != S.device):
        raise ValueError("out must be a contiguous tensor of S's shape and type out_dtype")
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = lib.gemm_softmax_rows(_ptr(S), rows, cols, cols, float(scale), _ptr(out), cols,
                               _CODE[out_dtype], ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise GemmError(rc, "gemm_softmax_rows")
    return out


def attention_probs(Q, Kmat, scale: float = 1.0, k_layout: str = "kn", out_dtype: str = "bf16",
                    out=None, stream=None):
    """P = softmax(scale * Q K^T) per batch item in one kernel (gemm_attention_probs).
    Q [batch, M, D] bf16/f16; Kmat [batch, D, N] (K^T, k_layout "kn") or [batch, N, D]
    (the keys, "nk"), Q's type; P [batch, M, N] of out_dtype. All contiguous cuda."""
    if Q.dim() != 3 or Kmat.dim() != 3 or k_layout not in ("kn", "nk"):
        raise ValueError("Q and Kmat must be 3-d; k_layout 'kn' or 'nk'")
    nb, M, D = Q.shape
    N = Kmat.shape[2] if k_layout == "kn" else Kmat.shape[1]
    want = (nb, D, N) if k_layout == "kn" else (nb, N, D)
    if tuple(Kmat.shape) != want or Kmat.dtype != Q.dtype:
        raise ValueError(f"Kmat must be {want} of Q's type")
    for t in (Q, Kmat):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("Q and Kmat must be contiguous cuda tensors")
    if Q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("Q must be bf16 or f16")
    dt = "bf16" if Q.dtype == torch.bfloat16 else "f16"
    if out is None:
        out = torch.empty((nb, M, N), dtype=_TORCH[_CODE[out_dtype]], device=Q.device)
    elif (tuple(out.shape) != (nb, M, N) or out.dtype != _TORCH[_CODE[out_dtype]]
          or not out.is_contiguous() or out.device != Q.device):
        raise ValueError("out must be a contiguous [batch, M, N] tensor of out_dtype")
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = lib.gemm_attention_probs(_ptr(Q), _ptr(Kmat), nb, M, N, D, _CODE[dt],
                                  0 if k_layout == "kn" else 1, float(scale), _ptr(out),
                                  _CODE[out_dtype], ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise GemmError(rc, "gemm_attention_probs")
    return out
