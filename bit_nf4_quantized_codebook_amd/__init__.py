"""MI355X (gfx950) NF4 quantized-codebook linear layer with a LoRA side branch.

Thin Python binding over the C ABI of ``libnf4.so`` (declared in ``include/nf4.h``).  Every
function here only marshals arguments: tensors are passed by device pointer, the stream is the
current torch stream, and all arithmetic runs in the library's HIP kernels.  If the library is
not built, importing the binding raises; there is no fallback path.

Names follow the C ABI:
  nf4_build_codebook, nf4_build_int4_codebook, nf4_build_fp4_codebook, nf4_quantize,
  nf4_double_quant, nf4_double_quant_int8, nf4_dequant, nf4_dequant_single, qlora_linear_fwd,
  qlora_linear_fwd_static, qlora_linear_bwd, qlora_swiglu_fwd, qlora_swiglu_bwd, qlora_gated_fwd, qlora_gated_bwd,
  qlora_multi_fwd.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4.so")

NF4_OK = 0
QLORA_DX_ACCUMULATE = 1
BLOCK = 64
DQ_BLOCK = 256

#: Symbols the C ABI exports (include/nf4.h).
EXPORTS = (
    "nf4_status_string", "nf4_last_error", "nf4_version", "nf4_build_codebook",
    "nf4_build_int4_codebook", "nf4_build_fp4_codebook", "nf4_quantize",
    "nf4_double_quant_workspace_size", "nf4_double_quant", "nf4_double_quant_int8", "nf4_dequant",
    "nf4_dequant_single",
    "qlora_linear_workspace_size", "qlora_linear_route", "qlora_linear_fwd", "qlora_linear_fwd_static", "qlora_linear_bwd",
    "qlora_swiglu_fwd", "qlora_swiglu_bwd", "qlora_gated_workspace_size", "qlora_gated_fwd", "qlora_gated_bwd",
    "qlora_multi_workspace_size", "qlora_multi_fwd",
    "nf4_set_gemm_timing_events", "nf4_gemm_timing_count",
)


class NF4Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class _WeightDesc(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("absmax_q", ctypes.c_void_p),
        ("absmax_scale", ctypes.c_void_p),
        ("absmax_mean", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("block", ctypes.c_int32),
        ("dq_block", ctypes.c_int32),
        ("codebook", ctypes.c_float * 16),
        ("dq_format", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_nf4_quantized_codebook_amd.build` "
                          "or __graft_entry__.build()")
    # torch ships its own HIP runtime under the same soname; loading torch first makes the library
    # bind to that one copy, so the tensors' device memory and the kernels share one runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    i = ctypes.c_int
    W = ctypes.POINTER(_WeightDesc)
    sigs = {
        "nf4_status_string": (ctypes.c_char_p, [i]),
        "nf4_last_error": (ctypes.c_char_p, []),
        "nf4_version": (ctypes.c_char_p, []),
        "nf4_build_codebook": (i, [P, ctypes.c_double]),
        "nf4_build_int4_codebook": (i, [P]),
        "nf4_build_fp4_codebook": (i, [P]),
        "nf4_quantize": (i, [P, i64, i32, P, P, P, P]),
        "nf4_double_quant_workspace_size": (sz, [i64, i32]),
        "nf4_double_quant": (i, [P, i64, i32, P, P, P, P, sz, P]),
        "nf4_double_quant_int8": (i, [P, i64, i32, P, P, P, P, sz, P]),
        "nf4_dequant": (i, [W, P, P]),
        "nf4_dequant_single": (i, [P, P, i64, i32, P, P, P]),
        "qlora_linear_workspace_size": (sz, [i64, i64, i64, i32]),
        "qlora_linear_route": (i, [i64, i64, i64, i32, P]),
        "qlora_linear_fwd": (i, [W, P, P, P, ctypes.c_float, i64, i32, P, P, P, sz, P]),
        "qlora_linear_fwd_static": (i, [W, P, P, P, ctypes.c_float, i64, i32, P, P, P]),
        "qlora_linear_bwd": (i, [W, P, P, P, P, P, ctypes.c_float, i64, i32, P, P, P,
                                 ctypes.c_uint32, P, sz, P]),
        "qlora_swiglu_fwd": (i, [P, P, P, i64, P]),
        "qlora_gated_workspace_size": (sz, [i64, i64, i64, i32]),
        "qlora_gated_bwd": (i, [W, W, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, i64, i32, P, P, P, P, P,
                                ctypes.c_uint32, P, sz, P]),
        "qlora_gated_fwd": (i, [W, W, P, P, P, P, P, ctypes.c_float, i64, i32, P, P, P, P, P,
                                ctypes.c_uint32, P, sz, P]),
        "qlora_swiglu_bwd": (i, [P, P, P, P, P, i64, P]),
        "qlora_multi_workspace_size": (sz, [i32, P, i64, i64, i32]),
        "qlora_multi_fwd": (i, [i32, P, P, P, P, ctypes.c_float, i64, i32, P, P, P, sz, P]),
        "nf4_set_gemm_timing_events": (i, [P, P, P, i32]),
        "nf4_gemm_timing_count": (i32, []),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def _check(status: int, where: str):
    if status != NF4_OK:
        raise NF4Error(status, where, lib.nf4_last_error().decode())


def status_string(status: int) -> str:
    return lib.nf4_status_string(status).decode()


def version() -> str:
    return lib.nf4_version().decode()


# ------------------------------------------------------------------------------------------
# torch plumbing (device memory and streams only)
# ------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device, workspace=None):
    torch = _torch()
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------------
# Codebook, quantize, double quant, dequant
# ------------------------------------------------------------------------------------------

def nf4_build_codebook(delta: float = 0.0) -> np.ndarray:
    """The 16 NF4 codewords (host, float32, ascending); delta 0 selects the default."""
    out = np.zeros(16, dtype=np.float32)
    _check(lib.nf4_build_codebook(ctypes.c_void_p(out.ctypes.data), float(delta)), "nf4_build_codebook")
    return out


def nf4_build_int4_codebook() -> np.ndarray:
    """The 4-bit integer table (k / 7, k = -8 .. 7), host float32, ascending."""
    out = np.zeros(16, dtype=np.float32)
    _check(lib.nf4_build_int4_codebook(ctypes.c_void_p(out.ctypes.data)), "nf4_build_int4_codebook")
    return out


def nf4_build_fp4_codebook() -> np.ndarray:
    """The 4-bit float (E2M1 / 6) table, host float32, ascending, two zero entries."""
    out = np.zeros(16, dtype=np.float32)
    _check(lib.nf4_build_fp4_codebook(ctypes.c_void_p(out.ctypes.data)), "nf4_build_fp4_codebook")
    return out


def nf4_quantize(W, codebook=None, block: int = BLOCK):
    """Level-1 quantization of a float32 device tensor: returns (packed uint8, absmax float32)."""
    torch = _torch()
    _need(W, torch.float32, "W")
    cb = nf4_build_codebook() if codebook is None else np.ascontiguousarray(codebook, dtype=np.float32)
    n = W.numel()
    packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=W.device)
    absmax = torch.empty((n + block - 1) // block, dtype=torch.float32, device=W.device)
    _check(lib.nf4_quantize(_ptr(W), n, block, ctypes.c_void_p(cb.ctypes.data), _ptr(packed),
                            _ptr(absmax), _stream(W.device)), "nf4_quantize")
    return packed, absmax


#: second-level code formats (nf4_weight.dq_format)
DQ_FORMATS = {"e4m3": 0, "int8": 1}


def nf4_double_quant(absmax, dq_block: int = DQ_BLOCK, workspace=None, fmt: str = "e4m3"):
    """Level-2 quantization: returns (absmax_q uint8, absmax_scale float32, absmax_mean float32[1]).
    fmt "e4m3" (nf4_double_quant) or "int8" (nf4_double_quant_int8)."""
    torch = _torch()
    _need(absmax, torch.float32, "absmax")
    nb = absmax.numel()
    q = torch.empty(nb, dtype=torch.uint8, device=absmax.device)
    sc = torch.empty((nb + dq_block - 1) // dq_block, dtype=torch.float32, device=absmax.device)
    mean = torch.empty(1, dtype=torch.float32, device=absmax.device)
    wsb = lib.nf4_double_quant_workspace_size(nb, dq_block)
    ws = _workspace(wsb, absmax.device, workspace)
    fn = {"e4m3": lib.nf4_double_quant, "int8": lib.nf4_double_quant_int8}[fmt]
    _check(fn(_ptr(absmax), nb, dq_block, _ptr(q), _ptr(sc), _ptr(mean), _ptr(ws), wsb,
              _stream(absmax.device)), "nf4_double_quant(%s)" % fmt)
    return q, sc, mean


@dataclass
class NF4Weight:
    """A frozen NF4 weight [rows = N_out, cols = K_in] in double-quantized form (device tensors)."""
    packed: object
    absmax_q: object
    absmax_scale: object
    absmax_mean: object
    rows: int
    cols: int
    codebook: np.ndarray
    block: int = BLOCK
    dq_block: int = DQ_BLOCK
    dq_format: str = "e4m3"

    def descriptor(self) -> _WeightDesc:
        d = _WeightDesc()
        d.packed = self.packed.data_ptr()
        d.absmax_q = self.absmax_q.data_ptr()
        d.absmax_scale = self.absmax_scale.data_ptr()
        d.absmax_mean = self.absmax_mean.data_ptr()
        d.rows, d.cols = int(self.rows), int(self.cols)
        d.block, d.dq_block = int(self.block), int(self.dq_block)
        d.dq_format = DQ_FORMATS[self.dq_format]
        for j in range(16):
            d.codebook[j] = float(self.codebook[j])
        return d

    @property
    def device(self):
        return self.packed.device

    @classmethod
    def from_float(cls, W, codebook=None, dq_format: str = "e4m3"):
        """Quantize + double-quantize a float32 [rows, cols] device tensor."""
        cb = nf4_build_codebook() if codebook is None else np.ascontiguousarray(codebook, dtype=np.float32)
        packed, absmax = nf4_quantize(W.contiguous(), cb)
        q, sc, mean = nf4_double_quant(absmax, fmt=dq_format)
        return cls(packed, q, sc, mean, W.shape[0], W.shape[1], cb, dq_format=dq_format)


def nf4_dequant(w: NF4Weight):
    """Double dequantization: bf16 [rows, cols] device tensor."""
    torch = _torch()
    out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=w.device)
    d = w.descriptor()
    _check(lib.nf4_dequant(ctypes.byref(d), _ptr(out), _stream(w.device)), "nf4_dequant")
    return out


def nf4_dequant_single(packed, absmax, numel: int, codebook=None, block: int = BLOCK):
    """Single-level dequantization (float32 block constants, no DQ): bf16 [numel] device tensor."""
    torch = _torch()
    _need(packed, torch.uint8, "packed")
    _need(absmax, torch.float32, "absmax")
    cb = nf4_build_codebook() if codebook is None else np.ascontiguousarray(codebook, dtype=np.float32)
    out = torch.empty(numel, dtype=torch.bfloat16, device=packed.device)
    _check(lib.nf4_dequant_single(_ptr(packed), _ptr(absmax), numel, block, ctypes.c_void_p(cb.ctypes.data),
                                  _ptr(out), _stream(packed.device)), "nf4_dequant_single")
    return out


# ------------------------------------------------------------------------------------------
# Linear layer
# ------------------------------------------------------------------------------------------

def qlora_linear_workspace_size(M: int, N: int, K: int, r: int) -> int:
    return int(lib.qlora_linear_workspace_size(M, N, K, r))


_PATHS = {0: None, 1: "gemv", 2: "gemv_wide", 3: "fused", 4: "expanded"}


def qlora_linear_route(M: int, N: int, K: int, r: int) -> dict:
    """How the layer runs this shape: the forward's and backward's path and how many workgroups
    each output tile's reduction is split over (1: not split)."""
    info = (ctypes.c_int32 * 4)()
    _check(lib.qlora_linear_route(M, N, K, r, info), "qlora_linear_route")
    return {"fwd": _PATHS[info[0]], "fwd_split": int(info[1]), "bwd": _PATHS[info[3]], "bwd_split": int(info[2])}


def qlora_linear_fwd(w: NF4Weight, X, L1, L2, scale: float, keep_T: bool = True, Y=None,
                     workspace=None, T=None):
    """Y = X deq(W)^T + scale (X L1) L2.  Returns (Y, T) with T = X L1 (or None)."""
    torch = _torch()
    for t, n in ((X, "X"), (L1, "L1"), (L2, "L2")):
        _need(t, torch.bfloat16, n)
    M, r = X.shape[0], L1.shape[1]
    if X.shape[1] != w.cols or L1.shape[0] != w.cols or tuple(L2.shape) != (r, w.rows):
        raise ValueError("shape mismatch")
    if Y is None:
        Y = torch.empty((M, w.rows), dtype=torch.bfloat16, device=X.device)
    if T is None and keep_T:
        T = torch.empty((M, r), dtype=torch.bfloat16, device=X.device)
    wsb = qlora_linear_workspace_size(M, w.rows, w.cols, r)
    ws = _workspace(wsb, X.device, workspace)
    d = w.descriptor()
    _check(lib.qlora_linear_fwd(ctypes.byref(d), _ptr(X), _ptr(L1), _ptr(L2), float(scale), M, r,
                                _ptr(Y), _ptr(T), _ptr(ws), wsb, _stream(X.device)), "qlora_linear_fwd")
    return Y, T


#: bytes of the static scratch behind qlora_linear_fwd_static (include/nf4.h)
QLORA_STATIC_SCRATCH_BYTES = 128 << 20


def qlora_linear_fwd_static(w: NF4Weight, X, L1, L2, scale: float, Y, T=None):
    """qlora_linear_fwd without a workspace: the library's static device scratch stands in for it
    and the call allocates nothing (Y, and T when wanted, are the caller's).  Returns (Y, T)."""
    torch = _torch()
    for t, n in ((X, "X"), (L1, "L1"), (L2, "L2"), (Y, "Y")):
        _need(t, torch.bfloat16, n)
    if T is not None:
        _need(T, torch.bfloat16, "T")
    M, r = X.shape[0], L1.shape[1]
    if X.shape[1] != w.cols or L1.shape[0] != w.cols or tuple(L2.shape) != (r, w.rows) or \
            tuple(Y.shape) != (M, w.rows) or (T is not None and tuple(T.shape) != (M, r)):
        raise ValueError("shape mismatch")
    d = w.descriptor()
    _check(lib.qlora_linear_fwd_static(ctypes.byref(d), _ptr(X), _ptr(L1), _ptr(L2), float(scale), M, r, _ptr(Y),
                                       _ptr(T), _stream(X.device)), "qlora_linear_fwd_static")
    return Y, T


def qlora_linear_bwd(w: NF4Weight, dY, X, L1, L2, T, scale: float, need_dX: bool = True,
                     dX=None, accumulate: bool = False, workspace=None, dL1=None, dL2=None):
    """Returns (dX or None, dL1, dL2) for the layer above; W is not touched."""
    torch = _torch()
    for t, n in ((dY, "dY"), (X, "X"), (L1, "L1"), (L2, "L2")):
        _need(t, torch.bfloat16, n)
    if T is not None:
        _need(T, torch.bfloat16, "T")
    M, r = X.shape[0], L1.shape[1]
    if tuple(dY.shape) != (M, w.rows) or X.shape[1] != w.cols:
        raise ValueError("shape mismatch")
    if need_dX and dX is None:
        dX = torch.empty((M, w.cols), dtype=torch.bfloat16, device=X.device)
    if not need_dX:
        dX = None
    if dL1 is None:
        dL1 = torch.empty((w.cols, r), dtype=torch.bfloat16, device=X.device)
    if dL2 is None:
        dL2 = torch.empty((r, w.rows), dtype=torch.bfloat16, device=X.device)
    wsb = qlora_linear_workspace_size(M, w.rows, w.cols, r)
    ws = _workspace(wsb, X.device, workspace)
    d = w.descriptor()
    flags = QLORA_DX_ACCUMULATE if accumulate else 0
    _check(lib.qlora_linear_bwd(ctypes.byref(d), _ptr(dY), _ptr(X), _ptr(L1), _ptr(L2), _ptr(T),
                                float(scale), M, r, _ptr(dX), _ptr(dL1), _ptr(dL2), flags, _ptr(ws),
                                wsb, _stream(X.device)), "qlora_linear_bwd")
    return dX, dL1, dL2


def qlora_swiglu_fwd(g, u, h=None):
    torch = _torch()
    _need(g, torch.bfloat16, "g")
    _need(u, torch.bfloat16, "u")
    if h is None:
        h = torch.empty_like(g)
    _check(lib.qlora_swiglu_fwd(_ptr(g), _ptr(u), _ptr(h), g.numel(), _stream(g.device)), "qlora_swiglu_fwd")
    return h


QLORA_GATED_FUSE = 2   # include/nf4.h (QLORA_DX_ACCUMULATE is 1)


def qlora_gated_fwd(w_gate: NF4Weight, w_up: NF4Weight, X, L1_gate, L2_gate, L1_up, L2_up, scale: float,
                    keep_T: bool = True, workspace=None, fuse: bool = False):
    """Gated MLP forward (gate and up linears + SwiGLU): returns (G, U, H, T_gate, T_up).
    fuse: one GEMM for both products with the glue in its epilogue (QLORA_GATED_FUSE)."""
    torch = _torch()
    M, K = X.shape
    F, r = w_gate.rows, L1_gate.shape[1]
    dev = X.device
    G = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    U = torch.empty_like(G)
    H = torch.empty_like(G)
    Tg = torch.empty((M, r), dtype=torch.bfloat16, device=dev) if keep_T else None
    Tu = torch.empty((M, r), dtype=torch.bfloat16, device=dev) if keep_T else None
    wsb = lib.qlora_gated_workspace_size(M, F, K, r)
    ws = _workspace(wsb, dev, workspace)
    dg, du = w_gate.descriptor(), w_up.descriptor()
    _check(lib.qlora_gated_fwd(ctypes.byref(dg), ctypes.byref(du), _ptr(X), _ptr(L1_gate), _ptr(L2_gate),
                               _ptr(L1_up), _ptr(L2_up), float(scale), M, r, _ptr(G), _ptr(U), _ptr(H),
                               _ptr(Tg) if keep_T else None, _ptr(Tu) if keep_T else None,
                               QLORA_GATED_FUSE if fuse else 0, _ptr(ws), wsb, _stream(dev)), "qlora_gated_fwd")
    return G, U, H, Tg, Tu


def qlora_gated_bwd(w_gate: NF4Weight, w_up: NF4Weight, dH, X, G, U, L1_gate, L2_gate, L1_up, L2_up,
                    T_gate, T_up, scale: float, need_dX: bool = True, dX=None, accumulate: bool = False,
                    workspace=None, fuse: bool = False):
    """Gated MLP backward: returns (dX, dL1_gate, dL2_gate, dL1_up, dL2_up).
    fuse: dX as one GEMM over both weights (QLORA_GATED_FUSE)."""
    torch = _torch()
    M, K = X.shape
    F, r = w_gate.rows, L1_gate.shape[1]
    dev = X.device
    if need_dX and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    grads = [torch.empty(shp, dtype=torch.bfloat16, device=dev) for shp in ((K, r), (r, F), (K, r), (r, F))]
    wsb = lib.qlora_gated_workspace_size(M, F, K, r)
    ws = _workspace(wsb, dev, workspace)
    flags = (QLORA_GATED_FUSE if fuse else 0) | (1 if accumulate else 0)
    dg, du = w_gate.descriptor(), w_up.descriptor()
    p = lambda t: _ptr(t) if t is not None else None  # noqa: E731
    _check(lib.qlora_gated_bwd(ctypes.byref(dg), ctypes.byref(du), _ptr(dH), _ptr(X), _ptr(G), _ptr(U),
                               _ptr(L1_gate), _ptr(L2_gate), _ptr(L1_up), _ptr(L2_up), p(T_gate), p(T_up),
                               float(scale), M, r, p(dX if need_dX else None), *(_ptr(t) for t in grads), flags,
                               _ptr(ws), wsb, _stream(dev)), "qlora_gated_bwd")
    return (dX if need_dX else None), grads[0], grads[1], grads[2], grads[3]


def qlora_multi_workspace_size(Ns, K: int, M: int, r: int) -> int:
    arr = (ctypes.c_int64 * len(Ns))(*[int(n) for n in Ns])
    return int(lib.qlora_multi_workspace_size(len(Ns), ctypes.cast(arr, ctypes.c_void_p), K, M, r))


def qlora_multi_fwd(ws, X, L1s, L2s, scale: float, keep_T: bool = True, workspace=None):
    """Forward of up to three linears sharing X (e.g. the q, k and v projections), each with its own
    adapter: returns ([Y_i], [T_i or None]).  From 1024 tokens one bf16 GEMM over the concatenated
    weights; the results equal qlora_linear_fwd's bit for bit."""
    torch = _torch()
    n = len(ws)
    if not (1 <= n <= 3) or len(L1s) != n or len(L2s) != n:
        raise ValueError("one to three weights, each with L1 and L2")
    _need(X, torch.bfloat16, "X")
    M, K = X.shape
    r = L1s[0].shape[1]
    for w, L1, L2 in zip(ws, L1s, L2s):
        _need(L1, torch.bfloat16, "L1")
        _need(L2, torch.bfloat16, "L2")
        if w.cols != K or tuple(L1.shape) != (K, r) or tuple(L2.shape) != (r, w.rows):
            raise ValueError("shape mismatch")
    Ys = [torch.empty((M, w.rows), dtype=torch.bfloat16, device=X.device) for w in ws]
    Ts = [torch.empty((M, r), dtype=torch.bfloat16, device=X.device) for _ in ws] if keep_T else [None] * n
    wsb = qlora_multi_workspace_size([w.rows for w in ws], K, M, r)
    wsp = _workspace(wsb, X.device, workspace)
    descs = [w.descriptor() for w in ws]
    P = ctypes.c_void_p
    dptr = (P * n)(*[ctypes.addressof(d) for d in descs])
    l1p = (P * n)(*[t.data_ptr() for t in L1s])
    l2p = (P * n)(*[t.data_ptr() for t in L2s])
    yp = (P * n)(*[t.data_ptr() for t in Ys])
    tp = (P * n)(*[t.data_ptr() for t in Ts]) if keep_T else None
    _check(lib.qlora_multi_fwd(n, ctypes.cast(dptr, P), _ptr(X), ctypes.cast(l1p, P), ctypes.cast(l2p, P),
                               float(scale), M, r, ctypes.cast(yp, P), ctypes.cast(tp, P) if keep_T else None,
                               _ptr(wsp), wsb, _stream(X.device)), "qlora_multi_fwd")
    return Ys, Ts


def qlora_swiglu_bwd(dh, g, u):
    torch = _torch()
    for t, n in ((dh, "dh"), (g, "g"), (u, "u")):
        _need(t, torch.bfloat16, n)
    dg = torch.empty_like(g)
    du = torch.empty_like(u)
    _check(lib.qlora_swiglu_bwd(_ptr(dh), _ptr(g), _ptr(u), _ptr(dg), _ptr(du), g.numel(),
                                _stream(g.device)), "qlora_swiglu_bwd")
    return dg, du


class GemmTimer:
    """HIP events bound by the library to each instrumented kernel launch (fused GEMMs, GEMV) on
    this thread."""

    def __init__(self, capacity: int):
        self._hip = ctypes.CDLL("libamdhip64.so.7")     # the runtime already loaded (by soname)
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.n = capacity
        self.begin = (ctypes.c_void_p * capacity)()
        self.end = (ctypes.c_void_p * capacity)()
        self.kinds = (ctypes.c_int32 * capacity)()
        for i in range(capacity):
            for arr in (self.begin, self.end):
                ev = ctypes.c_void_p()
                if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev.value

    def arm(self):
        _check(lib.nf4_set_gemm_timing_events(ctypes.cast(self.begin, ctypes.c_void_p),
                                              ctypes.cast(self.end, ctypes.c_void_p),
                                              ctypes.cast(self.kinds, ctypes.c_void_p), self.n),
               "nf4_set_gemm_timing_events")

    def arm_at(self, offset: int, n: int):
        """Record the next n instrumented launches into slots offset .. offset + n - 1."""
        if offset < 0 or n < 0 or offset + n > self.n:
            raise ValueError("timing slots out of range")
        size = ctypes.sizeof(ctypes.c_void_p)
        _check(lib.nf4_set_gemm_timing_events(ctypes.c_void_p(ctypes.addressof(self.begin) + offset * size),
                                              ctypes.c_void_p(ctypes.addressof(self.end) + offset * size),
                                              ctypes.c_void_p(ctypes.addressof(self.kinds) + offset * 4), n),
               "nf4_set_gemm_timing_events")

    def disarm(self) -> int:
        cnt = int(lib.nf4_gemm_timing_count())
        _check(lib.nf4_set_gemm_timing_events(None, None, None, 0), "nf4_set_gemm_timing_events")
        return cnt

    def durations_ms(self, count: int):
        """[(kind, ms)] of the recorded launches (call after a device synchronisation)."""
        out = []
        for i in range(count):
            ms = ctypes.c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.begin[i], self.end[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((int(self.kinds[i]), float(ms.value)))
        return out

    def close(self):
        for arr in (self.begin, self.end):
            for i in range(self.n):
                if arr[i]:
                    self._hip.hipEventDestroy(arr[i])
                    arr[i] = None
