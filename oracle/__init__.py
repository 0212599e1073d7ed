"""CPU oracle for the NF4 quantized-codebook linear layer with a LoRA side branch.

TEST INFRASTRUCTURE ONLY.  This package is imported by the test-suite, by the smoke check and by
the CPU-baseline leg of the benchmark, and by nothing else.  It shares no code, header, table or
constant generator with the HIP library, and it never imports it.

What it computes, and where each step comes from (page: "QLoRA: Efficient Finetuning of
Quantized LLMs" study notes, gitcode.csdn.net/6a0046f754b52172bc72e356, unless noted):

* ``codebook``      -- section 3.2, eq. (4) and the asymmetric exact-zero construction;
                       section 5.1.2, Fig. 7 text (8 values on one half, 7 on the other, plus 0).
* ``codebook_int4``, ``codebook_fp4`` -- the 4-bit integer and 4-bit float types NF4 is compared
                       with (abstract page gitcode.csdn.net/69bbdcd90a2f6a37c5989d83, section 1;
                       study notes, section 5.1.2); the pages give no layout, so each is a
                       reading stated in its docstring.
* ``quantize``      -- section 3.1 (flatten, blocks of B, one constant per block), eq. (1) in its
                       absmax form, section 3.2 step 3 (absmax normalisation to [-1, 1]).  Any
                       ascending 16-entry table; equal neighbours allowed (the lower index wins).
* ``double_quant``  -- section 3.3 (mean-centred 8-bit float constants, block 256); with
                       ``fmt="int8"`` eq. (1) at 8 bits on the same centred constants (the
                       integer alternative to the pages' 8-bit float; a reading).
* ``dequant``       -- section 3.5, eq. (6), with eq. (2) at each level; output in BF16.
* ``forward``       -- section 3.5 eq. (5) with the scalar s of eq. (3) (section 4, LoRA).
* ``backward``      -- section 3.5: gradients for the adapters only, through the BF16 weight.
* ``swiglu_*``      -- not a step of the method: the gated MLP that the LLaMA-shaped workloads
                       wrap around three such linears.

The bit-exact steps (codebook, quantize, double quant, dequant, bf16 and E4M3 rounding) are plain
C in ``nf4_oracle.c``, built with gcc ``-O2 -ffp-contract=off``.  The linear-layer algebra is
plain float64 numpy: matrix products are library primitives, nothing is blocked or fused, and no
intermediate is rounded.

Pins (tests/test_oracle_pins.py) tie every function to something other than itself: the page's
printed numbers, closed forms, library routines (scipy's normal quantile, torch's bf16 and
float8_e4m3fn casts, torch autograd), exact rational brute force and finite differences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nf4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

#: Tail probability of the codebook grid (reading of the open constant in eq. 4): the midpoint
#: between the outermost-bin centres of a 16-value symmetric type (1 - 1/32) and of a 15-value
#: symmetric type with a zero (1 - 1/30).
DELTA_DEFAULT = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
BLOCK = 64          # first-level block (section 3.5: blocksize 64 for W)
DQ_BLOCK = 256      # second-level block (section 3.3: blocksize 256)
E4M3_MAX = 448.0


def build(force: bool = False) -> str:
    """Compile the C part of the oracle with gcc (no HIP involved)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            i64, i32, f64, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_float
            sig = {
                "oracle_norm_ppf": (f64, [f64]),
                "oracle_codebook": (ctypes.c_int, [f64, P]),
                "oracle_bf16_rne_vec": (None, [P, i64, P]),
                "oracle_e4m3_encode_vec": (None, [P, i64, P]),
                "oracle_e4m3_decode_vec": (None, [P, i64, P]),
                "oracle_quantize": (ctypes.c_int, [P, i64, i32, P, P, P]),
                "oracle_grouped_sum": (f64, [P, i64, i32]),
                "oracle_double_quant": (ctypes.c_int, [P, i64, i32, P, P, P]),
                "oracle_block_scales": (ctypes.c_int, [P, P, f32, i64, i32, P]),
                "oracle_dequant": (ctypes.c_int, [P, P, P, f32, i64, i32, i32, P, P]),
                "oracle_dequant_plain": (ctypes.c_int, [P, P, i64, i32, P, P]),
                "oracle_double_quant_int8": (ctypes.c_int, [P, i64, i32, P, P, P]),
                "oracle_block_scales_int8": (ctypes.c_int, [P, P, f32, i64, i32, P]),
                "oracle_dequant_int8dq": (ctypes.c_int, [P, P, P, f32, i64, i32, i32, P, P]),
                "oracle_unpack": (None, [P, i64, P]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ------------------------------------------------------------------------------------------
# Number formats
# ------------------------------------------------------------------------------------------

def norm_ppf(p: float) -> float:
    """Standard normal quantile by bisection on erfc (float64)."""
    return _load().oracle_norm_ppf(float(p))


def bf16_rne(x) -> np.ndarray:
    """float32 -> bfloat16 bits, nearest by value, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_rne_vec(_p(x), x.size, _p(out))
    return out


def bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def e4m3_encode(x) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 code: nearest finite value, ties to even, saturating, sign kept."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_vec(_p(x), x.size, _p(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    _load().oracle_e4m3_decode_vec(_p(c), c.size, _p(out))
    return out


# ------------------------------------------------------------------------------------------
# Codebook, quantize, double quant, dequant
# ------------------------------------------------------------------------------------------

def codebook(delta: float = DELTA_DEFAULT) -> np.ndarray:
    """The 16 NF4 values, ascending, float32 (index 7 is the exact zero)."""
    out = np.empty(16, dtype=np.float32)
    rc = _load().oracle_codebook(float(delta), _p(out))
    if rc != 0:
        raise ValueError("oracle_codebook failed (%d)" % rc)
    return out


def codebook_int4() -> np.ndarray:
    """4-bit integer codebook over the absmax-normalised value n = x / absmax.

    Neither page defines the Int4 type it compares NF4 against (abstract page, section 1;
    study notes, section 5.1.2).  Reading: eq. (1) of section 3.1 at 4 bits, round(7 / absmax *
    x) in [-7, 7], i.e. the codeword k / 7; the 16 codes are the two's complement integers
    k = -8 .. 7 in ascending order (code c holds k = c - 8).  k = -8 (value -8/7) lies outside
    [-1, 1] and is never the nearest codeword."""
    return np.array([(c - 8) / 7.0 for c in range(16)], dtype=np.float64).astype(np.float32)


def codebook_fp4() -> np.ndarray:
    """4-bit float codebook over n = x / absmax.

    The pages compare NF4 with FP4 (study notes, section 5.1.2, and Table 3 there) but do not
    give its layout.  Reading: E2M1 (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), divided by its largest magnitude 6 so that absmax maps
    to +-1.  In ascending order the sign-and-magnitude codes give 15 distinct values: the
    negative zero sits next to the positive one, both stored as +0.0, and the nearest-codeword
    rule (ties to the lower index) never produces the second."""
    mags = []
    for e in range(4):            # exponent field
        for m in range(2):        # mantissa field
            mags.append(m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m))
    mags.sort()
    vals = [-v / 6.0 for v in reversed(mags)] + [v / 6.0 for v in mags]
    return np.array([v if v != 0.0 else 0.0 for v in vals], dtype=np.float64).astype(np.float32)


def quantize(W, cb=None, block: int = BLOCK):
    """Level-1 quantization of the row-major flattening of ``W``.

    Returns (packed uint8 [ceil(n/2)], absmax float32 [ceil(n/block)])."""
    W = np.ascontiguousarray(W, dtype=np.float32).reshape(-1)
    cb = codebook() if cb is None else np.ascontiguousarray(cb, dtype=np.float32)
    n = W.size
    packed = np.zeros((n + 1) // 2, dtype=np.uint8)
    absmax = np.zeros((n + block - 1) // block, dtype=np.float32)
    rc = _load().oracle_quantize(_p(W), n, block, _p(cb), _p(packed), _p(absmax))
    if rc != 0:
        raise ValueError("oracle_quantize failed (%d)" % rc)
    return packed, absmax


def grouped_sum(v, group: int = 256) -> float:
    v = np.ascontiguousarray(v, dtype=np.float64)
    return _load().oracle_grouped_sum(_p(v), v.size, group)


DQ_FORMATS = ("e4m3", "int8")


def double_quant(absmax, dq_block: int = DQ_BLOCK, fmt: str = "e4m3"):
    """Level-2 quantization of the block constants: section 3.3's 8-bit float (E4M3), or with
    ``fmt="int8"`` eq. (1)'s 8-bit integers on the same centred constants.

    Returns (codes uint8 [nb], scales float32 [ceil(nb/dq_block)], mean float32)."""
    assert fmt in DQ_FORMATS
    a = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    nb = a.size
    codes = np.zeros(nb, dtype=np.uint8)
    scales = np.zeros((nb + dq_block - 1) // dq_block, dtype=np.float32)
    mean = np.zeros(1, dtype=np.float32)
    fn = _load().oracle_double_quant if fmt == "e4m3" else _load().oracle_double_quant_int8
    rc = fn(_p(a), nb, dq_block, _p(codes), _p(scales), _p(mean))
    if rc != 0:
        raise ValueError("oracle_double_quant failed (%d)" % rc)
    return codes, scales, np.float32(mean[0])


def block_scales(codes, scales, mean, dq_block: int = DQ_BLOCK, fmt: str = "e4m3") -> np.ndarray:
    """The rebuilt first-level constants a' (inner dequant of eq. 6)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    out = np.empty(codes.size, dtype=np.float32)
    fn = _load().oracle_block_scales if fmt == "e4m3" else _load().oracle_block_scales_int8
    fn(_p(codes), _p(scales), float(mean), codes.size, dq_block, _p(out))
    return out


def dequant(packed, codes, scales, mean, numel: int, cb=None, block: int = BLOCK,
            dq_block: int = DQ_BLOCK, fmt: str = "e4m3") -> np.ndarray:
    """Eq. (6): bf16 bit patterns [numel] of the double-dequantized weight."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    cb = codebook() if cb is None else np.ascontiguousarray(cb, dtype=np.float32)
    out = np.empty(numel, dtype=np.uint16)
    fn = _load().oracle_dequant if fmt == "e4m3" else _load().oracle_dequant_int8dq
    rc = fn(_p(packed), _p(codes), _p(scales), float(mean), numel, block, dq_block, _p(cb), _p(out))
    if rc != 0:
        raise ValueError("oracle_dequant failed (%d)" % rc)
    return out


def dequant_plain(packed, absmax, numel: int, cb=None, block: int = BLOCK) -> np.ndarray:
    """Eq. (2) with float32 block constants (no double quantization), bf16 bits."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    cb = codebook() if cb is None else np.ascontiguousarray(cb, dtype=np.float32)
    out = np.empty(numel, dtype=np.uint16)
    _load().oracle_dequant_plain(_p(packed), _p(absmax), numel, block, _p(cb), _p(out))
    return out


def unpack(packed, numel: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(numel, dtype=np.uint8)
    _load().oracle_unpack(_p(packed), numel, _p(out))
    return out


def quantize_dq(W, cb=None, fmt: str = "e4m3"):
    """Quantize + double-quantize a weight; returns a dict of the stored pieces."""
    W = np.asarray(W, dtype=np.float32)
    packed, absmax = quantize(W, cb)
    codes, scales, mean = double_quant(absmax, fmt=fmt)
    return {"packed": packed, "absmax": absmax, "codes": codes, "scales": scales, "mean": mean,
            "shape": W.shape, "fmt": fmt}


def dequant_weight(q, cb=None) -> np.ndarray:
    """bf16 bits of the weight described by ``quantize_dq``'s dict, reshaped."""
    n = int(np.prod(q["shape"]))
    return dequant(q["packed"], q["codes"], q["scales"], q["mean"], n, cb,
                   fmt=q.get("fmt", "e4m3")).reshape(q["shape"])


def bits_per_parameter(dq: bool, block: int = BLOCK, dq_block: int = DQ_BLOCK) -> float:
    """Storage per weight (section 3.3's accounting): 4-bit codes plus one float32 constant per
    block, or with DQ one 8-bit code per block plus one float32 per dq_block constants (the
    single float32 mean is not counted)."""
    return 4.0 + (8.0 / block + 32.0 / (block * dq_block) if dq else 32.0 / block)


def quant_error(W, cb=None, dq: bool = True, fmt: str = "e4m3") -> dict:
    """Quantization error of ``W`` under table ``cb`` (the comparison of section 5.1.2, on
    synthetic weights): the weight is quantized, double-quantized when ``dq``, dequantized to
    bf16 (eq. 6, or eq. 2 at one level without DQ), and compared with W in float64.

    Returns mse and max_abs of (deq - W), the count of elements per code (occupancy), the
    entropy of that distribution in bits, and bits_per_param."""
    W = np.ascontiguousarray(W, dtype=np.float32).reshape(-1)
    cb = codebook() if cb is None else np.ascontiguousarray(cb, dtype=np.float32)
    n = W.size
    packed, absmax = quantize(W, cb)
    if dq:
        codes, scales, mean = double_quant(absmax, fmt=fmt)
        deq = dequant(packed, codes, scales, mean, n, cb, fmt=fmt)
    else:
        deq = dequant_plain(packed, absmax, n, cb)
    err = bf16_to_f32(deq).astype(np.float64) - W.astype(np.float64)
    occ = np.bincount(unpack(packed, n), minlength=16).astype(np.int64)
    p = occ[occ > 0] / float(n)
    return {"mse": float(np.mean(err * err)), "max_abs": float(np.max(np.abs(err))),
            "occupancy": occ, "entropy_bits": float(-np.sum(p * np.log2(p))),
            "bits_per_param": bits_per_parameter(dq)}


# ------------------------------------------------------------------------------------------
# QLoRA linear layer, float64 (section 3.5 eq. 5 with the s of eq. 3)
# W is stored [N_out, K_in]; the pages' W (h x o) is its transpose, so Y = X deq(W)^T + ...
# ------------------------------------------------------------------------------------------

def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = bf16_to_f32(a)
    return a.astype(np.float64)


def forward(X, Wdq, L1, L2, s: float):
    """Y = X Wdq^T + s (X L1) L2.  Returns (Y, T) in float64; T = X L1 (unscaled)."""
    X, Wdq, L1, L2 = _f64(X), _f64(Wdq), _f64(L1), _f64(L2)
    T = X @ L1
    Y = X @ Wdq.T + float(s) * (T @ L2)
    return Y, T


def backward(dY, X, Wdq, L1, L2, s: float):
    """Gradients of E with respect to X, L1 and L2 given dE/dY; no gradient for W (frozen).

    dT = s dY L2^T;  dL2 = s (X L1)^T dY;  dL1 = X^T dT;  dX = dY Wdq + dT L1^T."""
    dY, X, Wdq, L1, L2 = _f64(dY), _f64(X), _f64(Wdq), _f64(L1), _f64(L2)
    s = float(s)
    T = X @ L1
    dT = s * (dY @ L2.T)
    dL2 = s * (T.T @ dY)
    dL1 = X.T @ dT
    dX = dY @ Wdq + dT @ L1.T
    return {"dX": dX, "dL1": dL1, "dL2": dL2, "dT": dT}


def forward_rows(X, Wdq, L1, L2, s: float, rows):
    """Forward for a subset of token rows only (full-size spot checks): each output row depends
    on its own token row alone."""
    X = _f64(np.asarray(X)[rows])
    Y, T = forward(X, Wdq, L1, L2, s)
    return Y, T


def backward_rows(dY, X, Wdq, L1, L2, s: float, rows=None):
    """``backward`` for full-size spot checks: the adapter gradients dL1 and dL2 sum over every
    token, so they take all rows; dX row i depends on dY row i alone (through dT row i), so it is
    evaluated on ``rows`` only (all rows when None).  Same formulas and order as ``backward``."""
    dY, X, L1, L2 = _f64(dY), _f64(X), _f64(L1), _f64(L2)
    s = float(s)
    T = X @ L1
    dT = s * (dY @ L2.T)
    dL2 = s * (T.T @ dY)
    dL1 = X.T @ dT
    sel = slice(None) if rows is None else rows
    dX = dY[sel] @ _f64(Wdq) + dT[sel] @ L1.T
    return {"dX": dX, "dL1": dL1, "dL2": dL2, "dT": dT, "T": T}


# ------------------------------------------------------------------------------------------
# SwiGLU glue for the MLP workloads (not a step of the method)
# ------------------------------------------------------------------------------------------

def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def swiglu_fwd(g, u) -> np.ndarray:
    """h = silu(g) * u, silu(g) = g * sigmoid(g); float64."""
    g, u = _f64(g), _f64(u)
    return g * _sigmoid(g) * u


def swiglu_bwd(dh, g, u):
    """(dg, du) for h = silu(g) * u."""
    dh, g, u = _f64(dh), _f64(g), _f64(u)
    sg = _sigmoid(g)
    du = dh * g * sg
    dg = dh * u * sg * (1.0 + g * (1.0 - sg))
    return dg, du


# ------------------------------------------------------------------------------------------
# Error measures used by the parity tests
# ------------------------------------------------------------------------------------------

REL_FRO_TOL = 5e-3
MAX_ABS_TOL = 2e-2


def rel_fro(got, ref) -> float:
    got, ref = _f64(got), _f64(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def max_abs_ratio(got, ref) -> float:
    got, ref = _f64(got), _f64(ref)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    return float(err / den) if den > 0 else float(err)


def within_tolerance(got, ref) -> bool:
    return rel_fro(got, ref) <= REL_FRO_TOL and max_abs_ratio(got, ref) <= MAX_ABS_TOL
