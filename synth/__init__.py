"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the bench.

This module only draws numbers: it holds none of the quantization or linear-layer
arithmetic.  Every tensor is a pure function of (seed, shape, distribution):

* uniform bits: SplitMix64 used as a counter-based generator (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014; the finaliser constants
  are the published ones).  Element ``i`` of stream ``seed`` is ``mix(seed + (i+1)*gamma)``.
* uniform doubles: the top 53 bits of each 64-bit word, scaled by 2**-53.
* normals: Box-Muller on consecutive pairs of uniforms, in float64, then scaled by the
  standard deviation and rounded once to float32 (round to nearest even).
* bf16 tensors: the float32 values rounded to bfloat16 by ``torch.Tensor.to``.

Seeds per tensor and the per-workload shapes live in ``WORKLOADS``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22
_THREADS = max(1, min(16, (__import__('os').cpu_count() or 1)))


def _splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of SplitMix64 stream ``seed`` (uint64)."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _chunks(n: int, chunk: int, fn) -> None:
    """Run fn(c0, c) over [0, n) in pieces of ``chunk``; pieces are independent (every element is
    a function of its index), so they run on a thread pool (numpy releases the GIL)."""
    starts = list(range(0, n, chunk))
    if len(starts) <= 1:
        for c0 in starts:
            fn(c0, min(chunk, n - c0))
        return
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(_THREADS, len(starts))) as ex:
        list(ex.map(lambda c0: fn(c0, min(chunk, n - c0)), starts))


def _uniform_into(out: np.ndarray, seed: int, start: int, c0: int, c: int) -> None:
    out[c0:c0 + c] = (_splitmix64(seed, start + c0, c) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform(seed: int, n: int, start: int = 0) -> np.ndarray:
    """``n`` doubles in [0, 1) from stream ``seed``."""
    out = np.empty(n, dtype=np.float64)
    _chunks(n, _CHUNK, lambda c0, c: _uniform_into(out, seed, start, c0, c))
    return out


def normal(seed: int, n: int) -> np.ndarray:
    """``n`` standard normal doubles (Box-Muller over word pairs 2j, 2j+1)."""
    out = np.empty(n, dtype=np.float64)
    pairs = (n + 1) // 2

    def piece(p0: int, p: int) -> None:
        u = np.empty(2 * p, dtype=np.float64)
        _uniform_into(u, seed, 2 * p0, 0, 2 * p)
        r = np.sqrt(-2.0 * np.log1p(-u[0::2]))   # 1 - u1 lies in (0, 1]
        th = (2.0 * math.pi) * u[1::2]
        z = np.empty(2 * p, dtype=np.float64)
        z[0::2] = r * np.cos(th)
        z[1::2] = r * np.sin(th)
        lo = 2 * p0
        hi = min(n, lo + 2 * p)
        out[lo:hi] = z[:hi - lo]

    _chunks(pairs, _CHUNK // 2, piece)
    return out


def normal_f32(seed: int, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    return (normal(seed, n) * std).astype(np.float32).reshape(shape)


def heavy_tail_f32(seed: int, mask_seed: int, shape, std: float, tail_std: float, frac: float) -> np.ndarray:
    """Each entry independently ~N(0, tail_std) with probability ``frac``, else ~N(0, std)."""
    n = int(np.prod(shape))
    z = normal(seed, n)
    tail = uniform(mask_seed, n) < frac
    return (z * np.where(tail, tail_std, std)).astype(np.float32).reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even, via torch), returned as uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------------
# Workloads: shapes and seeds.  W is stored [N_out, K_in] row-major; X is [M, K].
# ----------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Linear:
    name: str
    N: int            # output features (rows of W)
    K: int            # input features (cols of W)
    w_seed: int
    l1_seed: int
    l2_seed: int
    heavy_tail: bool = False


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    r: int
    alpha: float
    linears: tuple
    x_seed: int = 2000
    dy_seed: int = 5000
    w_std: float = 0.02
    x_std: float = 1.0
    l2_std: float = 0.01
    dy_std: float = 1.0
    swiglu: bool = False
    notes: str = ""

    @property
    def scale(self) -> float:
        return self.alpha / self.r


def _lin(name, N, K, i, heavy=False):
    return Linear(name, N, K, 1000 + i, 3000 + i, 4000 + i, heavy)


WORKLOADS = {
    "tiny": Workload("tiny", M=8, r=8, alpha=16.0, linears=(_lin("proj", 256, 256, 0),),
                     notes="256x256 linear, 8 tokens, r=8, alpha=16"),
    "llama7b_attn": Workload("llama7b_attn", M=4096, r=64, alpha=16.0,
                             linears=(_lin("proj", 4096, 4096, 0),),
                             notes="LLaMA-7B attention projection, 8x512 tokens"),
    "llama7b_mlp": Workload("llama7b_mlp", M=4096, r=64, alpha=16.0, swiglu=True,
                            linears=(_lin("gate", 11008, 4096, 0), _lin("up", 11008, 4096, 1),
                                     _lin("down", 4096, 11008, 2)),
                            notes="LLaMA-7B SwiGLU MLP, 4096 tokens"),
    "llama65b_mlp": Workload("llama65b_mlp", M=2048, r=64, alpha=16.0, swiglu=True,
                             linears=(_lin("gate", 22016, 8192, 0, True), _lin("up", 22016, 8192, 1, True),
                                      _lin("down", 8192, 22016, 2, True)),
                             notes="LLaMA-65B-shaped SwiGLU MLP, 2048 tokens, 1% heavy-tail weights"),
    "gemv": Workload("gemv", M=1, r=64, alpha=16.0, linears=(_lin("proj", 28672, 8192, 0),),
                     notes="decode-size dequant-GEMV, M in {1, 4, 16}"),
}

HEAVY_TAIL_STD = 0.2
HEAVY_TAIL_FRAC = 0.01


def weight_f32(wl: Workload, lin: Linear, rows: int | None = None) -> np.ndarray:
    shape = (lin.N if rows is None else rows, lin.K)
    if lin.heavy_tail:
        return heavy_tail_f32(lin.w_seed, lin.w_seed + 5000, shape, wl.w_std, HEAVY_TAIL_STD, HEAVY_TAIL_FRAC)
    return normal_f32(lin.w_seed, shape, wl.w_std)


def lora_f32(wl: Workload, lin: Linear):
    """(L1 [K, r] ~ N(0, 1/r), L2 [r, N] ~ N(0, l2_std)) as float32."""
    l1 = normal_f32(lin.l1_seed, (lin.K, wl.r), 1.0 / wl.r)
    l2 = normal_f32(lin.l2_seed, (wl.r, lin.N), wl.l2_std)
    return l1, l2


def x_f32(wl: Workload, M: int | None = None, K: int | None = None) -> np.ndarray:
    M = wl.M if M is None else M
    K = wl.linears[0].K if K is None else K
    return normal_f32(wl.x_seed, (M, K), wl.x_std)


def dy_f32(wl: Workload, M: int, N: int) -> np.ndarray:
    return normal_f32(wl.dy_seed, (M, N), wl.dy_std)
