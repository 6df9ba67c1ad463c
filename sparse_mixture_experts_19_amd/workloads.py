"""Seeded synthetic workloads for the sparse top-k MoE FFN forward.

This module only *builds inputs*.  It holds none of the block's arithmetic
(no router, softmax, top-k, permutation, GEMM or combine), so both the CPU
oracle and the GPU path can be fed from it without sharing any of the
method's code.

Page legend (titles of the pages the workloads are described on):
  [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
  [Hunyuan page]   "混合专家架构大模型Hunyuan-Large：原理剖析与实现机制"

Generator recipe (every array is a pure function of (seed, config id,
tensor id, block id)):
  * numpy ``Generator(PCG64(SeedSequence([seed, config_id, tensor_id, block])))``
    drawing ``standard_normal(dtype=float32)`` in row-major order;
  * tensor ids: 0 = hidden states x (block = 1024-row chunk), 1 = router
    weight W_r [E,H] (block 0), 2 = gate/up weight W13[e] [2I,H] (gate rows
    first, block = expert e), 3 = down weight W2[e] [H,I] (block = expert e);
  * weights are scaled by float32(1/sqrt(fan_in)) with fan_in = H for W_r and
    W13 and I for W2, so every weight is N(0, 1/fan_in); x is N(0, 1);
  * bf16 workloads round the float32 draws to bf16 with round-to-nearest-even
    and keep them as raw uint16 bit patterns (numpy has no bf16 type).

The router bias b_g of the gating formula in [Hunyuan page] §二.1 is zero
unless a workload says otherwise; the skewed workload uses
b[e] = 2*ln(w_r / sum_j w_j) with Zipf weights w_r = r^-1.2 at rank r = e+1.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

X_CHUNK_ROWS = 1024

TENSOR_X = 0
TENSOR_WR = 1
TENSOR_W13 = 2
TENSOR_W2 = 3
TENSOR_WS13 = 4       # shared expert (optional)
TENSOR_WS2 = 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one MoE block workload."""

    name: str
    config_id: int
    T: int          # tokens (rows of x)
    H: int          # hidden size
    E: int          # number of experts
    k: int          # top-k
    I: int          # SwiGLU intermediate size per expert
    dtype: str      # "f32" or "bf16"
    renormalize: bool = False
    bias: str = "zero"   # "zero" or "zipf1.2"
    seed: int = 0

    @property
    def M(self) -> int:
        return self.T * self.k


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 512, 256, 8, 2, 512, "f32"),
    "coarse_bf16": Workload("coarse_bf16", 2, 4096, 4096, 8, 2, 14336, "bf16"),
    "fine_bf16": Workload("fine_bf16", 3, 16384, 2048, 128, 8, 768, "bf16",
                          renormalize=True),
    "vfine_bf16": Workload("vfine_bf16", 4, 8192, 4096, 256, 8, 256, "bf16"),
    "skewed_bf16": Workload("skewed_bf16", 5, 32768, 2048, 64, 4, 1024, "bf16",
                            bias="zipf1.2"),
}
WORKLOAD_ORDER = ["tiny_f32", "coarse_bf16", "fine_bf16", "vfine_bf16", "skewed_bf16"]


def scaled(w: Workload, **changes) -> Workload:
    """Same recipe with some sizes replaced (used for small parity cases)."""
    return dataclasses.replace(w, **changes)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, config_id: int, tensor: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [seed, config_id, tensor, block])))


def _draw(seed, config_id, tensor, block, shape, scale: Optional[float]) -> np.ndarray:
    a = _rng(seed, config_id, tensor, block).standard_normal(
        int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if scale is not None:
        a *= np.float32(scale)
    return a


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def zipf_bias(E: int, s: float = 1.2) -> np.ndarray:
    """b[e] = 2*ln(p_e) for Zipf(s) rank probabilities p_e, expert 0 = rank 1."""
    w = np.array([(r + 1.0) ** (-s) for r in range(E)], dtype=np.float64)
    return (2.0 * np.log(w / w.sum())).astype(np.float32)


@dataclasses.dataclass
class Inputs:
    """Host arrays of one workload.  bf16 tensors are uint16 bit patterns."""

    wl: Workload
    x: np.ndarray          # [T,H]
    w_router: np.ndarray   # [E,H]
    bias: Optional[np.ndarray]   # [E] float32 or None
    w13: np.ndarray        # [E,2I,H]
    w2: np.ndarray         # [E,H,I]

    def f32(self, name: str) -> np.ndarray:
        """Float32 view of an input (exact for bf16)."""
        a = getattr(self, name)
        if a is None:
            return None
        return bf16_bits_to_f32(a) if self.wl.dtype == "bf16" else a


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(wl: Workload, threads: Optional[int] = None,
                with_experts: bool = True) -> Inputs:
    """Draw every input of ``wl``.  Deterministic for a given workload."""
    T, H, E, I = wl.T, wl.H, wl.E, wl.I
    sid, cid = wl.seed, wl.config_id
    nthreads = threads or _threads()

    x = np.empty((T, H), dtype=np.uint16 if wl.dtype == "bf16" else np.float32)

    def x_chunk(c):
        r0 = c * X_CHUNK_ROWS
        r1 = min(T, r0 + X_CHUNK_ROWS)
        x[r0:r1] = _finish(_draw(sid, cid, TENSOR_X, c, (r1 - r0, H), None), wl.dtype)

    w_router = _finish(_draw(sid, cid, TENSOR_WR, 0, (E, H), 1.0 / math.sqrt(H)), wl.dtype)

    wdt = np.uint16 if wl.dtype == "bf16" else np.float32
    w13 = np.empty((E, 2 * I, H), dtype=wdt) if with_experts else None
    w2 = np.empty((E, H, I), dtype=wdt) if with_experts else None

    def w13_e(e):
        w13[e] = _finish(_draw(sid, cid, TENSOR_W13, e, (2 * I, H), 1.0 / math.sqrt(H)), wl.dtype)

    def w2_e(e):
        w2[e] = _finish(_draw(sid, cid, TENSOR_W2, e, (H, I), 1.0 / math.sqrt(I)), wl.dtype)

    jobs = [(x_chunk, c) for c in range((T + X_CHUNK_ROWS - 1) // X_CHUNK_ROWS)]
    if with_experts:
        jobs += [(w13_e, e) for e in range(E)] + [(w2_e, e) for e in range(E)]
    if nthreads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(lambda j: j[0](j[1]), jobs))
    else:
        for fn, arg in jobs:
            fn(arg)

    if wl.bias == "zero":
        bias = None
    elif wl.bias == "zipf1.2":
        bias = zipf_bias(E, 1.2)
    else:
        raise ValueError(f"unknown bias recipe {wl.bias!r}")
    return Inputs(wl, x, w_router, bias, w13, w2)


def make_shared_weights(wl: Workload, Is: int):
    """Weights of a shared expert with intermediate size Is for ``wl``: ws13
    [2Is,H] (gate rows then up rows, scale 1/sqrt(H)) and ws2 [H,Is] (scale
    1/sqrt(Is)), same recipe as the routed experts, own tensor ids."""
    H = wl.H
    ws13 = _finish(_draw(wl.seed, wl.config_id, TENSOR_WS13, 0, (2 * Is, H), 1.0 / math.sqrt(H)), wl.dtype)
    ws2 = _finish(_draw(wl.seed, wl.config_id, TENSOR_WS2, 0, (H, Is), 1.0 / math.sqrt(Is)), wl.dtype)
    return ws13, ws2


def random_small(T: int, H: int, E: int, k: int, I: int, dtype: str, seed: int,
                 renormalize: bool = False, bias: str = "zero") -> Inputs:
    """Small workload with the same recipe (config id 0) for parity sweeps."""
    wl = Workload(f"small_T{T}_H{H}_E{E}_k{k}_I{I}_{dtype}_s{seed}", 0, T, H, E, k, I,
                  dtype, renormalize=renormalize, bias=bias, seed=seed)
    return make_inputs(wl, threads=1)
