"""Shared helpers of the GPU parity tests (upload, tolerances, comparisons)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from sparse_mixture_experts_19_amd import workloads as W

# Output tolerances of the block: largest per-token ratio
#   max_h |got - want| / max_h |want|
# against the float64 oracle.  bf16 inputs with fp32 accumulation: 2e-2;
# fp32 workloads: 1e-4.
TOL_OUT = {"bf16": 2e-2, "f32": 1e-4}
# Routing weights (fp32 softmax of fp32 logits vs the float64 oracle).
TOL_WEIGHTS = 1e-5
# Oracle logit gap below which two experts count as tied in float64 itself.
TIE_GAP = 1e-9


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Host array -> device tensor (bf16 arrays are uint16 bit patterns)."""
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(inp: W.Inputs, device="cuda"):
    dt = inp.wl.dtype
    return dict(
        x=dev_tensor(inp.x, dt, device),
        w_router=dev_tensor(inp.w_router, dt, device),
        bias=None if inp.bias is None else torch.from_numpy(inp.bias).to(device),
        w13=dev_tensor(inp.w13, dt, device),
        w2=dev_tensor(inp.w2, dt, device),
    )


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def row_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max over rows of max_h |got-want| / max_h |want|."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if got.size == 0:
        return 0.0
    num = np.abs(got - want).max(axis=1)
    den = np.maximum(np.abs(want).max(axis=1), 1e-30)
    return float((num / den).max())


def compare_ids(gpu_ids: np.ndarray, ora_ids: np.ndarray, ora_logits: np.ndarray):
    """Bit-exact ids, except tokens whose differing experts are tied in float64
    itself (gap < TIE_GAP): those are counted and returned."""
    diff = np.nonzero((gpu_ids != ora_ids).any(axis=1))[0]
    ties = []
    for t in diff:
        g, o = gpu_ids[t], ora_ids[t]
        # the GPU's choice must be a valid ordering of the same values
        gl, ol = ora_logits[t, g], ora_logits[t, o]
        assert len(set(g.tolist())) == len(g), f"token {t}: duplicate ids {g}"
        assert np.all(np.abs(gl - ol) < TIE_GAP), (
            f"token {t}: ids {g.tolist()} vs oracle {o.tolist()}, logits {gl} vs {ol}")
        ties.append(int(t))
    return ties


def sample_tokens(T: int, ids: np.ndarray, offsets: np.ndarray, perm: np.ndarray, k: int,
                  n_random: int = 16, seed: int = 1234, cap: int = 320):
    """Tokens for sampled output checks: the first and last row of every
    non-empty expert (so every active expert is used, including the ragged
    tail of its last row tile), both ends, and random ones.  When more than
    ``cap`` tokens are collected, only the random extras are dropped, never
    an expert's first or last row."""
    r = np.random.default_rng(seed)
    ends = set()
    E = len(offsets) - 1
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            ends.add(int(perm[a]) // k)
            ends.add(int(perm[b - 1]) // k)
    extra = set(range(min(4, T))) | set(range(max(0, T - 4), T))
    extra |= set(r.choice(T, size=min(n_random, T), replace=False).tolist())
    extra = sorted(extra - ends)
    room = max(0, cap - len(ends))
    if len(extra) > room:
        extra = r.choice(extra, size=room, replace=False).tolist()
    return sorted(ends | set(extra))


def oracle_outputs_all_tokens(inp: W.Inputs, ids: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """The block output of every token from the oracle's routing ``ids`` /
    ``weights``, computed expert by expert (the whole output tensor, float64)."""
    to_f32 = W.bf16_bits_to_f32 if inp.wl.dtype == "bf16" else None
    from oracle import moe_oracle as O
    return O.forward_tokens(inp.x, ids, weights, inp.w13, inp.w2, range(inp.wl.T), to_f32=to_f32)


def row_errors(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Per token row: max_h |got-want| / max_h |want|."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return np.abs(got - want).max(axis=1) / np.maximum(np.abs(want).max(axis=1), 1e-30)
