"""CPU oracle of the sparse top-k MoE FFN forward (test infrastructure).

This is the plain, slow, obviously-correct reference the HIP path is checked
against.  It is *test infrastructure*: only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import or
run it.  The product library never calls it and shares no code with it.

Everything is numpy in float64.  Inputs arrive as float32 arrays (bf16 inputs
are widened to float32 exactly by the caller), so every product of two inputs
is exact in float64 and each dot product carries only float64 summation error.

Page legend (titles of the pages the steps are taken from):
  [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
  [Hunyuan page]   "混合专家架构大模型Hunyuan-Large：原理剖析与实现机制"
  [SonicMoE page]  "SonicMoE与传统MoE架构对比：Token舍入技术如何实现训练效率跃升"

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):
  * top-k orders experts by descending logit, ties to the lowest expert index,
    slot j holding the (j+1)-th largest; selection is made on logits, which
    gives the same set and order as selecting on the softmax probabilities
    because softmax is strictly increasing;
  * the routing weight multiplies the expert output after the down
    projection (the weighted sum of expert outputs of [Qwen3-MoE page] §1,
    phase 4), and is optionally renormalised over the k selected experts;
  * the expert MLP is SwiGLU: W2 @ (silu(Wg @ x) * (Wu @ x)), with W13[e]
    holding the gate rows Wg first and the up rows Wu after them;
  * the permutation is stable over the flat assignment index f = t*k + j;
  * the shared expert (optional) is a dense SwiGLU expert over every token
    whose output is added with weight 1 to the routed sum;
  * token rounding (optional) follows the integer rule in ``token_round``;
  * MXFP8 (optional): expert GEMMs on e4m3 values with E8M0 block scales of
    32 along the reduction axis (``mx_quantize``), router unquantized;
  * the backward (``backward``) differentiates L = sum(dout * out) with the
    top-k choice held fixed (it is piecewise constant).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
something other than itself (brute force, closed forms, library routines,
special cases, invariants, metamorphic relations).  Nothing is "parity
unpinned".
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Steps 1-3: router linear layer, softmax over all experts, top-k.
# ---------------------------------------------------------------------------

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """Router linear layer: l[t,e] = sum_h x[t,h] * W_r[e,h] + b[e].

    [Qwen3-MoE page] §1 forward listing: the gate is a linear layer applied
    to the flattened hidden states; [Hunyuan page] §二.1 gating formula: the
    gate is W_g x + b_g.  W_r is stored (out, in) = [E, H].
    """
    l = _f64(x) @ _f64(w_router).T
    if bias is not None:
        l = l + _f64(bias)[None, :]
    return l


def softmax_all(logits) -> np.ndarray:
    """Softmax over *all* experts of each token, in float64.

    [Qwen3-MoE page] §1 forward listing (softmax along the expert dimension,
    before top-k); [Hunyuan page] §二.1 gating formula G(x) = Softmax(W_g x + b_g).
    The max is subtracted first; this does not change the value.
    """
    l = _f64(logits)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def topk_ids(logits, k: int) -> np.ndarray:
    """Per-token top-k expert ids, int32 [T, k].

    [Qwen3-MoE page] §1 forward listing (topk over the routing scores).
    Order: descending logit, ties to the lowest expert index, slot j = rank j.
    numpy's lexsort sorts by the last key first: key (-logit), then expert id.
    """
    l = _f64(logits)
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    eid = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((eid, -l), axis=-1)
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def route(x, w_router, bias, k: int, renormalize: bool):
    """Steps 1-3 together: returns ids [T,k] int32 and weights [T,k] float64.

    The weight of slot j is the softmax probability of the chosen expert
    ([Qwen3-MoE page] §1 forward listing keeps the top-k probabilities);
    with ``renormalize`` the k weights of a token are divided by their sum.
    Also returns the logits and probabilities for the tests.
    """
    l = router_logits(x, w_router, bias)
    p = softmax_all(l)
    ids = topk_ids(l, k)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w, l, p


# ---------------------------------------------------------------------------
# Step 4: permutation that groups assignment rows by expert.
# ---------------------------------------------------------------------------

def permute(ids, E: int):
    """Expert histogram, offsets and the stable expert-sorted permutation.

    [Qwen3-MoE page] §2.2 memory-access optimisation (reorder the tokens by
    their assigned expert so each expert reads a contiguous block) and its
    optimised forward pseudocode (sort by expert, gather, scatter back).

    For the flat assignment index f = t*k + j (token t, slot j):
      counts[e]   = number of f with ids.flat[f] == e
      offsets     = [0, cumsum(counts)]            (length E+1)
      perm[r]     = f of the r-th row in (expert, f) order   (stable)
      inv_perm[f] = r such that perm[r] == f
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    if counts.shape[0] != E:
        raise ValueError("expert id out of range")
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.shape[0], dtype=np.int32)
    return counts, offsets.astype(np.int32), perm, inv


def gather_rows(x, perm, k: int) -> np.ndarray:
    """x_perm[r] = x[perm[r] // k]: the reordered hidden states.

    [Qwen3-MoE page] §2.2 optimised forward pseudocode (reordered states).
    """
    return np.asarray(x)[np.asarray(perm, dtype=np.int64) // k]


# ---------------------------------------------------------------------------
# Steps 5-6: per-expert SwiGLU MLP over the rows each expert owns.
# ---------------------------------------------------------------------------

def silu(z) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_mlp(xe, w13_e, w2_e) -> np.ndarray:
    """One expert's SwiGLU MLP on rows xe [n,H]: W2 (silu(Wg x) * (Wu x)).

    The pages only call each expert a small MLP ([Qwen3-MoE page] §1); the
    SwiGLU form, with gate rows then up rows stacked in W13 [2I,H] and the
    down weight W2 [H,I], is the reading taken for this block.
    """
    w13_e = _f64(w13_e)
    I = w13_e.shape[0] // 2
    xe = _f64(xe)
    g = xe @ w13_e[:I].T
    u = xe @ w13_e[I:].T
    h = silu(g) * u
    return h @ _f64(w2_e).T


def experts(x, perm, offsets, w13, w2, k: int) -> np.ndarray:
    """Grouped expert compute: Y[r] = expert_{e(r)}(x[perm[r] // k]).

    [Qwen3-MoE page] §1 forward listing (loop over experts, each applied to
    the tokens routed to it) and §2.1 (all experts in one batched compute);
    the rows of expert e are offsets[e]..offsets[e+1]-1 of the permutation.
    Empty experts are skipped and their weights never read.
    """
    x = _f64(x)
    M = int(offsets[-1])
    H = x.shape[1]
    Y = np.zeros((M, H), dtype=np.float64)
    E = len(offsets) - 1
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        rows = np.asarray(perm[r0:r1], dtype=np.int64) // k
        Y[r0:r1] = expert_mlp(x[rows], w13[e], w2[e])
    return Y


# ---------------------------------------------------------------------------
# Step 7: routing-weighted combine back to token order.
# ---------------------------------------------------------------------------

def combine(Y, inv_perm, weights, T: int, k: int) -> np.ndarray:
    """out[t] = sum_{j<k} w[t,j] * Y[inv_perm[t*k + j]].

    [Qwen3-MoE page] §1 phase 4 (outputs summed with the routing weights)
    and §2.2 pseudocode (scatter the expert outputs back to token order).
    """
    Y = _f64(Y)
    w = _f64(weights).reshape(T, k)
    inv = np.asarray(inv_perm, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * Y[inv[:, j]]
    return out


# ---------------------------------------------------------------------------
# Whole block.
# ---------------------------------------------------------------------------

def forward(x, w_router, bias, w13, w2, k: int, renormalize: bool) -> Dict[str, np.ndarray]:
    """The MoE block forward: route, permute, grouped SwiGLU, combine.

    Step order of the optimised forward pseudocode of [Qwen3-MoE page] §2.2
    (routing, reorder by expert, batched expert compute, scatter back).
    Returns the output and every intermediate, all float64 / int32.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    ids, w, l, p = route(x, w_router, bias, k, renormalize)
    counts, offsets, perm, inv = permute(ids, E)
    Y = experts(x, perm, offsets, w13, w2, k)
    out = combine(Y, inv, w, T, k)
    return dict(out=out, ids=ids, weights=w, logits=l, probs=p, counts=counts,
                offsets=offsets, perm=perm, inv_perm=inv, Y=Y)


# ---------------------------------------------------------------------------
# Shared expert.
# ---------------------------------------------------------------------------

def shared_expert(x, ws13, ws2) -> np.ndarray:
    """The shared expert: one SwiGLU MLP applied to every token, weight 1.

    [Hunyuan page] §二.1 routes tokens through a shared-expert pool besides the
    gated experts and gives no formula for it.  Reading taken: a dense expert
    of the same SwiGLU form as the routed ones (gate rows then up rows in
    ws13 [2Is,H], down weight ws2 [H,Is], its own intermediate size Is) whose
    output is added, unweighted, to the routed sum.
    """
    return expert_mlp(x, ws13, ws2)


def forward_shared(x, w_router, bias, w13, w2, ws13, ws2, k: int,
                   renormalize: bool) -> Dict[str, np.ndarray]:
    """MoE block with a shared expert: out = sum_j w[t,j] Y_j + S(x_t).

    The routed part is ``forward``; S is ``shared_expert``.  Returns every
    intermediate of ``forward`` plus S and the routed-only output.
    """
    res = forward(x, w_router, bias, w13, w2, k, renormalize)
    S = shared_expert(x, ws13, ws2)
    res["out_routed"] = res["out"]
    res["S"] = S
    res["out"] = res["out"] + S
    return res


# ---------------------------------------------------------------------------
# Token rounding (routing variant).
# ---------------------------------------------------------------------------

def _round_pool(ids, E: int, B: int):
    """Kept row counts floor(c_e/B)*B and the pooled flat indices (flat order)."""
    counts, offsets, perm, inv = permute(ids, E)
    keep = (counts // B) * B
    pooled = np.zeros(np.asarray(ids).size, dtype=bool)
    for e in range(E):
        pooled[perm[offsets[e] + keep[e]:offsets[e + 1]]] = True
    return keep, [int(f) for f in np.nonzero(pooled)[0]]


def _round_order(load):
    """Experts in the order a pooled tile is offered to them: load, then id."""
    return sorted(range(len(load)), key=lambda q: (load[q], q))


def _round_eligible(cur, t: int, j: int, e: int) -> bool:
    """Slot j of token t may move to e if no other slot of t holds e."""
    return all(cur[t, jj] != e for jj in range(cur.shape[1]) if jj != j)


def _round_weights(probs, ids, renormalize: bool):
    """Weight of each slot: the token's softmax probability of its expert."""
    w = _f64(probs)[np.arange(ids.shape[0])[:, None], ids]
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def token_round(ids, probs, E: int, B: int, renormalize: bool):
    """Token rounding: re-route assignments so expert row counts are tile multiples.

    [SonicMoE page] 核心差异 §3: each expert's assignment count is rounded
    down to a multiple of the tile size and the remaining tokens are given to
    the least-loaded experts, which removes the tile padding of the grouped
    GEMM.  The page's listing of this step is garbled and works on counts
    only; it does not say which token moves where.  The rule taken here, with
    every decision on integers:

    1. Expert e keeps the first floor(c_e / B) * B rows of its segment of the
       stable expert-sorted permutation (assignments in flat order f = t*k+j);
       the rest of its rows go to a pool.
    2. The pool is handed out in tiles of B rows, each to the least-loaded
       expert (rows kept plus rows received; ties to the lowest id) that can
       still take rows.  A tile takes up to B of the pooled assignments, in
       flat order, whose token holds the owner in no other slot, at most one
       slot per token.  A tile that takes nothing marks its owner as unable.
       The owners are planned a round at a time: a round with P pooled
       assignments left opens ceil(P / B) tiles and gives them out by
       water-filling (B rows per planned tile), as the page's listing spreads
       the remainder count over the rounded counts before any token moves;
       then the tiles are filled in order, and what a round leaves goes to
       the next one with the loads actually reached.
    3. A moved assignment keeps its slot j; its weight is the token's softmax
       probability of the new expert, renormalised over the token's k weights
       when the workload renormalises (unmoved slots keep the same formula).

    Planning a round ahead gives the same ids as choosing each tile's owner
    from the loads actually reached so far.  The two differ only after a tile
    comes out short (fewer than B rows), and such a tile has scanned the whole
    pool: every pooled slot it skipped belongs to a token that now holds its
    owner, or that held it in a slot the tile itself took (pooled slots of the
    owner are always eligible, and taken slots never move again).  So its
    owner can never take another row, whichever rule offers it more tiles.

    ids [T,k] int, probs [T,E] float64 (softmax over all experts).  Returns
    (new ids [T,k] int32, new weights [T,k] float64, moved [T,k] bool).
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    keep, pool = _round_pool(ids, E, B)
    load = keep.astype(np.int64).copy()
    unable = np.zeros(E, dtype=bool)
    cur = ids.astype(np.int32).copy()
    taken = [False] * len(pool)
    left = len(pool)
    while left:
        plan = load.copy()
        owners = []
        for _ in range(-(-left // B)):
            order = [e for e in _round_order(plan) if not unable[e]]
            if not order:
                raise RuntimeError("no expert can take a pooled assignment")   # needs k >= E
            owners.append(order[0])
            plan[order[0]] += B
        for e in owners:
            got, seen = 0, set()
            for i, f in enumerate(pool):
                if got == B:
                    break
                if taken[i]:
                    continue
                t, j = divmod(f, k)
                if t in seen or not _round_eligible(cur, t, j, e):
                    continue
                cur[t, j] = e
                taken[i] = True
                seen.add(t)
                got += 1
            load[e] += got
            left -= got
            if got == 0:
                unable[e] = True
    return cur, _round_weights(probs, cur, renormalize), cur != ids


def forward_rounded(x, w_router, bias, w13, w2, k: int, renormalize: bool,
                    B: int) -> Dict[str, np.ndarray]:
    """MoE block with token rounding (``token_round``, tile B) between routing
    and the permutation.  Returns the output and every intermediate."""
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    ids0, w0, l, p = route(x, w_router, bias, k, renormalize)
    ids, w, moved = token_round(ids0, p, E, B, renormalize)
    counts, offsets, perm, inv = permute(ids, E)
    Y = experts(x, perm, offsets, w13, w2, k)
    out = combine(Y, inv, w, T, k)
    return dict(out=out, ids=ids, weights=w, moved=moved, ids_topk=ids0, weights_topk=w0,
                logits=l, probs=p, counts=counts, offsets=offsets, perm=perm, inv_perm=inv, Y=Y)


# ---------------------------------------------------------------------------
# MXFP8 expert GEMMs (reduced-precision variant).
# ---------------------------------------------------------------------------
# [Hunyuan page] §七.1 says FP8 quantization needs the routing to be
# re-checked; the reading here keeps the router on the unquantized inputs
# (so its decisions do not move) and runs the expert GEMMs in the OCP MX
# format MXFP8: e4m3 elements, one E8M0 (power-of-two) scale per 32
# consecutive values along the reduction axis.

def _e4m3_values() -> np.ndarray:
    """Value of every e4m3 code 0..255 (OCP FP8 E4M3: bias 7, no infinities,
    S.1111.111 is NaN), in float64."""
    v = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
        elif e == 0:
            v[c] = (-1) ** s * 2.0 ** -6 * (m / 8)
        else:
            v[c] = (-1) ** s * 2.0 ** (e - 7) * (1 + m / 8)
    return v


E4M3 = _e4m3_values()
E4M3_MAX = 448.0
_POS_CODES = np.array([c for c in range(127)])          # 0x00..0x7E: +0 .. +448, increasing


def e4m3_encode(y) -> np.ndarray:
    """Nearest e4m3 code to each value (ties to the even code), saturating at
    +-448; float64 in, uint8 codes out."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    vals = E4M3[_POS_CODES]
    hi = np.searchsorted(vals, a, side="left")            # first value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = _POS_CODES[pick]
    return (code | np.where(np.signbit(y) & (code != 0), 0x80, 0)).astype(np.uint8)


def _mx_exponent(amax) -> np.ndarray:
    """Shared block exponent floor(log2 amax) - 8 (8 = emax of e4m3), clamped
    to the E8M0 range [-127, 127]; an all-zero block takes -127."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    ex = np.where(amax > 0, np.floor(np.log2(safe)) - 8, -127)
    return np.clip(ex, -127, 127)


def mx_quantize(v, block: int = 32):
    """MXFP8 quantization along the last axis (OCP MX v1.0 §6.3): per block of
    32 values, shared exponent floor(log2 amax) - 8 (8 = emax of e4m3), clamped
    to the E8M0 range [-127, 127] (an all-zero block takes -127); elements
    e4m3(v / 2^exp).  Returns (codes uint8 [..., K], scales uint8 [..., K/32]
    (biased: exp + 127), dequantized float64)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    b = v.reshape(v.shape[:-1] + (K // block, block))
    ex = _mx_exponent(np.abs(b).max(axis=-1))
    scale = np.ldexp(1.0, ex.astype(np.int64))
    codes = e4m3_encode(b / scale[..., None])
    deq = E4M3[codes] * scale[..., None]
    return (codes.reshape(v.shape), (ex + 127).astype(np.uint8),
            deq.reshape(v.shape))


def mx_dequantize(codes, scales, block: int = 32) -> np.ndarray:
    codes = np.asarray(codes)
    K = codes.shape[-1]
    sc = np.ldexp(1.0, np.asarray(scales).astype(np.int64) - 127)
    return (E4M3[codes].reshape(codes.shape[:-1] + (K // block, block)) * sc[..., None]).reshape(codes.shape)


def expert_h_mxfp8(xe, w13q_e, w13s_e):
    """One expert's h = silu(x Wg^T) * (x Wu^T) on MXFP8 operands (its rows of
    x quantized along H; products and sums in float64), quantized along I:
    (codes, scales, dequantized) as ``mx_quantize``, then h itself."""
    xd = mx_quantize(xe)[2]
    w13 = mx_dequantize(w13q_e, w13s_e)
    I = w13.shape[0] // 2
    h = silu(xd @ w13[:I].T) * (xd @ w13[I:].T)
    return mx_quantize(h) + (h,)


def expert_mlp_mxfp8(xe, w13q_e, w13s_e, w2q_e, w2s_e) -> np.ndarray:
    """One expert's SwiGLU MLP on MXFP8 operands: its rows of x and its h are
    quantized along their reduction axes; products and sums in float64."""
    hd = expert_h_mxfp8(xe, w13q_e, w13s_e)[2]
    return hd @ mx_dequantize(w2q_e, w2s_e).T


def forward_mxfp8(x, w_router, bias, w13q, w13s, w2q, w2s, k: int,
                  renormalize: bool) -> Dict[str, np.ndarray]:
    """The block with MXFP8 expert GEMMs: routing, permutation and combine as
    in ``forward``; each expert runs ``expert_mlp_mxfp8`` on its rows.
    w13q [E,2I,H] / w13s [E,2I,H/32] and w2q [E,H,I] / w2s [E,H,I/32] are
    the quantized expert weights (``mx_quantize`` of bf16/fp32 weights).
    Hq / Hs are the codes and scales of h and H is h before quantization,
    row r for permuted row r."""
    x = np.asarray(x)
    T = x.shape[0]
    E, I2 = np.asarray(w13q).shape[:2]
    I = I2 // 2
    ids, w, l, p = route(x, w_router, bias, k, renormalize)
    counts, offsets, perm, inv = permute(ids, E)
    xp = gather_rows(x, perm, k)
    M = xp.shape[0]
    Y = np.zeros((M, np.asarray(w2q).shape[1]))
    Hq = np.zeros((M, I), dtype=np.uint8)
    Hs = np.zeros((M, I // 32), dtype=np.uint8)
    Hf = np.zeros((M, I))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            Hq[a:b], Hs[a:b], hd, Hf[a:b] = expert_h_mxfp8(xp[a:b], w13q[e], w13s[e])
            Y[a:b] = hd @ mx_dequantize(w2q[e], w2s[e]).T
    out = combine(Y, inv, w, T, k)
    return dict(out=out, ids=ids, weights=w, logits=l, probs=p, counts=counts,
                offsets=offsets, perm=perm, inv_perm=inv, Y=Y, Hq=Hq, Hs=Hs, H=Hf)


# ---------------------------------------------------------------------------
# Backward of the block (the gradients of a training step).
# ---------------------------------------------------------------------------
# [SonicMoE page] 核心差异 §1 keeps only the gate outputs and the final expert
# outputs of the forward and recomputes the rest in the backward; [Hunyuan
# page] §二.2 gives parameter gradients only to the experts a token
# activated.  The top-k choice is piecewise constant, so the gradients flow
# through the selected experts' routing weights and MLPs; the loss is
# L = sum(dout * out) for an upstream gradient dout [T,H].

def silu_grad(z) -> np.ndarray:
    """d silu(z) / dz = s (1 + z (1 - s)) with s = 1 / (1 + e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def weights_grad(dw, probs_sel, renormalize: bool) -> np.ndarray:
    """Gradient with respect to the selected probabilities [T,k] from the
    gradient dw of the routing weights: the identity, or, through the
    renormalisation w_j = p_j / S with S = sum_i p_i,
    (dw_j - sum_i dw_i w_i) / S."""
    dw = _f64(dw)
    if not renormalize:
        return dw
    ps = _f64(probs_sel)
    S = ps.sum(axis=1, keepdims=True)
    w = ps / S
    return (dw - (dw * w).sum(axis=1, keepdims=True)) / S


def softmax_grad(p, dp) -> np.ndarray:
    """Gradient with respect to the logits of p = softmax(l):
    p * (dp - sum_e dp_e p_e) per token."""
    p, dp = _f64(p), _f64(dp)
    return p * (dp - (dp * p).sum(axis=1, keepdims=True))


def expert_mlp_backward(xe, w13_e, w2_e, dy):
    """One expert's SwiGLU MLP backward for its rows xe and their output
    gradient dy (the routing weight already applied), with g, u and h
    recomputed from xe: (dx of the rows, dW13_e, dW2_e)."""
    xe, w13_e, w2_e, dy = _f64(xe), _f64(w13_e), _f64(w2_e), _f64(dy)
    I = w13_e.shape[0] // 2
    g = xe @ w13_e[:I].T
    u = xe @ w13_e[I:].T
    h = silu(g) * u
    dw2 = dy.T @ h
    dh = dy @ w2_e
    dg = dh * u * silu_grad(g)
    du = dh * silu(g)
    dw13 = np.concatenate([dg.T @ xe, du.T @ xe])
    return dg @ w13_e[:I] + du @ w13_e[I:], dw13, dw2


def backward(x, w_router, bias, w13, w2, k: int, renormalize: bool, dout) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(dout * out) for the block of ``forward``: dx
    [T,H], dw_router [E,H], dbias [E], dw13 [E,2I,H], dw2 [E,H,I]; also dw
    [T,k] (routing weights) and dlogits [T,E].  The forward's routing, its
    permutation and its expert outputs Y are reused; g, u and h are
    recomputed per expert."""
    fw = forward(x, w_router, bias, w13, w2, k, renormalize)
    x, w_router, dout = _f64(x), _f64(w_router), _f64(dout)
    T, H = x.shape
    E = np.asarray(w13).shape[0]
    ids, w, p = fw["ids"], fw["weights"], fw["probs"]
    perm, offsets, inv = fw["perm"], fw["offsets"], fw["inv_perm"]
    # routing weights: out_t = sum_j w_tj y_tj, so dL/dw_tj = <dout_t, y_tj>
    y_slots = fw["Y"][inv].reshape(T, k, H)
    dw = (dout[:, None, :] * y_slots).sum(axis=2)
    # experts, on the permuted rows
    xp = gather_rows(x, perm, k)
    dp_rows = gather_rows(dout, perm, k)
    w_rows = w.reshape(-1)[perm]
    dxp = np.zeros_like(xp)
    dw13 = np.zeros(np.asarray(w13).shape)
    dw2 = np.zeros(np.asarray(w2).shape)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            dy = w_rows[a:b, None] * dp_rows[a:b]
            dxp[a:b], dw13[e], dw2[e] = expert_mlp_backward(xp[a:b], w13[e], w2[e], dy)
    dx = combine(dxp, inv, np.ones((T, k)), T, k)
    # router: through the selected probabilities and the softmax
    dp = np.zeros((T, E))
    np.put_along_axis(dp, ids, weights_grad(dw, np.take_along_axis(p, ids, axis=1), renormalize),
                      axis=1)
    dl = softmax_grad(p, dp)
    dx = dx + dl @ w_router
    return dict(dx=dx, dw_router=dl.T @ x, dbias=dl.sum(axis=0), dw13=dw13, dw2=dw2, dw=dw,
                dlogits=dl, fw=fw)


def backward_sampled(x, w_router, bias, w13, w2, k: int, renormalize: bool, dout,
                     tokens: Sequence[int], cols: Sequence[int],
                     to_f32=None) -> Dict[str, np.ndarray]:
    """Parts of ``backward`` for workloads too large to run it whole: dx,
    dlogits and dw of the given tokens, and per expert the columns
    dW2[e][:, i] and the rows dW13[e][i], dW13[e][I + i] for i in ``cols``.

    With the top-k choice fixed a token's input gradient depends only on its
    own row, routing and dout row (g, u and h recomputed from that row, as
    [SonicMoE page] 核心差异 §1 recomputes them), and one column or row of a
    weight gradient only on the expert's rows ([Hunyuan page] §二.2: the
    tokens that activated it) and one row of each of its matrices.  The
    algebra is that of ``backward``.  ``to_f32`` widens stored values (bf16
    bit patterns) expert by expert, as in ``forward_tokens``.
    """
    conv = to_f32 if to_f32 is not None else (lambda a: a)
    tokens = np.asarray([int(t) for t in tokens], dtype=np.int64)
    cols = np.asarray([int(c) for c in cols], dtype=np.int64)
    X = _f64(conv(np.asarray(x)))
    wr = _f64(conv(np.asarray(w_router)))
    dout = _f64(dout)
    T, H = X.shape
    E = np.asarray(w13).shape[0]
    ids, w, _, p = route(X, wr, bias, k, renormalize)
    counts, offsets, perm, inv = permute(ids, E)
    ids64 = ids.astype(np.int64)
    n = len(tokens)
    dx = np.zeros((n, H))
    dw = np.zeros((n, k))
    dw2_cols = np.zeros((E, H, len(cols)))
    dw13_rows = np.zeros((E, 2, len(cols), H))
    for e in range(E):
        si, sj = np.nonzero(ids64[tokens] == e)     # sampled (token, slot) pairs on e
        a, b = int(offsets[e]), int(offsets[e + 1])
        if len(si) == 0 and b == a:
            continue
        w13_e, w2_e = _f64(conv(w13[e])), _f64(conv(w2[e]))
        I = w13_e.shape[0] // 2
        if len(si):
            ts = tokens[si]
            xs = X[ts]
            g, u = xs @ w13_e[:I].T, xs @ w13_e[I:].T
            y = (silu(g) * u) @ w2_e.T
            dw[si, sj] = (dout[ts] * y).sum(axis=1)
            dh = (w[ts, sj][:, None] * dout[ts]) @ w2_e
            dg, du = dh * u * silu_grad(g), dh * silu(g)
            np.add.at(dx, si, dg @ w13_e[:I] + du @ w13_e[I:])
        if b > a:
            f = perm[a:b].astype(np.int64)            # the expert's rows, flat indices
            xe = X[f // k]
            dy = w.reshape(-1)[f][:, None] * dout[f // k]
            gc, uc = xe @ w13_e[cols].T, xe @ w13_e[I + cols].T
            dw2_cols[e] = dy.T @ (silu(gc) * uc)
            dhc = dy @ w2_e[:, cols]
            dw13_rows[e, 0] = (dhc * uc * silu_grad(gc)).T @ xe
            dw13_rows[e, 1] = (dhc * silu(gc)).T @ xe
    ps = p[tokens]
    dp = np.zeros_like(ps)
    np.put_along_axis(dp, ids64[tokens], weights_grad(dw, np.take_along_axis(ps, ids64[tokens], axis=1),
                                                      renormalize), axis=1)
    dl = softmax_grad(ps, dp)
    dx = dx + dl @ wr
    return dict(dx=dx, dlogits=dl, dw=dw, dw2_cols=dw2_cols, dw13_rows=dw13_rows, ids=ids,
                counts=counts)


def forward_tokens(x, ids, weights, w13, w2, tokens: Sequence[int],
                   to_f32=None) -> np.ndarray:
    """Block output for a subset of tokens, one token at a time.

    A token's output depends only on its own row, its k ids and weights
    ([Qwen3-MoE page] §1: each selected expert processes the token, the
    results are summed with the routing weights), so large workloads are
    checked on sampled tokens.  ``ids``/``weights`` are the oracle's routing
    of those tokens (row i belongs to tokens[i]).  ``to_f32`` widens stored
    weights (e.g. bf16 bit patterns) expert by expert so a large weight set
    never has to be widened at once.
    """
    conv = to_f32 if to_f32 is not None else (lambda a: a)
    tokens = [int(t) for t in tokens]
    ids = np.asarray(ids).reshape(len(tokens), -1)
    weights = _f64(weights).reshape(len(tokens), -1)
    H = np.asarray(x).shape[1]
    out = np.zeros((len(tokens), H), dtype=np.float64)
    xs = _f64(conv(np.asarray(x)[tokens]))
    for e in np.unique(ids):
        sel = np.nonzero(ids == e)
        rows, slots = sel[0], sel[1]
        y = expert_mlp(xs[rows], conv(w13[e]), conv(w2[e]))
        out[rows] += weights[rows, slots][:, None] * y
    return out
