"""Pins of the CPU oracle against things other than itself.

Each pin is a plain function ``pin_*()`` so that ``test_planted_mistakes``
can plant plausible mistakes into the oracle (on the CPU) and show that at
least one pin catches every one of them.

Page legend:
  [Qwen3-MoE page] "稀疏混合专家系统的并行化改造：Qwen3MoeSparseMoeBlock性能优化实战"
  [Hunyuan page]   "混合专家架构大模型Hunyuan-Large：原理剖析与实现机制"
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _rand_case(T=7, H=6, E=5, k=2, I=3, seed=0, bias=True, ties=False):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, H))
    wr = r.standard_normal((E, H)) / math.sqrt(H)
    if ties:   # dyadic grid -> many exactly tied logits
        x = np.round(x * 2) / 2
        wr = np.round(wr * 2) / 2
    b = r.standard_normal(E) * 0.5 if bias else None
    w13 = r.standard_normal((E, 2 * I, H)) / math.sqrt(H)
    w2 = r.standard_normal((E, H, I)) / math.sqrt(I)
    return x, wr, b, w13, w2


def _torch_swiglu(x, w13_e, w2_e):
    """Textbook SwiGLU MLP through torch's own float64 ops (a library routine)."""
    xt = torch.as_tensor(np.asarray(x, np.float64))
    w = torch.as_tensor(np.asarray(w13_e, np.float64))
    I = w.shape[0] // 2
    g = torch.nn.functional.linear(xt, w[:I])
    u = torch.nn.functional.linear(xt, w[I:])
    h = torch.nn.functional.silu(g) * u
    return torch.nn.functional.linear(h, torch.as_tensor(np.asarray(w2_e, np.float64))).numpy()


# --------------------------------------------------------------------------
# Worked example (hand-derived, tests/golden/worked_example.json)
# --------------------------------------------------------------------------

def pin_worked_example():
    g = json.load(open(GOLDEN))
    x, wr, b = np.array(g["x"], float), np.array(g["w_router"], float), np.array(g["bias"], float)
    w13, w2, k = np.array(g["w13"], float), np.array(g["w2"], float), g["k"]
    res = O.forward(x, wr, b, w13, w2, k, renormalize=False)
    assert np.array_equal(res["logits"], np.array(g["expected_logits"], float))
    assert np.array_equal(res["ids"], np.array(g["expected_ids"]))
    assert np.array_equal(res["counts"], np.array(g["expected_counts"]))
    assert np.array_equal(res["offsets"], np.array(g["expected_offsets"]))
    assert np.array_equal(res["perm"], np.array(g["expected_perm"]))
    assert np.array_equal(res["inv_perm"], np.array(g["expected_inv_perm"]))
    e = math.e
    silu = lambda z: z / (1 + math.exp(-z))  # noqa: E731  (scalar textbook SiLU)
    # hand-derived outputs (gate value g, up value u of each chosen expert):
    # t0 -> experts 0 (g=1,u=0) and 2 (g=-1,u=2); both have p = e/(3e+1)
    p0 = e / (3 * e + 1)
    out0 = p0 * 0.0 + p0 * (silu(-1.0) * 2.0) * np.array([0.5, 0.5])
    # t1 -> experts 1 (g=.5,u=1) and 3 (g=.75,u=-1); Z = 1 + 2e + 1/e, both p = e/Z
    Z1 = 1 + 2 * e + 1 / e
    out1 = (e / Z1) * silu(0.5) * np.array([-1.0, 1.0]) + (e / Z1) * (-silu(0.75)) * np.array([3.0, -2.0])
    # t2 -> experts 3 (g=1,u=0) and 0 (g=1,u=1); Z = 2e + 1 + e^1.5
    Z2 = 2 * e + 1 + math.exp(1.5)
    out2 = (math.exp(1.5) / Z2) * 0.0 + (e / Z2) * silu(1.0) * np.array([1.0, 2.0])
    want = np.stack([out0, out1, out2])
    assert np.allclose(res["out"], want, rtol=1e-14, atol=1e-15)
    want_w = np.array([[p0, p0], [e / Z1, e / Z1], [math.exp(1.5) / Z2, e / Z2]])
    assert np.allclose(res["weights"], want_w, rtol=1e-14)


# --------------------------------------------------------------------------
# Router, softmax, top-k
# --------------------------------------------------------------------------

def pin_logits_exact_dyadic():
    # integers / halves: the exact dot product is known, any summation order gives it
    x = np.array([[1.0, -2.0, 0.5], [3.0, 0.0, -1.0]])
    wr = np.array([[2.0, 1.0, 4.0], [-1.0, 0.5, 0.0]])
    b = np.array([0.25, -1.0])
    want = np.array([[2 - 2 + 2 + 0.25, -1 - 1 + 0 - 1.0], [6 + 0 - 4 + 0.25, -3 + 0 + 0 - 1.0]])
    assert np.array_equal(O.router_logits(x, wr, b), want)


def pin_softmax_closed_forms():
    r = np.random.default_rng(1)
    l = r.standard_normal((9, 6)) * 3
    p = O.softmax_all(l)
    assert np.all(p > 0)
    assert np.allclose(p.sum(1), 1.0, atol=1e-15)
    # ratio of probabilities is exp of the logit difference (a dropped or
    # negated term breaks it)
    assert np.allclose(p[:, 1] / p[:, 4], np.exp(l[:, 1] - l[:, 4]), rtol=1e-13)
    # two experts: softmax reduces to the logistic function of the gap
    l2 = r.standard_normal((5, 2))
    p2 = O.softmax_all(l2)
    assert np.allclose(p2[:, 0], 1 / (1 + np.exp(l2[:, 1] - l2[:, 0])), rtol=1e-14)
    # equal logits -> uniform; huge logits do not overflow
    assert np.allclose(O.softmax_all(np.zeros((2, 8))), 1 / 8)
    big = O.softmax_all(np.array([[1000.0, 999.0]]))
    assert np.allclose(big[0, 0], 1 / (1 + math.exp(-1)), rtol=1e-14)


def _brute_topk(l, k):
    """Exhaustive search over ordered k-tuples for the lexicographically best
    (value desc, id asc) sequence; independent of any sort routine."""
    E = len(l)
    best, best_key = None, None
    for tup in itertools.permutations(range(E), k):
        key = tuple((l[e], -e) for e in tup)
        if best_key is None or key > best_key:
            best, best_key = tup, key
    return list(best)


def pin_topk_bruteforce():
    for seed, ties in [(2, False), (3, True), (4, True)]:
        x, wr, b, _, _ = _rand_case(T=12, H=4, E=6, seed=seed, ties=ties, bias=False)
        l = O.router_logits(x, wr, None)
        for k in (1, 2, 3, 6):
            ids = O.topk_ids(l, k)
            for t in range(l.shape[0]):
                assert list(ids[t]) == _brute_topk(l[t], k), (seed, k, t)


def pin_topk_special_cases():
    # zero router: every logit ties, ids are 0..k-1 and weights are 1/E
    x = np.random.default_rng(5).standard_normal((4, 8))
    ids, w, _, _ = O.route(x, np.zeros((6, 8)), None, 3, False)
    assert np.array_equal(ids, np.tile(np.arange(3), (4, 1)))
    assert np.allclose(w, 1 / 6)
    # duplicated router rows: the lower index of a tied pair comes first
    wr = np.random.default_rng(6).standard_normal((5, 8))
    wr[4] = wr[1]
    l = O.router_logits(x, wr, None)
    ids = O.topk_ids(l, 5)
    for t in range(4):
        pos = list(ids[t])
        assert pos.index(1) + 1 == pos.index(4)
    # bias acts inside the softmax: a huge bias on one expert always selects it
    # with weight ~1 (Hunyuan gating formula)
    b = np.zeros(5)
    b[3] = 100.0
    ids, w, _, _ = O.route(x, wr, b, 1, False)
    assert np.all(ids[:, 0] == 3) and np.allclose(w[:, 0], 1.0)


def pin_route_invariants():
    for seed in range(3):
        x, wr, b, _, _ = _rand_case(T=20, H=8, E=7, seed=seed)
        for k, ren in [(1, False), (3, False), (3, True), (7, True)]:
            ids, w, l, p = O.route(x, wr, b, k, ren)
            assert ids.dtype == np.int32 and ids.shape == (20, k)
            for t in range(20):
                assert len(set(ids[t])) == k
                sel = l[t, ids[t]]
                rest = np.delete(l[t], ids[t])
                assert rest.size == 0 or sel.min() >= rest.max()
                assert np.all(np.diff(sel) <= 0)
            if ren:
                assert np.allclose(w.sum(1), 1.0)
                assert np.allclose(w, p[np.arange(20)[:, None], ids] /
                                   p[np.arange(20)[:, None], ids].sum(1, keepdims=True))
            else:
                assert np.array_equal(w, np.take_along_axis(p, ids.astype(np.int64), 1))


# --------------------------------------------------------------------------
# Permutation
# --------------------------------------------------------------------------

def _brute_permute(ids, E):
    flat = [int(v) for v in np.asarray(ids).ravel()]
    M = len(flat)
    counts = [sum(1 for v in flat if v == e) for e in range(E)]
    offsets = [sum(counts[:e]) for e in range(E + 1)]
    perm = [None] * M
    for f in range(M):
        rank = sum(1 for g in range(M) if (flat[g], g) < (flat[f], f))
        perm[rank] = f
    inv = [perm.index(f) for f in range(M)]
    return counts, offsets, perm, inv


def pin_permute_bruteforce():
    r = np.random.default_rng(7)
    for T, k, E in [(1, 1, 1), (5, 2, 3), (9, 3, 8), (16, 4, 4), (0, 2, 3)]:
        ids = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]) if T else \
            np.zeros((0, k), np.int32)
        c, o, p, i = O.permute(ids, E)
        bc, bo, bp, bi = _brute_permute(ids, E)
        assert list(c) == bc and list(o) == bo and list(p) == bp and list(i) == bi


def pin_permute_invariants():
    r = np.random.default_rng(8)
    T, k, E = 50, 3, 6
    ids = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)])
    c, o, p, i = O.permute(ids, E)
    assert c.sum() == T * k and o[-1] == T * k and np.all(np.diff(o) == c)
    assert np.array_equal(np.sort(p), np.arange(T * k))
    assert np.array_equal(i[p], np.arange(T * k)) and np.array_equal(p[i], np.arange(T * k))
    e_of_row = ids.ravel()[p]
    assert np.all(np.diff(e_of_row) >= 0)
    for e in range(E):
        seg = p[o[e]:o[e + 1]]
        assert np.all(np.diff(seg) > 0)
    # each token appears exactly k times
    assert np.array_equal(np.bincount(p // k, minlength=T), np.full(T, k))
    xg = O.gather_rows(np.arange(T)[:, None] * np.ones((1, 2)), p, k)
    assert np.array_equal(xg[:, 0], p // k)


# --------------------------------------------------------------------------
# Experts, combine, whole block
# --------------------------------------------------------------------------

def pin_silu_closed_forms():
    z = np.linspace(-6, 6, 25)
    s = O.silu(z)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(s - O.silu(-z), z, atol=1e-14)            # silu(z) - silu(-z) = z
    assert np.isclose(O.silu(np.array([math.log(3)]))[0], 0.75 * math.log(3), rtol=1e-15)
    assert O.silu(np.array([60.0]))[0] == 60.0
    assert abs(O.silu(np.array([-800.0]))[0]) < 1e-300


def pin_expert_mlp_textbook():
    r = np.random.default_rng(9)
    H, I = 5, 3
    xe = r.standard_normal((4, H))
    w13 = r.standard_normal((2 * I, H))
    w2 = r.standard_normal((H, I))
    assert np.allclose(O.expert_mlp(xe, w13, w2), _torch_swiglu(xe, w13, w2), rtol=1e-13, atol=1e-14)
    # H != I on purpose: a transposed weight would not even broadcast


def _brute_dense(x, ids, weights, w13, w2):
    """Every expert runs on every token; the one-hot top-k mask keeps the
    chosen ones ([Qwen3-MoE page] §1 forward listing builds that mask)."""
    T = x.shape[0]
    E = w13.shape[0]
    mask = np.zeros((T, E))
    wt = np.zeros((T, E))
    for t in range(T):
        for j, e in enumerate(ids[t]):
            mask[t, e] = 1.0
            wt[t, e] = weights[t, j]
    out = np.zeros_like(np.asarray(x, np.float64))
    for e in range(E):
        ye = _torch_swiglu(x, w13[e], w2[e])
        out += (mask[:, e] * wt[:, e])[:, None] * ye
    return out


def pin_block_vs_brute_dense():
    for seed, (T, H, E, k, I, ren) in enumerate([(6, 4, 3, 1, 2, False), (11, 6, 5, 2, 3, False),
                                                 (13, 5, 8, 3, 4, True), (9, 4, 4, 4, 6, False)]):
        x, wr, b, w13, w2 = _rand_case(T, H, E, k, I, seed=10 + seed)
        res = O.forward(x, wr, b, w13, w2, k, ren)
        want = _brute_dense(x, res["ids"], res["weights"], w13, w2)
        assert np.allclose(res["out"], want, rtol=1e-12, atol=1e-13)
        # token-at-a-time form used for sampled checks agrees too
        toks = [0, T - 1, T // 2]
        sub = O.forward_tokens(x, res["ids"][toks], res["weights"][toks], w13, w2, toks)
        assert np.allclose(sub, want[toks], rtol=1e-12, atol=1e-13)


def pin_special_case_dense_mlp():
    # E = 1, k = 1: probability 1, the block is the textbook SwiGLU MLP
    x, wr, b, w13, w2 = _rand_case(T=8, H=5, E=1, k=1, I=3, seed=20)
    out = O.forward(x, wr, b, w13, w2, 1, False)["out"]
    assert np.allclose(out, _torch_swiglu(x, w13[0], w2[0]), rtol=1e-13, atol=1e-14)


def pin_special_case_identical_experts():
    # identical experts + renormalised weights: output is MLP(x) whatever the routing
    x, wr, b, w13, w2 = _rand_case(T=10, H=6, E=5, k=3, I=4, seed=21)
    w13 = np.repeat(w13[:1], 5, axis=0)
    w2 = np.repeat(w2[:1], 5, axis=0)
    out = O.forward(x, wr, b, w13, w2, 3, True)["out"]
    assert np.allclose(out, _torch_swiglu(x, w13[0], w2[0]), rtol=1e-12, atol=1e-13)


def pin_special_case_soft_moe():
    # k = E without renormalisation: the dense soft mixture sum_e p_e MLP_e(x)
    x, wr, b, w13, w2 = _rand_case(T=7, H=4, E=4, k=4, I=3, seed=22)
    out = O.forward(x, wr, b, w13, w2, 4, False)["out"]
    lt = torch.nn.functional.linear(torch.as_tensor(x), torch.as_tensor(wr), torch.as_tensor(b))
    p = torch.softmax(lt, dim=1).numpy()
    want = sum(p[:, e:e + 1] * _torch_swiglu(x, w13[e], w2[e]) for e in range(4))
    assert np.allclose(out, want, rtol=1e-12, atol=1e-13)


def pin_metamorphic():
    x, wr, b, w13, w2 = _rand_case(T=12, H=5, E=6, k=2, I=3, seed=23)
    base = O.forward(x, wr, b, w13, w2, 2, False)
    # relabel experts consistently -> same output, ids relabelled
    s = np.array([3, 0, 5, 1, 4, 2])          # new expert n is old expert s[n]
    rel = O.forward(x, wr[s], b[s], w13[s], w2[s], 2, False)
    assert np.allclose(rel["out"], base["out"], rtol=1e-13, atol=1e-14)
    assert np.array_equal(s[rel["ids"]], base["ids"])
    # permute tokens -> permuted output
    q = np.random.default_rng(24).permutation(12)
    pt = O.forward(x[q], wr, b, w13, w2, 2, False)
    assert np.allclose(pt["out"], base["out"][q], rtol=1e-13, atol=1e-14)
    # the output is linear in the down weights
    sc = O.forward(x, wr, b, w13, 3.0 * w2, 2, False)
    assert np.allclose(sc["out"], 3.0 * base["out"], rtol=1e-13, atol=1e-14)


def pin_combine_direct():
    # combine alone on a hand-built Y: out[t] = sum_j w[t,j] Y[inv[t*k+j]]
    T, k, H = 3, 2, 2
    inv = np.array([5, 0, 1, 4, 2, 3])
    Y = np.arange(12, dtype=float).reshape(6, 2)
    w = np.array([[1.0, 2.0], [0.5, 0.25], [3.0, -1.0]])
    out = O.combine(Y, inv, w, T, k)
    want = np.array([[1 * 10 + 2 * 0, 1 * 11 + 2 * 1],
                     [0.5 * 2 + 0.25 * 8, 0.5 * 3 + 0.25 * 9],
                     [3 * 4 - 6, 3 * 5 - 7]], dtype=float)
    assert np.array_equal(out, want)


def pin_shared_expert():
    from scipy.special import expit
    x, wr, b, w13, w2 = _rand_case(T=9, H=5, E=4, k=2, I=3, seed=31)
    for renorm in (False, True):
        base = O.forward(x, wr, b, w13, w2, 2, renorm)
        # a zero shared down projection leaves the routed output untouched
        zero = O.forward_shared(x, wr, b, w13, w2, np.ones((8, 5)), np.zeros((5, 4)), 2, renorm)
        assert np.array_equal(zero["out"], base["out"])
        # gate = 2 x, up = x, down = identity: S(x) = silu(2x) * x = 2 x^2 sigmoid(2x),
        # added with weight 1 whatever the routing weights are
        ws13 = np.vstack([2.0 * np.eye(5), np.eye(5)])
        sh = O.forward_shared(x, wr, b, w13, w2, ws13, np.eye(5), 2, renorm)
        assert np.allclose(sh["out"] - base["out"], 2.0 * x ** 2 * expit(2.0 * x), rtol=1e-12, atol=1e-14)
        # the shared contribution is linear in its down weights
        r = np.random.default_rng(32)
        a13, a2 = r.standard_normal((6, 5)), r.standard_normal((5, 3))
        one = O.forward_shared(x, wr, b, w13, w2, a13, a2, 2, renorm)["out"] - base["out"]
        three = O.forward_shared(x, wr, b, w13, w2, a13, 3.0 * a2, 2, renorm)["out"] - base["out"]
        assert np.allclose(three, 3.0 * one, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# Token rounding ([SonicMoE page] 核心差异 §3; the integer rule in the
# oracle's token_round docstring)
# --------------------------------------------------------------------------

def _route_case(T, E, k, seed, H=8):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, H))
    w = r.standard_normal((E, H)) / 3
    ids, wts, l, p = O.route(x, w, None, k, False)
    return ids, p


def _rank_in_expert(ids):
    """rank[t, j]: how many earlier assignments (flat order) share the expert."""
    seen = {}
    rank = np.zeros(ids.shape, dtype=np.int64)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            rank[t, j] = seen.get(e, 0)
            seen[e] = rank[t, j] + 1
    return rank


def pin_token_round_hand_example():
    """Worked by hand: T=6, E=3, k=2, B=3.  Counts are 4,4,4, so each expert
    keeps 3 and pools its last assignment in flat order: (t4,j0)->0,
    (t5,j0)->2, (t5,j1)->1.  Tile 1 (all loads 3, lowest id) goes to expert 0
    and takes (t4,j0) (back to 0) and (t5,j0) (2 -> 0); (t5,j1) is the same
    token's second slot, so the pool runs out for this tile at 2 rows.  Tile
    2 goes to expert 1 (load 3 < 5) and takes (t5,j1), whose expert stays 1."""
    ids = np.array([[0, 1], [0, 2], [0, 1], [1, 2], [0, 2], [2, 1]])
    p = np.full((6, 3), 1.0 / 3.0)
    p[5] = [0.5, 0.2, 0.3]
    new, w, moved = O.token_round(ids, p, 3, 3, False)
    want = ids.copy()
    want[5, 0] = 0
    assert np.array_equal(new, want)
    assert moved.sum() == 1 and moved[5, 0]
    assert np.allclose(w[5], [0.5, 0.2]) and np.allclose(w[:5], 1.0 / 3.0)
    _, wr, _ = O.token_round(ids, p, 3, 3, True)
    assert np.allclose(wr[5], [0.5 / 0.7, 0.2 / 0.7])


GOLDEN_ROUND = os.path.join(os.path.dirname(__file__), "golden", "token_round_short_tile.json")


def pin_token_round_short_tile_golden():
    """Hand-derived case (tests/golden/token_round_short_tile.json): one round
    plans three tiles and the second comes out short (2 of 3 rows)."""
    with open(GOLDEN_ROUND) as f:
        g = json.load(f)
    ids = np.array(g["ids"])
    p = np.array(g["probs"], dtype=np.float64)
    new, w, moved = O.token_round(ids, p, g["E"], g["B"], False)
    assert np.array_equal(new, np.array(g["expected_ids"]))
    assert np.array_equal(moved, np.array(g["expected_moved"]))
    assert np.array_equal(np.bincount(new.ravel(), minlength=g["E"]), g["expected_counts"])
    assert np.allclose(w, g["expected_weights"], rtol=0, atol=1e-15)
    _, wr, _ = O.token_round(ids, p, g["E"], g["B"], True)
    assert np.allclose(wr, g["expected_weights_renormalised"], rtol=1e-15, atol=0)


def _greedy_token_round(ids, E, B):
    """The plainest reading of the hand-out, written independently of the
    oracle: every tile goes to the expert with the lowest load reached so far
    (ties to the lowest id) among those whose last tile was not empty; it
    takes up to B pooled assignments in flat order, at most one per token,
    none whose token holds the owner in another slot."""
    T, k = ids.shape
    counts = np.bincount(ids.ravel(), minlength=E)
    keep = counts // B * B
    rank = _rank_in_expert(ids)
    pool = [(t, j) for t in range(T) for j in range(k) if rank[t, j] >= keep[ids[t, j]]]
    load = [int(c) for c in keep]
    able = [True] * E
    cur = ids.copy()
    done = [False] * len(pool)
    while not all(done):
        cand = [e for e in range(E) if able[e]]
        e = min(cand, key=lambda q: (load[q], q))
        got, toks = 0, set()
        for i, (t, j) in enumerate(pool):
            if got == B:
                break
            if done[i] or t in toks or any(cur[t, jj] == e for jj in range(k) if jj != j):
                continue
            cur[t, j] = e
            done[i] = True
            toks.add(t)
            got += 1
        load[e] += got
        if got == 0:
            able[e] = False
    return cur


def pin_token_round_equals_greedy():
    """Random cases, about a quarter of them with a tile that comes out short
    before the last tile of its round (small E, k close to E, B near the pool
    size): the oracle's
    ids equal those of choosing each tile's owner from the loads reached so
    far (``_greedy_token_round``)."""
    r = np.random.default_rng(77)
    n_cases = 0
    for _ in range(600):
        E = int(r.integers(3, 7))
        k = int(r.integers(2, E))
        B = int(r.integers(2, 6))
        T = int(r.integers(3, 14))
        ids = np.array([r.choice(E, k, replace=False) for _ in range(T)])
        p = np.full((T, E), 1.0 / E)
        try:
            new, _, _ = O.token_round(ids, p, E, B, False)
        except RuntimeError:
            continue
        assert np.array_equal(new, _greedy_token_round(ids, E, B)), (E, k, B, ids.tolist())
        n_cases += 1
    assert n_cases > 400


def pin_token_round_k1_closed_form():
    """k = 1 has no eligibility limit: the pool (flat order) is cut into
    consecutive blocks of B, and block i goes to the i-th choice of the
    water-filling (least kept-plus-received rows, lowest id), so the padded
    tile count becomes exactly ceil(T / B)."""
    for T, E, B, seed in [(97, 5, 8, 1), (300, 7, 16, 2), (64, 3, 64, 3), (50, 6, 7, 4)]:
        ids, p = _route_case(T, E, 1, seed)
        flat = ids[:, 0]
        counts = np.array([(flat == e).sum() for e in range(E)])
        keep = counts // B * B
        rank = _rank_in_expert(ids)[:, 0]
        pool = [t for t in range(T) if rank[t] >= keep[flat[t]]]
        load = list(keep)
        owners = []
        left = len(pool)
        while left > 0:
            e = min(range(E), key=lambda q: (load[q], q))
            n = min(B, left)
            owners.append(e)
            load[e] += n
            left -= n
        want = flat.copy()
        for i, t in enumerate(pool):
            want[t] = owners[i // B]
        new, w, moved = O.token_round(ids, p, E, B, False)
        assert np.array_equal(new[:, 0], want), (T, E, B)
        c2 = np.bincount(new[:, 0], minlength=E)
        assert np.ceil(c2 / B).sum() == -(-T // B)
        assert np.allclose(w[:, 0], p[np.arange(T), new[:, 0]])


def pin_token_round_wide_tile():
    """B > T: every count is below B, so everything is pooled and all loads
    start at 0.  Expert 0 then takes one slot of every token, expert 1 the
    next, ...: each token ends with exactly the experts {0, ..., k-1}."""
    for T, E, k, seed in [(9, 5, 2, 5), (20, 8, 3, 6), (6, 4, 4, 7)]:
        ids, p = _route_case(T, E, k, seed)
        new, w, moved = O.token_round(ids, p, E, T + 1, True)
        for t in range(T):
            assert sorted(new[t]) == list(range(k))
        assert np.allclose(w.sum(axis=1), 1.0)


def pin_token_round_invariants():
    """Random cases: no token holds an expert twice; the kept rows (the first
    floor(c_e/B)*B of each expert in flat order) never move; only pooled rows
    move; weights are the probabilities of the final experts; nothing moves
    when B = 1, when every count is already a multiple of B, or when k = E."""
    for T, E, k, B, seed, renorm in [(200, 8, 2, 16, 8, False), (150, 16, 4, 8, 9, True),
                                      (300, 32, 8, 12, 10, True), (80, 6, 3, 5, 11, False)]:
        ids, p = _route_case(T, E, k, seed)
        new, w, moved = O.token_round(ids, p, E, B, renorm)
        counts = np.bincount(ids.ravel(), minlength=E)
        keep = counts // B * B
        rank = _rank_in_expert(ids)
        kept = rank < keep[ids]
        assert np.array_equal(new[kept], ids[kept])
        assert np.array_equal(moved, new != ids) and not moved[kept].any()
        assert moved.any()
        for t in range(T):
            assert len(set(new[t].tolist())) == k
        want = p[np.arange(T)[:, None], new]
        if renorm:
            want = want / want.sum(axis=1, keepdims=True)
        assert np.allclose(w, want, rtol=1e-14, atol=0)
        assert np.bincount(new.ravel(), minlength=E).sum() == T * k
    ids, p = _route_case(60, 8, 2, 12)
    for B in (1,):
        new, w, moved = O.token_round(ids, p, 8, B, False)
        assert not moved.any() and np.array_equal(new, ids)
    # every count a multiple of 4: tokens cycle through pairs (e, e+1 mod 8)
    ids = np.array([[t % 8, (t + 1) % 8] for t in range(32)])
    new, w, moved = O.token_round(ids, np.full((32, 8), 0.125), 8, 4, False)
    assert not moved.any()
    ids, p = _route_case(40, 4, 4, 13)
    new, w, moved = O.token_round(ids, p, 4, 3, False)
    assert not moved.any()


def pin_forward_rounded_composition():
    """The rounded block is the plain block run on the rounded routing."""
    x, w, b, w13, w2 = _rand_case(T=30, H=6, E=5, k=2, I=3, seed=31)
    r = O.forward_rounded(x, w, b, w13, w2, 2, True, 4)
    c = np.bincount(r["ids"].ravel(), minlength=5)
    assert np.array_equal(c, r["counts"])
    ref = _brute_dense(x, r["ids"], r["weights"], w13, w2)
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# MXFP8 (OCP FP8 E4M3 elements, OCP MX v1.0 E8M0 block scales of 32)
# --------------------------------------------------------------------------

def pin_e4m3_table():
    """Code values fixed by the OCP FP8 E4M3 definition (bias 7, 3 mantissa
    bits, no infinities, only S.1111.111 is NaN)."""
    V = O.E4M3
    assert V[0x38] == 1.0 and V[0x40] == 2.0 and V[0x30] == 0.5
    assert V[0x7E] == 448.0 and V[0xFE] == -448.0         # largest normal
    assert V[0x08] == 2.0 ** -6                            # smallest normal
    assert V[0x01] == 2.0 ** -9 and V[0x07] == 7 * 2.0 ** -9   # subnormals
    assert np.isnan(V[0x7F]) and np.isnan(V[0xFF])
    assert np.isnan(V).sum() == 2
    assert V[0x80] == 0 and np.signbit(V[0x80])
    finite = V[:0x7F]
    assert np.all(np.diff(finite) > 0)                     # codes 0..126 increase
    assert V[0x39] - V[0x38] == 0.125                      # spacing 2^-3 in [1, 2)


def pin_e4m3_encode():
    V = O.E4M3
    codes = np.arange(0x7F)
    assert np.array_equal(O.e4m3_encode(V[codes]), codes)          # exact values map to themselves
    neg = np.arange(0x81, 0xFF)
    assert np.array_equal(O.e4m3_encode(V[neg]), neg)
    # ties go to the even code: 1.0625 sits between 1.0 (0x38) and 1.125 (0x39)
    assert O.e4m3_encode([1.0625])[0] == 0x38
    assert O.e4m3_encode([1.1875])[0] == 0x3A                      # between 0x39 and 0x3A
    assert O.e4m3_encode([-1.0625])[0] == 0xB8
    assert O.e4m3_encode([2.0 ** -10])[0] == 0x00                  # half the smallest subnormal
    assert O.e4m3_encode([3 * 2.0 ** -11])[0] == 0x01              # 0.75 of it rounds up
    assert O.e4m3_encode([1.06])[0] == 0x38 and O.e4m3_encode([1.07])[0] == 0x39
    # saturation at +-448 (no infinities)
    assert O.e4m3_encode([449.0, 1e9])[0] == 0x7E and O.e4m3_encode([-1e9])[0] == 0xFE
    assert O.e4m3_encode([464.0])[0] == 0x7E                       # past the 448/480 midpoint
    r = np.random.default_rng(40).uniform(-500, 500, 2000)
    d = V[O.e4m3_encode(r)]
    order = np.argsort(r)
    assert np.all(np.diff(d[order]) >= 0)                          # monotone
    inr = np.abs(r) <= 448
    assert np.all(np.abs(d - r)[inr] <= np.maximum(np.abs(r), 2.0 ** -6)[inr] * 2.0 ** -4 + 1e-300)


def pin_mx_quantize():
    """Block scale 2^(floor(log2 amax) - 8): a block whose largest magnitude
    is 2^e stores it as 256 = code 0x78; powers of two scale only the
    exponents; a zero block stays zero; elements within 2^-4 relative."""
    v = np.zeros((3, 64))
    v[0, :32] = np.linspace(-1, 1, 32) * 0.75
    v[0, 5] = 2.0 ** 3                                 # amax of block 0 = 8
    v[0, 32:] = np.linspace(0.1, 3.0, 32)              # block 1: amax 3
    v[1, :] = 1e-3 * np.arange(64)
    codes, sc, deq = O.mx_quantize(v)
    assert sc[0, 0] == 127 + 3 - 8 and codes[0, 5] == 0x78
    assert sc[0, 1] == 127 + 1 - 8                     # floor(log2 3) = 1
    assert np.all(codes[2] == 0) and np.all(deq[2] == 0) and np.all(sc[2] == 0)
    c2, s2, d2 = O.mx_quantize(v * 2.0 ** 5)
    assert np.array_equal(c2, codes) and np.array_equal(s2[:2], sc[:2] + 5)
    assert np.array_equal(d2, deq * 2.0 ** 5)
    r = np.random.default_rng(41).standard_normal((16, 256))
    c, s_, d = O.mx_quantize(r)
    blocks = np.abs(r).reshape(16, 8, 32)
    scale = np.ldexp(1.0, s_.astype(int) - 127)[..., None]
    # elements not saturated and above the subnormal range: within 2^-4 relative
    ok = (blocks / scale <= 448) & (blocks / scale >= 2.0 ** -6)
    err = np.abs(d - r).reshape(16, 8, 32)
    assert np.all(err[ok] <= blocks[ok] * 2.0 ** -4)
    assert np.array_equal(O.mx_dequantize(c, s_), d)


def _mx_case(T=40, H=64, E=4, k=2, I=32, seed=50):
    x, w, b, w13, w2 = _rand_case(T=T, H=H, E=E, k=k, I=I, seed=seed)
    q13, s13, _ = O.mx_quantize(w13)
    q2, s2, _ = O.mx_quantize(w2)
    return x, w, b, w13, w2, q13, s13, q2, s2


def pin_forward_mxfp8():
    """Per-token brute force (each token through its experts alone: blocks
    run along each row, so batching must not matter); exact power-of-two
    scaling through W2 and through the up half of W13; and the quantization
    error against the unquantized block stays at the fp8 level."""
    x, w, b, w13, w2, q13, s13, q2, s2 = _mx_case()
    k = 2
    r = O.forward_mxfp8(x, w, b, q13, s13, q2, s2, k, True)
    brute = np.zeros_like(r["out"])
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(r["ids"][t, j])
            brute[t] += r["weights"][t, j] * O.expert_mlp_mxfp8(x[t:t + 1], q13[e], s13[e], q2[e], s2[e])[0]
    assert np.allclose(r["out"], brute, rtol=1e-12, atol=1e-12)
    # W2 * 2^3: identical codes, scales + 3, output exactly * 8
    r8 = O.forward_mxfp8(x, w, b, q13, s13, q2, s2 + 3, k, True)
    assert np.array_equal(r8["out"], r["out"] * 8)
    # up half of W13 * 2^-2: h (and its MX scales) exactly / 4
    I = q13.shape[1] // 2
    s13u = s13.copy()
    s13u[:, I:] -= 2
    ru = O.forward_mxfp8(x, w, b, q13, s13u, q2, s2, k, True)
    assert np.array_equal(ru["out"], r["out"] / 4)
    ref = O.forward(x, w, b, w13, w2, k, True)["out"]
    rel = np.linalg.norm(r["out"] - ref) / np.linalg.norm(ref)   # 4 operands at 3 mantissa bits
    assert 1e-3 < rel < 0.15, rel


# --------------------------------------------------------------------------
# Backward: directional derivatives of the (pinned) forward by central
# differences, exact special cases, linearity in dout
# --------------------------------------------------------------------------

def _loss(x, wr, b, w13, w2, k, renorm, dout):
    r = O.forward(x, wr, b, w13, w2, k, renorm)
    return float((dout * r["out"]).sum()), r["ids"]


_BWD_CASES = [
    # T, H, E, k, I, bias, renormalize
    (6, 5, 4, 2, 3, True, False),
    (6, 5, 4, 2, 3, True, True),
    (5, 4, 3, 3, 2, False, False),   # k = E: every expert, soft mixture
    (4, 6, 5, 1, 4, True, True),     # k = 1 renormalised: weight 1, no router gradient
]


def pin_backward_finite_differences():
    for ci, (T, H, E, k, I, bias, renorm) in enumerate(_BWD_CASES):
        x, wr, b, w13, w2 = _rand_case(T=T, H=H, E=E, k=k, I=I, seed=40 + ci, bias=bias)
        r = np.random.default_rng(90 + ci)
        dout = r.standard_normal((T, H))
        g = O.backward(x, wr, b, w13, w2, k, renorm, dout)
        params = {"x": x, "w_router": wr, "w13": w13, "w2": w2}
        if bias:
            params["bias"] = b
        grads = {"x": g["dx"], "w_router": g["dw_router"], "bias": g["dbias"], "w13": g["dw13"],
                 "w2": g["dw2"]}
        ids0 = g["fw"]["ids"]
        for name, val in params.items():
            for trial in range(2):
                V = r.standard_normal(val.shape)
                eps = 1e-5
                args = {"x": x, "w_router": wr, "bias": b, "w13": w13, "w2": w2}
                args[name] = val + eps * V
                fp, idp = _loss(args["x"], args["w_router"], args["bias"], args["w13"], args["w2"],
                                k, renorm, dout)
                args[name] = val - eps * V
                fm, idm = _loss(args["x"], args["w_router"], args["bias"], args["w13"], args["w2"],
                                k, renorm, dout)
                assert np.array_equal(idp, ids0) and np.array_equal(idm, ids0), "selection moved"
                fd = (fp - fm) / (2 * eps)
                an = float((grads[name] * V).sum())
                assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0), (ci, name, fd, an)


def pin_backward_special_cases():
    # a single expert: p = 1, so the router receives no gradient at all
    x, wr, b, w13, w2 = _rand_case(T=4, H=5, E=1, k=1, I=3, seed=3)
    dout = np.random.default_rng(1).standard_normal((4, 5))
    g = O.backward(x, wr, b, w13, w2, 1, False, dout)
    assert np.array_equal(g["dw_router"], np.zeros_like(wr)) and np.array_equal(g["dbias"], np.zeros(1))
    # the same block is then a plain SwiGLU MLP: torch's float64 autograd gives its gradients
    xt = torch.tensor(x, requires_grad=True)
    w13t = torch.tensor(w13[0], requires_grad=True)
    w2t = torch.tensor(w2[0], requires_grad=True)
    gt = torch.nn.functional.linear(xt, w13t[:3])
    ut = torch.nn.functional.linear(xt, w13t[3:])
    out = torch.nn.functional.linear(torch.nn.functional.silu(gt) * ut, w2t)
    (out * torch.tensor(dout)).sum().backward()
    assert np.allclose(g["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dw13"][0], w13t.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dw2"][0], w2t.grad.numpy(), rtol=1e-12, atol=1e-12)
    # W2 = 0: every expert output is zero, so the routing weights, the logits
    # and the gate/up weights receive nothing
    x, wr, b, w13, w2 = _rand_case(T=6, H=5, E=4, k=2, I=3, seed=5)
    dout = np.random.default_rng(2).standard_normal((6, 5))
    g = O.backward(x, wr, b, w13, np.zeros_like(w2), 2, True, dout)
    assert np.array_equal(g["dlogits"], np.zeros((6, 4))) and np.array_equal(g["dw13"], np.zeros_like(w13))
    # experts no token chose get exactly zero gradients ([Hunyuan page] §二.2)
    b2 = np.array([5.0, 5.0, -50.0, -50.0])
    g = O.backward(x, wr, b2, w13, w2, 2, False, dout)
    assert set(g["fw"]["ids"].ravel().tolist()) == {0, 1}
    assert not g["dw13"][2:].any() and not g["dw2"][2:].any()
    assert g["dw13"][:2].any() and g["dw2"][:2].any()
    # linear in dout
    g2 = O.backward(x, wr, b, w13, w2, 2, True, 2 * dout)
    g1 = O.backward(x, wr, b, w13, w2, 2, True, dout)
    for n in ("dx", "dw_router", "dbias", "dw13", "dw2"):
        assert np.allclose(g2[n], 2 * g1[n], rtol=1e-12, atol=1e-14), n


def pin_backward_sampled_matches_backward():
    # the one-by-one parts used at full size equal the whole backward (itself
    # pinned above by finite differences and torch autograd), every token and
    # a few columns, with and without renormalisation and bias
    for (T, H, E, k, I, bias, renorm), seed in ((( 9, 6, 4, 2, 5, True, False), 11),
                                                (( 8, 5, 5, 3, 4, False, True), 12),
                                                (( 7, 4, 3, 1, 3, True, True), 13)):
        x, wr, b, w13, w2 = _rand_case(T=T, H=H, E=E, k=k, I=I, seed=seed, bias=bias)
        dout = np.random.default_rng(seed + 100).standard_normal((T, H))
        full = O.backward(x, wr, b, w13, w2, k, renorm, dout)
        cols = [0, I // 2, I - 1]
        toks = list(range(T))[::-1]
        sm = O.backward_sampled(x, wr, b, w13, w2, k, renorm, dout, toks, cols)
        assert np.allclose(sm["dx"], full["dx"][toks], rtol=1e-12, atol=1e-14)
        assert np.allclose(sm["dlogits"], full["dlogits"][toks], rtol=1e-12, atol=1e-14)
        assert np.allclose(sm["dw"], full["dw"][toks], rtol=1e-12, atol=1e-14)
        assert np.allclose(sm["dw2_cols"], full["dw2"][:, :, cols], rtol=1e-12, atol=1e-14)
        assert np.allclose(sm["dw13_rows"][:, 0], full["dw13"][:, cols, :], rtol=1e-12, atol=1e-14)
        assert np.allclose(sm["dw13_rows"][:, 1], full["dw13"][:, [I + c for c in cols], :],
                           rtol=1e-12, atol=1e-14)


PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_") and callable(v)]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the oracle must fail some pin.
# --------------------------------------------------------------------------

def _orig(name):
    return getattr(O, name)


def _mut_topk_ties_high(l, k):
    l = np.asarray(l, float)
    E = l.shape[1]
    order = np.lexsort((-np.broadcast_to(np.arange(E), l.shape), -l), axis=-1)
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def _mut_topk_ascending_slots(l, k):
    return _orig_topk(l, k)[:, ::-1].copy()


_orig_topk = O.topk_ids
_orig_softmax = O.softmax_all
_orig_permute = O.permute
_orig_expert = O.expert_mlp
_orig_logits = O.router_logits
_orig_combine = O.combine


def _mut_no_bias(x, w, b=None):
    return _orig_logits(x, w, None)


def _mut_softmax_no_max_sub_wrong(l):
    z = np.exp(np.asarray(l, float))
    return z / z.sum(axis=0, keepdims=True)      # normalised over the wrong axis


def _mut_permute_unstable(ids, E):
    c, o, p, i = _orig_permute(ids, E)
    p = p.copy()
    for e in range(E):                            # reverse within each expert
        p[o[e]:o[e + 1]] = p[o[e]:o[e + 1]][::-1]
    inv = np.empty_like(p)
    inv[p] = np.arange(p.size, dtype=np.int32)
    return c, o, p, inv


def _mut_offsets_inclusive(ids, E):
    c, o, p, i = _orig_permute(ids, E)
    o = o.copy()
    o[:-1] = o[1:]
    return c, o, p, i


def _mut_swap_gate_up(xe, w13_e, w2_e):
    I = np.asarray(w13_e).shape[0] // 2
    sw = np.concatenate([w13_e[I:], w13_e[:I]], axis=0)
    return _orig_expert(xe, sw, w2_e)


def _mut_no_silu(xe, w13_e, w2_e):
    w13_e = np.asarray(w13_e, float)
    I = w13_e.shape[0] // 2
    return ((xe @ w13_e[:I].T) * (xe @ w13_e[I:].T)) @ np.asarray(w2_e, float).T


def _mut_combine_perm_for_inv(Y, inv, w, T, k):
    p = np.empty_like(np.asarray(inv))
    p[np.asarray(inv)] = np.arange(len(inv))
    return _orig_combine(Y, p, w, T, k)


def _mut_combine_unweighted(Y, inv, w, T, k):
    return _orig_combine(Y, inv, np.ones_like(np.asarray(w, float)), T, k)


_orig_shared = O.shared_expert


def _mut_shared_gate_up_swapped(x, ws13, ws2):
    I = np.asarray(ws13).shape[0] // 2
    return _orig_shared(x, np.concatenate([ws13[I:], ws13[:I]], axis=0), ws2)


def _mut_shared_omitted(x, ws13, ws2):
    return np.zeros((np.asarray(x).shape[0], np.asarray(ws2).shape[0]))


def _mut_silu_sign(z):
    z = np.asarray(z, float)
    return z / (1.0 + np.exp(z))


_orig_round_pool = O._round_pool
_orig_round_order = O._round_order
_orig_round_weights = O._round_weights


def _mut_round_pool_reversed(ids, E, B):
    keep, pool = _orig_round_pool(ids, E, B)
    return keep, pool[::-1]


def _mut_round_pool_ceil(ids, E, B):
    keep, pool = _orig_round_pool(ids, E, B)
    c = np.bincount(np.asarray(ids).ravel(), minlength=E)
    return -(-c // B) * B, []


def _mut_round_most_loaded(load):
    return _orig_round_order(load)[::-1]


def _mut_round_ties_high(load):
    return sorted(range(len(load)), key=lambda q: (load[q], -q))


def _mut_round_any_slot(cur, t, j, e):
    return True


def _mut_round_weights_not_renormalised(probs, ids, renormalize):
    return _orig_round_weights(probs, ids, False)


_orig_e4m3_encode = O.e4m3_encode
_orig_mx_exponent = O._mx_exponent


def _mut_e4m3_ties_up(y):
    y = np.asarray(y, dtype=np.float64)
    c = _orig_e4m3_encode(y).astype(np.int64)
    # nudge exact midpoints away from zero: round half up in magnitude
    v = O.E4M3[c & 0x7F]
    nxt = O.E4M3[np.minimum((c & 0x7F) + 1, 0x7E)]
    mid = np.abs(np.abs(y) - (v + nxt) / 2) < 1e-300
    c = np.where(mid & ((c & 0x7F) < 0x7E), c + 1, c)
    return c.astype(np.uint8)


def _mut_e4m3_no_saturation(y):
    c = _orig_e4m3_encode(y)
    return np.where(np.abs(np.asarray(y, float)) > 448, np.uint8(0x7F), c).astype(np.uint8)


def _mut_mx_emax7(amax):
    return np.clip(_orig_mx_exponent(amax) + 1, -127, 127)


def _mut_mx_no_floor(amax):
    a = np.asarray(amax, float)
    return np.where(a > 0, np.clip(np.round(np.log2(np.where(a > 0, a, 1))) - 8, -127, 127), -127)


_orig_expert_mlp_backward = O.expert_mlp_backward


def _mut_silu_grad_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, float)))


def _mut_weights_grad_no_mean(dw, probs_sel, renormalize):
    dw = np.asarray(dw, float)
    if not renormalize:
        return dw
    return dw / np.asarray(probs_sel, float).sum(axis=1, keepdims=True)


def _mut_softmax_grad_uncentred(p, dp):
    return np.asarray(p, float) * np.asarray(dp, float)


def _mut_expert_bwd_swapped(xe, w13_e, w2_e, dy):
    dxe, dw13, dw2 = _orig_expert_mlp_backward(xe, w13_e, w2_e, dy)
    I = dw13.shape[0] // 2
    return dxe, np.concatenate([dw13[I:], dw13[:I]]), dw2


_orig_backward_sampled = O.backward_sampled


def _mut_sampled_no_router(x, w_router, bias, w13, w2, k, renormalize, dout, tokens, cols, to_f32=None):
    r = _orig_backward_sampled(x, w_router, bias, w13, w2, k, renormalize, dout, tokens, cols, to_f32)
    r["dx"] = r["dx"] - r["dlogits"] @ np.asarray(w_router, dtype=np.float64)
    return r


def _mut_sampled_up_rows_swapped(x, w_router, bias, w13, w2, k, renormalize, dout, tokens, cols,
                                 to_f32=None):
    r = _orig_backward_sampled(x, w_router, bias, w13, w2, k, renormalize, dout, tokens, cols, to_f32)
    r["dw13_rows"] = r["dw13_rows"][:, ::-1]
    return r


MUTATIONS = {
    "sampled backward without the router term": ("backward_sampled", _mut_sampled_no_router),
    "sampled backward gate and up rows swapped": ("backward_sampled", _mut_sampled_up_rows_swapped),
    "topk ties to the highest index": ("topk_ids", _mut_topk_ties_high),
    "topk slots ascending": ("topk_ids", _mut_topk_ascending_slots),
    "router bias dropped": ("router_logits", _mut_no_bias),
    "softmax over tokens": ("softmax_all", _mut_softmax_no_max_sub_wrong),
    "unstable permutation": ("permute", _mut_permute_unstable),
    "inclusive offsets": ("permute", _mut_offsets_inclusive),
    "gate and up swapped": ("expert_mlp", _mut_swap_gate_up),
    "activation dropped": ("expert_mlp", _mut_no_silu),
    "perm used for inv_perm in combine": ("combine", _mut_combine_perm_for_inv),
    "routing weight dropped": ("combine", _mut_combine_unweighted),
    "silu sign flipped": ("silu", _mut_silu_sign),
    "shared expert gate and up swapped": ("shared_expert", _mut_shared_gate_up_swapped),
    "shared expert omitted": ("shared_expert", _mut_shared_omitted),
    "rounding pool in reverse order": ("_round_pool", _mut_round_pool_reversed),
    "rounding keeps rounded-up counts": ("_round_pool", _mut_round_pool_ceil),
    "rounding tile to the most-loaded expert": ("_round_order", _mut_round_most_loaded),
    "rounding ties to the highest id": ("_round_order", _mut_round_ties_high),
    "rounding ignores the token's other slots": ("_round_eligible", _mut_round_any_slot),
    "rounded weights not renormalised": ("_round_weights", _mut_round_weights_not_renormalised),
    "e4m3 ties away from zero": ("e4m3_encode", _mut_e4m3_ties_up),
    "e4m3 overflow to NaN": ("e4m3_encode", _mut_e4m3_no_saturation),
    "MX scale exponent one too large": ("_mx_exponent", _mut_mx_emax7),
    "MX scale exponent rounded": ("_mx_exponent", _mut_mx_no_floor),
    "silu gradient without its z s (1 - s) term": ("silu_grad", _mut_silu_grad_sigmoid),
    "renormalisation gradient without the mean term": ("weights_grad", _mut_weights_grad_no_mean),
    "softmax gradient not centred": ("softmax_grad", _mut_softmax_grad_uncentred),
    "gate and up gradients swapped": ("expert_mlp_backward", _mut_expert_bwd_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # AssertionError or a shape error both count as caught
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{name}' passed every pin"
