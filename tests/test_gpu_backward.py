"""GPU parity of moe_backward against the float64 oracle's backward.

The forward runs first (moe_forward); its workspace carries the routing and
the expert outputs into the backward.  dout is a seeded bf16 draw.

Metrics.  Per-element relative error means nothing where the exact gradient
is a cancellation: dw = <dout, y> with a random dout, the logit gradients
(exactly zero for unselected experts under renormalisation), and the gate
rows of dW13 at the stationary point of silu (g = -1.278..., where silu'
vanishes and a bf16 g moves it by a relative amount of order 1).  So each
gradient tensor is held to the bf16 tolerance as a tensor: its normwise
error |got - want|_F / |want|_F and its largest error relative to its
largest value, both <= TOL_GRAD, taken per expert block for the weight
gradients; dx (the block's input gradient, like the forward's output)
also per token row.  Experts no token chose must get exactly zero.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_mixture_experts_19_amd import binding as B
from sparse_mixture_experts_19_amd import workloads as W
from moe_test_utils import dev_tensor, host_f64, log, sample_tokens, upload

pytestmark = pytest.mark.gpu

# bf16 tolerance of every gradient tensor (normwise, largest error over the
# largest value; per token row for dx)
TOL_GRAD = 2e-2


def _dout(T, H, seed):
    r = np.random.default_rng(seed)
    return W.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))


def _row_err(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    den = np.abs(want).max(axis=1)
    live = den > 0
    num = np.abs(got - want).max(axis=1)
    return float((num[live] / den[live]).max()) if live.any() else 0.0


def _tensor_err(got, want):
    """(normwise error, largest error / largest value) of one tensor."""
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    d = got - want
    n = np.linalg.norm(want)
    return float(np.linalg.norm(d) / n), float(np.abs(d).max() / np.abs(want).max())


def _run(inp, dout_bits, d=None, events=None):
    wl = inp.wl
    d = d or upload(inp)
    out, fws = B.moe_forward(d["x"], d["w_router"], d["bias"], d["w13"], d["w2"], wl.k,
                             wl.renormalize)
    dout = dev_tensor(dout_bits, "bf16")
    res = B.moe_backward(d["x"], d["w_router"], d["bias"], d["w13"], d["w2"], wl.k, wl.renormalize,
                         fws, dout, events=events)
    torch.cuda.synchronize()
    return res, d


def _compare(inp, dout_bits, res, what):
    wl = inp.wl
    dx, dwr, db, dw13, dw2, ws = res
    ref = O.backward(inp.f32("x"), inp.f32("w_router"), inp.bias, inp.f32("w13"), inp.f32("w2"),
                     wl.k, wl.renormalize, W.bf16_bits_to_f32(dout_bits).astype(np.float64))
    mid = B.backward_intermediates(ws, wl.T, wl.H, wl.I, wl.E, wl.k)
    errs = {}
    for n, got, want in (("dw", mid["dw"].cpu().numpy(), ref["dw"]),
                         ("dlogits", mid["dlogits"].cpu().numpy(), ref["dlogits"]),
                         ("dx", host_f64(dx), ref["dx"]),
                         ("dw_router", dwr.cpu().numpy(), ref["dw_router"]),
                         ("dbias", db.cpu().numpy(), ref["dbias"])):
        errs[n] = _tensor_err(got, want)
    errs["dx rows"] = (_row_err(host_f64(dx), ref["dx"]), 0.0)
    # dh = gather(dout) W2_e before the routing weight, the product that reads
    # W2 as stored ([E, H, I] taken as [E, K, N]): row by row against the
    # oracle's permutation (which the GPU's equals bit for bit)
    fw = ref["fw"]
    dp = O.gather_rows(W.bf16_bits_to_f32(dout_bits).astype(np.float64), fw["perm"], wl.k)
    w2 = inp.f32("w2").astype(np.float64)
    dh_ref = np.zeros((wl.T * wl.k, wl.I))
    for e in range(wl.E):
        a, b = int(fw["offsets"][e]), int(fw["offsets"][e + 1])
        dh_ref[a:b] = dp[a:b] @ w2[e]
    errs["dh rows"] = (_row_err(host_f64(mid["dh"]), dh_ref), 0.0)
    counts = ref["fw"]["counts"]
    g13, g2 = dw13.cpu().numpy(), dw2.cpu().numpy()
    for n, got, want in (("dw13", g13, ref["dw13"]), ("dw2", g2, ref["dw2"])):
        per = [_tensor_err(got[e], want[e]) for e in range(wl.E) if counts[e] > 0]
        errs[n] = (max(p[0] for p in per), max(p[1] for p in per))
        idle = np.nonzero(counts == 0)[0]
        assert not got[idle].any(), f"{n}: nonzero gradient of an idle expert"
    log(f"  {what}: " + " ".join(f"{n} {a:.1e}/{b:.1e}" for n, (a, b) in errs.items()) +
        f"; {int((counts == 0).sum())} idle experts with zero gradients")
    for n, (a, b) in errs.items():
        assert a <= TOL_GRAD and b <= TOL_GRAD, (n, a, b)


CASES = {
    # base workload, size changes
    "coarse": ("coarse_bf16", dict(T=300, H=256, I=512)),
    "fine_renorm": ("fine_bf16", dict(T=400, H=256, I=256)),
    "vfine": ("vfine_bf16", dict(T=200, H=512, I=256)),
    "skewed": ("skewed_bf16", dict(T=600, H=256, I=192)),
    # long reductions in the weight gradients: ~1000 rows per expert
    "wgrad_long_k": ("coarse_bf16", dict(T=2048, H=512, I=256, E=2, k=1)),
    # few tiles with K = 4096: the dgrad GEMMs cut them along K
    "ksplit_h": ("coarse_bf16", dict(T=64, H=4096, I=256, E=4, k=2)),
    "ksplit_i": ("coarse_bf16", dict(T=64, H=256, I=4096, E=4, k=2)),
    "one_token": ("fine_bf16", dict(T=1, H=128, I=128)),
    "k_eq_e": ("coarse_bf16", dict(T=257, H=128, I=256, E=4, k=4)),
    "ragged_renorm": ("coarse_bf16", dict(T=203, H=192, I=320, E=6, k=3, renormalize=True)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_small_full_compare(case):
    base, ch = CASES[case]
    wl = W.scaled(W.WORKLOADS[base], **ch)
    log(f"backward {case}: {wl}")
    inp = W.make_inputs(wl)
    dout = _dout(wl.T, wl.H, seed=wl.T + 7)
    res, _ = _run(inp, dout)
    _compare(inp, dout, res, case)


def test_backward_coarse_shapes():
    """The coarse workload's H, I, E and k (the GEMM shapes the forward
    benchmark runs), on 128 tokens so the float64 oracle stays quick."""
    wl = W.scaled(W.WORKLOADS["coarse_bf16"], T=128)
    log(f"backward coarse shapes: {wl}")
    inp = W.make_inputs(wl)
    dout = _dout(wl.T, wl.H, seed=3)
    res, _ = _run(inp, dout)
    _compare(inp, dout, res, "coarse shapes")


def test_backward_deterministic_and_events():
    wl = W.scaled(W.WORKLOADS["fine_bf16"], T=700, H=256, I=256)
    inp = W.make_inputs(wl)
    dout = _dout(wl.T, wl.H, seed=11)
    r1, d = _run(inp, dout)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(B.PROFILE_EVENTS_BACKWARD)]
    for e in ev:
        e.record()          # creates the HIP event behind the torch object
    torch.cuda.synchronize()
    r2, _ = _run(inp, dout, d, events=ev)
    for a, b in zip(r1[:5], r2[:5]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
    times = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    log("  stage ms " + " ".join(f"{s}={t:.3f}" for s, t in zip(B.PROFILE_STAGES_BACKWARD, times)))
    assert all(t >= 0 for t in times)


@pytest.mark.parametrize("case", ["coarse", "ksplit_h", "skewed"])
def test_backward_cached_gate_up(case):
    """The caching variant: moe_forward_train keeps g and u (its output is
    moe_forward's, bit for bit); they equal the sums the recomputing backward
    forms again, to one bf16 ulp (the two GEMMs tile the columns differently,
    so a tile cut along K may group its partial sums differently); and the
    backward that reads them meets the same bounds against the oracle."""
    base, ch = CASES[case]
    wl = W.scaled(W.WORKLOADS[base], **ch)
    log(f"backward cached {case}: {wl}")
    inp = W.make_inputs(wl)
    dbits = _dout(wl.T, wl.H, seed=wl.T + 7)
    d = upload(inp)
    out_t, gu, fws = B.moe_forward_train(d["x"], d["w_router"], d["bias"], d["w13"], d["w2"], wl.k,
                                         wl.renormalize)
    out_f, _ = B.moe_forward(d["x"], d["w_router"], d["bias"], d["w13"], d["w2"], wl.k,
                             wl.renormalize)
    torch.cuda.synchronize()
    assert torch.equal(out_t.view(torch.int16), out_f.view(torch.int16))
    dout = dev_tensor(dbits, "bf16")
    cached = B.moe_backward(d["x"], d["w_router"], d["bias"], d["w13"], d["w2"], wl.k,
                            wl.renormalize, fws, dout, gate_up=gu)
    recomp = B.moe_backward(d["x"], d["w_router"], d["bias"], d["w13"], d["w2"], wl.k,
                            wl.renormalize, fws, dout)
    torch.cuda.synchronize()
    g_rec = B.backward_intermediates(recomp[5], wl.T, wl.H, wl.I, wl.E, wl.k)["gu"].float()
    g_kept = gu.float()
    ulp = torch.maximum(g_rec.abs(), g_kept.abs()) * 2.0 ** -7
    assert bool(((g_kept - g_rec).abs() <= ulp).all()), "kept g/u differ from the recomputed ones"
    log(f"  kept g/u: {int((g_kept != g_rec).sum())} of {g_kept.numel()} differ by one ulp")
    _compare(inp, dbits, cached, case + " cached")


def test_backward_full_size_sampled():
    """The coarse workload at full size, as the training benchmark runs it
    (moe_forward_train keeping g and u, then moe_backward reading them):
    dx, dlogits and dw of sampled tokens, and per expert whole columns of
    dW2 and whole rows of dW13, against the oracle's one-by-one backward."""
    wl = W.WORKLOADS["coarse_bf16"]
    log(f"backward full size: {wl}")
    inp = W.make_inputs(wl)
    dbits = _dout(wl.T, wl.H, seed=29)
    d = upload(inp)
    _, gu, fws = B.moe_forward_train(d["x"], d["w_router"], d["bias"], d["w13"], d["w2"], wl.k,
                                     wl.renormalize)
    dout = dev_tensor(dbits, "bf16")
    dx, _, _, dw13, dw2, ws = B.moe_backward(d["x"], d["w_router"], d["bias"], d["w13"], d["w2"],
                                             wl.k, wl.renormalize, fws, dout, gate_up=gu)
    torch.cuda.synchronize()
    mid = B.backward_intermediates(ws, wl.T, wl.H, wl.I, wl.E, wl.k)
    ids, _, _, _ = O.route(inp.f32("x"), inp.f32("w_router"), inp.bias, wl.k, wl.renormalize)
    _, offs, perm, _ = O.permute(ids, wl.E)
    toks = sample_tokens(wl.T, ids, offs, perm, wl.k)
    r = np.random.default_rng(31)
    cols = sorted({0, wl.I - 1} | set(r.choice(wl.I, size=4, replace=False).tolist()))
    log(f"  oracle on {len(toks)} tokens and columns {cols}")
    ref = O.backward_sampled(inp.x, inp.w_router, inp.bias, inp.w13, inp.w2, wl.k, wl.renormalize,
                             W.bf16_bits_to_f32(dbits), toks, cols, to_f32=W.bf16_bits_to_f32)
    gpu_ids = B.forward_intermediates(fws, wl.T, wl.H, wl.I, wl.E, wl.k, B.MOE_DTYPE_BF16)["ids"]
    assert np.array_equal(ref["ids"], gpu_ids.cpu().numpy()), "routing differs from the oracle's"
    ti = torch.tensor(toks, device=dx.device)
    ci = torch.tensor(cols, device=dx.device)
    errs = {"dx rows": (_row_err(host_f64(dx[ti]), ref["dx"]), 0.0),
            "dlogits": _tensor_err(mid["dlogits"][ti].cpu().numpy(), ref["dlogits"]),
            "dw": _tensor_err(mid["dw"][ti].cpu().numpy(), ref["dw"])}
    g2 = dw2[:, :, ci].cpu().numpy()
    g13 = torch.stack([dw13[:, ci, :], dw13[:, ci + wl.I, :]], dim=1).cpu().numpy()
    per2 = [_tensor_err(g2[e], ref["dw2_cols"][e]) for e in range(wl.E) if ref["counts"][e] > 0]
    per13 = [_tensor_err(g13[e], ref["dw13_rows"][e]) for e in range(wl.E) if ref["counts"][e] > 0]
    errs["dw2 columns"] = (max(q[0] for q in per2), max(q[1] for q in per2))
    errs["dw13 rows"] = (max(q[0] for q in per13), max(q[1] for q in per13))
    log("  " + " ".join(f"{n} {a:.1e}/{b:.1e}" for n, (a, b) in errs.items()))
    for n, (a, b) in errs.items():
        assert a <= TOL_GRAD and b <= TOL_GRAD, (n, a, b)

