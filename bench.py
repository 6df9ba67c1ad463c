#!/usr/bin/env python3
"""Benchmark of the MoE block forward on one MI355X.

One step = one moe_forward over one batch of synthetic input (router, softmax,
top-k, permutation, gate/up grouped GEMM + SwiGLU, down grouped GEMM,
combine), inputs resident in HBM.  W untimed warm-up steps, then exactly K
timed steps between synchronisations; per-stage times come from HIP events
recorded by the library on the stream the kernels run on.  Prints one JSON
line.  The CPU oracle is timed on a bounded token sample as a reported
baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + grouped-GEMM % bf16 MFMA peak, 1× MI355X"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (block-scaled MXFP8 included)
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
BM = 256                       # rows per grouped-GEMM tile (bf16 kernels)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SOURCES = ["sparse_mixture_experts_19_amd/csrc/gemm_mfma.hip",
                "sparse_mixture_experts_19_amd/csrc/moe_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic(wl, counts, Is: int = 0, mx: bool = False):
    """Algorithmic flops / bytes per launch of every stage (real rows only;
    only the weights of experts that own rows are counted).  Is: intermediate
    size of the shared expert (0: none).  mx: MXFP8 expert GEMMs (operands of
    1 byte plus one scale byte per 32; y stays bf16)."""
    b = 2 if wl.dtype == "bf16" else 4
    q = 1 + 1 / 32 if mx else b          # bytes per GEMM operand element
    T, H, E, k, I = wl.T, wl.H, wl.E, wl.k, wl.I
    M = T * k
    active = int(sum(1 for c in counts if c > 0))
    st = {}
    st["route"] = dict(bytes=T * H * b + E * H * b + 8 * M, flops=2 * T * H * E)
    st["permute"] = dict(bytes=4 * M + 4 * M + 4 * M + 8 * E, flops=0)
    st["quantize_x"] = dict(bytes=T * H * b + T * H * (1 + 1 / 32), flops=0)
    st["gemm_gate_up_swiglu"] = dict(flops=4 * M * H * I,
                                     bytes=2 * active * I * H * q + M * H * q + M * I * q + 4 * M)
    st["gemm_down"] = dict(flops=2 * M * I * H, bytes=active * H * I * q + M * I * q + M * H * b)
    st["combine"] = dict(bytes=M * H * b + T * H * b + 8 * M + (T * H * b if Is else 0), flops=0)
    # token rounding: permutation of the routed ids (12 B per assignment), the
    # pooled-slot pass (8 B read per assignment, 9 B written per token) and the
    # new ids / weights pass (4 B read per assignment)
    st["token_round"] = dict(bytes=24 * M + 9 * T, flops=0)
    if Is:
        st["shared_expert"] = dict(flops=6 * T * H * Is,
                                   bytes=3 * Is * H * b + T * H * b + 2 * T * Is * b + T * H * b)
    # backward (moe_backward), bf16: per stage its GEMM flops and the bytes its
    # kernels must move at least (weights of active experts once, activations
    # once per pass; fp32 weight gradients written once)
    W13, W2 = 2 * active * I * H * b, active * H * I * b
    st["router_grads"] = dict(flops=4 * T * H * E + 2 * M * H,
                              bytes=M * H * b + 2 * T * H * b + E * H * (b + 4) + T * H * b)
    st["recompute_gate_up"] = dict(flops=4 * M * H * I, bytes=W13 + M * H * b + 2 * M * I * b)
    st["dgrad_down_swiglu"] = dict(flops=2 * M * H * I,
                                   bytes=W2 + M * H * b + M * I * b + 3 * M * I * b + 3 * M * I * b)
    st["dgrad_gate_up"] = dict(flops=4 * M * H * I, bytes=W13 + 2 * M * I * b + 2 * M * H * b + T * H * b)
    st["wgrad_transpose"] = dict(flops=0, bytes=2 * (2 * M * H * b + 3 * M * I * b))
    st["wgrad_down"] = dict(flops=2 * M * H * I, bytes=M * H * b + M * I * b + active * H * I * 4)
    st["wgrad_gate_up"] = dict(flops=4 * M * H * I,
                               bytes=2 * M * I * b + M * H * b + 2 * active * I * H * 4)
    return st


def workload_key(name: str, Is: int = 0, round_tile: int = 0, mx: bool = False,
                 train: bool = False, cache: bool = True) -> str:
    """The record's config.workload: the workload's name plus its variant
    (shared expert of intermediate size Is, token rounding with tile
    round_tile, MXFP8 experts, forward + backward with or without the cached
    gate/up sums).  Also the key of the workload's HBM counters in
    profiles/traffic.json."""
    return (name + (f"+shared{Is}" if Is else "") + (f"+round{round_tile}" if round_tile else "") +
            ("+mxfp8" if mx else "") + (("+train" if cache else "+train_recompute") if train else ""))


def padding_waste(counts, bm=BM):
    tiles = sum((c + bm - 1) // bm for c in counts)
    return 1.0 - sum(counts) / (tiles * bm) if tiles else 0.0


def cpu_baseline(inp, sample_tokens: int, shared=None, round_tile: int = 0, train: bool = False):
    """Time the oracle as it stands on the first ``sample_tokens`` tokens
    (with ``shared`` = (ws13, ws2) float32 arrays: the block with a shared expert;
    with ``round_tile``: the block with token rounding over those tokens; with
    ``train``: the backward, which runs the forward itself)."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:  # pragma: no cover
        threads = 1
    wl = inp.wl
    S = min(sample_tokens, wl.T)
    x = inp.f32("x")[:S]
    wr, w13, w2 = inp.f32("w_router"), inp.f32("w13"), inp.f32("w2")
    if train:
        dout = np.random.default_rng(12345).standard_normal((S, wl.H))
    t0 = time.perf_counter()
    if train:
        res = O.backward(x, wr, inp.bias, w13, w2, wl.k, wl.renormalize, dout)
        res = {"out": res["dx"]}
    elif round_tile:
        res = O.forward_rounded(x, wr, inp.bias, w13, w2, wl.k, wl.renormalize, round_tile)
    elif shared is None:
        res = O.forward(x, wr, inp.bias, w13, w2, wl.k, wl.renormalize)
    else:
        res = O.forward_shared(x, wr, inp.bias, w13, w2, shared[0], shared[1], wl.k, wl.renormalize)
    dt = time.perf_counter() - t0
    assert np.isfinite(res["out"]).all()
    return {"value": S / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {S} of {wl.T} tokens of {wl.name}, float64 numpy oracle "
                      f"(route{'+token rounding' if round_tile else ''}+permute+experts"
                      f"{'+backward' if train else ''}"
                      f"{'+shared expert' if shared is not None else ''}"
                      f"+combine), {dt:.1f} s"}


def standalone_calls(B, x, wr, bias, w13, w2, wl, iters: int = 10):
    """Median time of each of the four separate entry points (route, permute
    with the gathered rows, grouped SwiGLU GEMM, combine) over ``iters`` runs
    after one warm-up, buffers and workspaces allocated beforehand; and their
    sum.  The fused moe_forward gathers rows while loading instead of writing
    x_perm, so the sum is expected to exceed its time.  Also the median time
    of torch device copies of x-sized and y-sized buffers (not in the sum)."""
    import torch
    T, H, E, k, I = wl.T, wl.H, wl.E, wl.k, wl.I
    dev = x.device
    dt = B.MOE_DTYPE_BF16 if wl.dtype == "bf16" else B.MOE_DTYPE_F32
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws_r = torch.empty(max(B.workspace_size(B.ENTRY_ROUTE, T, H, 64, E, k, dt), 256), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(max(B.workspace_size(B.ENTRY_PERMUTE, T, H, 64, E, k, dt), 256), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(max(B.workspace_size(B.ENTRY_GROUPED_GEMM, T * k, H, I, E, 1, dt), 256), dtype=torch.uint8, device=dev)
    h = torch.empty((T * k, I), dtype=x.dtype, device=dev)
    y = torch.empty((T * k, H), dtype=x.dtype, device=dev)
    out = torch.empty((T, H), dtype=x.dtype, device=dev)
    state = {}

    def route():
        B.moe_route(x, wr, bias, k, wl.renormalize, ids, wts, ws_r)

    pout = (torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
            torch.empty(T * k, dtype=torch.int32, device=dev), torch.empty(T * k, dtype=torch.int32, device=dev),
            torch.empty((T * k, H), dtype=x.dtype, device=dev))

    def permute():
        state["p"] = B.moe_permute(ids, E, x, ws_p, out=pout)

    def gemm():
        B.moe_grouped_swiglu_gemm(state["p"][4], state["p"][1], w13, w2, h, y, ws_g)

    def combine():
        B.moe_combine(y, state["p"][3], wts, out)

    res = {}
    for name, fn in (("route", route), ("permute", permute), ("grouped_gemm", gemm),
                     ("combine", combine)):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        res[name + "_ms"] = round(sorted(times)[len(times) // 2], 5)
    res["sum_ms"] = round(sum(v for n, v in res.items()), 5)
    # Context for the memory-bound entry points: torch's own device copies
    # of an x-sized buffer (the router reads x once) and of a y-sized one
    # (the combine reads y once), timed the same way.
    xa, xb = torch.empty_like(x), torch.empty_like(x)
    ya = torch.empty_like(y)
    ya.zero_()
    for name, fn in (("copy_x", lambda: xb.copy_(xa)), ("copy_y", lambda: y.copy_(ya))):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        res[name + "_ms"] = round(sorted(times)[len(times) // 2], 5)
    return res


def library_reference(torch, B, wl, x, w13, w2, iters: int = 10):
    """The vendor library on the expert GEMM shapes of the workload, for
    context: torch.matmul (hipBLASLt) of M = T*k rows against one expert's
    weights (dense: all rows in one GEMM) and against each expert's weights in
    turn (M/E rows each: the per-expert loop without gather, ragged tails or
    fused epilogue).  Operands as the library stores them (weights [N, K]
    row-major, read through a transposed view, K contiguous on both sides);
    two-dimensional products only.  Beside them, this library's grouped GEMM
    (both GEMMs of moe_grouped_swiglu_gemm) on the same dense problem: one
    expert holding all M rows."""
    M, H, I, E = wl.T * wl.k, wl.H, wl.I, wl.E
    if wl.dtype != "bf16" or M % E:
        raise SystemExit("bench.py: --library-reference needs a bf16 workload with T*k a multiple of E")
    g = torch.Generator(device=x.device).manual_seed(0)
    a = torch.randn(M, H, device=x.device, generator=g).to(torch.bfloat16)
    h = torch.randn(M, I, device=x.device, generator=g).to(torch.bfloat16)
    m = M // E

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    def per_expert(src, w):
        for e in range(E):
            torch.matmul(src[e * m:(e + 1) * m], w[e].t())

    off = torch.tensor([0, M], dtype=torch.int32, device=x.device)
    h_out = torch.empty(M, I, dtype=torch.bfloat16, device=x.device)
    y_out = torch.empty(M, H, dtype=torch.bfloat16, device=x.device)
    runs = {
        "this_library_dense_gate_up_and_down": (
            lambda: B.moe_grouped_swiglu_gemm(a, off, w13[0:1], w2[0:1], h_out, y_out), 6 * M * H * I,
            f"{M}x{2 * I}x{H} + {M}x{H}x{I}"),
        "dense_gate_up": (lambda: torch.matmul(a, w13[0].t()), 4 * M * H * I, f"{M}x{2 * I}x{H}"),
        "dense_down": (lambda: torch.matmul(h, w2[0].t()), 2 * M * I * H, f"{M}x{H}x{I}"),
        "per_expert_gate_up": (lambda: per_expert(a, w13), 4 * M * H * I, f"{E} x {m}x{2 * I}x{H}"),
        "per_expert_down": (lambda: per_expert(h, w2), 2 * M * I * H, f"{E} x {m}x{H}x{I}"),
    }
    out = {}
    for name, (fn, flops, shape) in runs.items():
        ms = timed(fn)
        tf = flops / ms / 1e9
        out[name] = {"shape (MxNxK)": shape, "ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    return {"library_reference": out, "workload": wl.name, "library": "torch.matmul (hipBLASLt)",
            "torch": torch.__version__, "iterations": iters, "statistic": "median"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="coarse_bf16")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens for the CPU oracle baseline (default: sized per workload)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--report", default=None, help="also append the JSON record to this file")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run device-to-device copies of MB MiB (scales HBM byte counters)")
    ap.add_argument("--shared-intermediate", type=int, default=0, metavar="IS",
                    help="add a shared expert of intermediate size IS (moe_forward_shared)")
    ap.add_argument("--round", action="store_true",
                    help="token rounding to the grouped GEMM's row tile (moe_forward_rounded)")
    ap.add_argument("--round-tile", type=int, default=0, metavar="B",
                    help="token rounding to B rows (moe_forward_rounded)")
    ap.add_argument("--train", action="store_true",
                    help="forward + backward per step (moe_forward_train keeping g and u + "
                         "moe_backward reading them; gradients of sum(dout * out) for a seeded dout)")
    ap.add_argument("--train-recompute", action="store_true",
                    help="as --train, with the backward recomputing g and u (moe_forward + moe_backward)")
    ap.add_argument("--mxfp8", action="store_true",
                    help="MXFP8 expert GEMMs (moe_forward_mxfp8; weights quantized once, "
                         "before the timed steps)")
    ap.add_argument("--library-reference", action="store_true",
                    help="instead of the MoE block: time the vendor library (torch.matmul, "
                         "hipBLASLt) on dense and per-expert equivalents of the workload's two "
                         "expert GEMM shapes, for context")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the benchmark measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_mixture_experts_19_amd import binding as B
    from sparse_mixture_experts_19_amd import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}))
        return

    wl = W.WORKLOADS[args.workload]
    log(f"[bench] generating {wl.name} ...")
    t0 = time.perf_counter()
    inp = W.make_inputs(wl)
    log(f"[bench] inputs in {time.perf_counter() - t0:.1f} s; uploading")

    def up(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x, wr, w13, w2 = up(inp.x), up(inp.w_router), up(inp.w13), up(inp.w2)
    if args.library_reference:
        print(json.dumps(library_reference(torch, B, wl, x, w13, w2)))
        return
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    dt_code = B.MOE_DTYPE_BF16 if wl.dtype == "bf16" else B.MOE_DTYPE_F32
    out = torch.empty((wl.T, wl.H), dtype=x.dtype, device=dev)
    Is = args.shared_intermediate
    RB = args.round_tile or (B.gemm_tile_rows(dt_code) if args.round else 0)
    MX = args.mxfp8
    TR = args.train or args.train_recompute
    CACHE = not args.train_recompute
    if (RB and Is) or (MX and (RB or Is)) or (TR and (RB or Is or MX)):
        print("bench.py: --round, --shared-intermediate, --mxfp8 and --train do not combine",
              file=sys.stderr)
        sys.exit(2)
    if TR and wl.dtype != "bf16":
        print("bench.py: --train needs a bf16 workload", file=sys.stderr)
        sys.exit(2)
    wq_ms = None
    if MX:
        if wl.dtype != "bf16":
            print("bench.py: --mxfp8 needs a bf16 workload", file=sys.stderr)
            sys.exit(2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        w13q, w13s = B.mx_quantize(w13)
        w2q, w2s = B.mx_quantize(w2)
        e1.record()
        torch.cuda.synchronize()
        wq_ms = e0.elapsed_time(e1)
        del w13, w2
        nbytes = B.mxfp8_layout(wl.T, wl.H, wl.I, wl.E, wl.k).total
        stages, n_ev = B.PROFILE_STAGES_MXFP8, B.PROFILE_EVENTS_MXFP8
    elif RB:
        nbytes = B.rounded_layout(wl.T, wl.H, wl.I, wl.E, wl.k, dt_code).total
        stages, n_ev = B.PROFILE_STAGES_ROUNDED, B.PROFILE_EVENTS_ROUNDED
    elif Is:
        hs13, hs2 = W.make_shared_weights(wl, Is)
        ws13, ws2 = up(hs13), up(hs2)
        nbytes = B.shared_layout(wl.T, wl.H, wl.I, Is, wl.E, wl.k, dt_code).total
        stages, n_ev = B.PROFILE_STAGES_SHARED, B.PROFILE_EVENTS_SHARED
    else:
        nbytes = B.workspace_size(B.ENTRY_FORWARD, wl.T, wl.H, wl.I, wl.E, wl.k, dt_code)
        stages, n_ev = B.PROFILE_STAGES, B.PROFILE_EVENTS
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if TR:
        r = np.random.default_rng(12345)
        dout = up(W.f32_to_bf16_bits(r.standard_normal((wl.T, wl.H)).astype(np.float32)))
        bws = torch.empty(B.backward_layout(wl.T, wl.H, wl.I, wl.E, wl.k).total, dtype=torch.uint8,
                          device=dev)
        grads = dict(dx=torch.empty_like(x), dw_router=torch.empty((wl.E, wl.H), device=dev),
                     dbias=torch.empty(wl.E, device=dev),
                     dw13=torch.empty((wl.E, 2 * wl.I, wl.H), device=dev),
                     dw2=torch.empty((wl.E, wl.H, wl.I), device=dev))
        stages = tuple(stages) + B.PROFILE_STAGES_BACKWARD
        n_ev = n_ev + B.PROFILE_EVENTS_BACKWARD
        gate_up = torch.empty((wl.T * wl.k, 2 * wl.I), dtype=x.dtype, device=dev) if CACHE else None
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
           for _ in range(max(args.steps, 1))]
    for row in evs:
        for e in row:
            e.record()   # creates the underlying HIP event
    torch.cuda.synchronize()

    def step(i):
        if MX:
            B.moe_forward_mxfp8(x, wr, bias, w13q, w13s, w2q, w2s, wl.k, wl.renormalize, out, ws,
                                events=evs[i % len(evs)])
        elif RB:
            B.moe_forward_rounded(x, wr, bias, w13, w2, wl.k, wl.renormalize, RB, out, ws,
                                  events=evs[i % len(evs)])
        elif Is:
            B.moe_forward_shared(x, wr, bias, w13, w2, ws13, ws2, wl.k, wl.renormalize, out, ws,
                                 events=evs[i % len(evs)])
        else:
            ev = evs[i % len(evs)]
            if TR and CACHE:
                B.moe_forward_train(x, wr, bias, w13, w2, wl.k, wl.renormalize, out, gate_up, ws,
                                    events=ev[:B.PROFILE_EVENTS])
            else:
                B.moe_forward_profiled(x, wr, bias, w13, w2, wl.k, wl.renormalize, out, ws,
                                       ev[:B.PROFILE_EVENTS])
            if TR:
                B.moe_backward(x, wr, bias, w13, w2, wl.k, wl.renormalize, ws, dout,
                               workspace=bws, events=ev[B.PROFILE_EVENTS:], gate_up=gate_up, **grads)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    stage_ms = {s: 0.0 for s in stages}
    # event index of each stage's start (with --train the backward's events
    # follow the forward's, whose last one closes the forward's last stage)
    starts = list(range(len(stages)))
    if TR:
        nf = B.PROFILE_EVENTS - 1
        starts = list(range(nf)) + [B.PROFILE_EVENTS + j for j in range(len(stages) - nf)]
    for i in range(args.steps):
        for j, s in enumerate(stages):
            stage_ms[s] += evs[i][starts[j]].elapsed_time(evs[i][starts[j] + 1]) / args.steps
    if MX:
        mid = B.mxfp8_intermediates(ws, wl.T, wl.H, wl.I, wl.E, wl.k)
    else:
        mid = B.forward_intermediates(ws, wl.T, wl.H, wl.I, wl.E, wl.k, dt_code)
    counts = mid["counts"].cpu().numpy().tolist()

    alg = algorithmic(wl, counts, Is, MX)
    if TR and CACHE:
        # the backward reads the kept g and u instead of forming them again
        alg["recompute_gate_up"] = dict(flops=0, bytes=0)
        alg["gemm_gate_up_swiglu"]["bytes"] += 4 * wl.T * wl.k * wl.I
    detail = {}
    for s in stages:
        t = stage_ms[s] * 1e-3
        d = {"ms": round(stage_ms[s], 5)}
        if alg[s]["bytes"]:
            d["GB/s"] = round(alg[s]["bytes"] / t / 1e9, 1)
            if not alg[s]["flops"]:
                d["frac_hbm"] = round(alg[s]["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4)
        if alg[s]["flops"]:
            d["TFLOP/s"] = round(alg[s]["flops"] / t / 1e12, 1)
        detail[s] = d
    gemm_stages = ["gemm_gate_up_swiglu", "gemm_down"]
    if TR:
        gemm_stages += ["dgrad_down_swiglu", "dgrad_gate_up", "wgrad_down", "wgrad_gate_up"]
        if not CACHE:
            gemm_stages.append("recompute_gate_up")
    g_t = sum(stage_ms[s] for s in gemm_stages) * 1e-3
    g_flops = sum(alg[s]["flops"] for s in gemm_stages)
    peak = PEAK_FP8_TFLOPS if MX else PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    grouped_tflops = g_flops / g_t / 1e12
    # attainable rate of the two forward GEMMs: min(MFMA peak, intensity x HBM peak)
    fw_bytes = sum(alg[s]["bytes"] for s in ("gemm_gate_up_swiglu", "gemm_down"))
    fw_flops = sum(alg[s]["flops"] for s in ("gemm_gate_up_swiglu", "gemm_down"))
    attainable = min(peak, fw_flops / fw_bytes * PEAK_HBM_GBS / 1e3) if fw_bytes else peak

    # expert loads ([Qwen3-MoE page] §3 suggests watching their spread) and
    # the router's share of the step ([Hunyuan page] §六.2 puts routing at
    # about 15% extra compute)
    cnt = np.asarray(counts, dtype=np.float64)
    load = {"counts": [int(c) for c in counts], "mean": round(float(cnt.mean()), 2),
            "std": round(float(cnt.std()), 2),
            "std_over_mean": round(float(cnt.std() / cnt.mean()), 4) if cnt.mean() else None,
            "max": int(cnt.max()), "max_over_mean": round(float(cnt.max() / cnt.mean()), 3) if cnt.mean() else None,
            "empty_experts": int((cnt == 0).sum())}
    step_stage_ms = sum(stage_ms.values())

    # dominant kernel roofline
    dom = max(stages, key=lambda s: stage_ms[s])
    a = alg[dom]
    tdom = stage_ms[dom] * 1e-3
    ai = a["flops"] / a["bytes"] if a["bytes"] else 0.0
    if a["flops"] and (wl.dtype != "bf16" or ai >= peak * 1e12 / (PEAK_HBM_GBS * 1e9)):
        roof = {"bound": "mfma" if wl.dtype == "bf16" else "alu", "achieved": a["flops"] / tdom / 1e12,
                "peak": peak, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": a["bytes"] / tdom / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["achieved"] = round(roof["achieved"], 2)
    roof["frac"] = round(roof["frac"], 4)
    roof["kernel"] = dom
    roof["traffic"] = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        # keyed by the workload string of the record's config (shared expert,
        # rounding, MXFP8 and training variants have their own entries)
        rec = tr.get(workload_key(wl.name, Is, RB, MX, TR, CACHE), {}).get(dom)
        if rec and rec.get("source_sha256") == gemm_source_hash():
            roof["traffic"] = rec["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    roof["algorithmic_bytes"] = int(a["bytes"])
    roof["traffic_over_algorithmic"] = (round(roof["traffic"] / a["bytes"], 3)
                                        if roof["traffic"] and a["bytes"] else None)

    rec = {
        "metric": METRIC,
        "value": round(wl.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if MX else "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,1/fan_in) weights)",
        "config": {"workload": workload_key(wl.name, Is, RB, MX, TR, CACHE), "tokens": wl.T,
                   "hidden": wl.H, "experts": wl.E, "top_k": wl.k, "intermediate": wl.I,
                   "shared_intermediate": Is, "round_tile": RB, "renormalize": wl.renormalize,
                   "router_bias": wl.bias, "parallelism": "single GPU"},
        "grouped_gemm": {"TFLOP/s": round(grouped_tflops, 1),
                         "frac_of_peak": round(grouped_tflops / peak, 4),
                         "attainable_TFLOP/s": round(attainable, 1),
                         "frac_of_attainable": round(grouped_tflops / attainable, 4),
                         "padding_waste_bm256": round(padding_waste(counts), 4)},
        "expert_load": load,
        "router_time_share": round(stage_ms.get("route", 0.0) / step_stage_ms, 4) if step_stage_ms else None,
        "stages": detail,
        "roofline": roof,
    }
    if not (MX or TR or RB or Is):
        log("[bench] standalone entry points")
        rec["standalone_calls"] = standalone_calls(B, x, wr, bias, w13, w2, wl)
    if MX:
        rec["weight_quantization_ms"] = round(wq_ms, 3)
    if MX and not args.no_cpu:
        rec["cpu_baseline"] = None
        rec["cpu_baseline_note"] = ("not timed for --mxfp8: the oracle's quantization of the "
                                    "expert weights alone takes minutes at this size; the bf16 "
                                    "line of the same workload carries the CPU baseline")
    elif not args.no_cpu:
        sample = args.cpu_sample or {"tiny_f32": 512, "coarse_bf16": 4096, "fine_bf16": 4096,
                                     "vfine_bf16": 4096, "skewed_bf16": 8192}.get(wl.name, 1024)
        log(f"[bench] CPU oracle baseline on {sample} tokens")
        sh = None
        if Is:
            cv = (lambda a: W.bf16_bits_to_f32(a)) if wl.dtype == "bf16" else (lambda a: a)
            sh = (cv(hs13), cv(hs2))
        if TR:
            sample = min(sample, 1024)
        rec["cpu_baseline"] = cpu_baseline(inp, sample, sh, RB, train=TR)
    line = json.dumps(rec)
    print(line, flush=True)
    if args.report:
        with open(args.report, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
