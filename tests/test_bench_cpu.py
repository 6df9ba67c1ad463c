"""Host logic of bench.py (no GPU): the refusal of more than one GPU, the
algorithmic flop counts against the closed forms of the configurations, the
padding-waste count and the key that ties a record to its HBM counters."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sparse_mixture_experts_19_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


# flops of the five configurations, from their dimensions alone:
# router 2·T·H·E, gate/up 4·M·H·I, down 2·M·I·H with M = T·k
@pytest.mark.parametrize("name,router,gate_up,down", [
    ("tiny_f32", 2.097152e6, 0.536870912e9, 0.268435456e9),
    ("coarse_bf16", 0.268435456e9, 1924.145348608e9, 962.072674304e9),
    ("fine_bf16", 8.589934592e9, 824.633720832e9, 412.316860416e9),
    ("vfine_bf16", 17.179869184e9, 274.877906944e9, 137.438953472e9),
    ("skewed_bf16", 8.589934592e9, 1099.511627776e9, 549.755813888e9),
])
def test_algorithmic_flops(name, router, gate_up, down):
    wl = W.WORKLOADS[name]
    st = bench.algorithmic(wl, [1] * wl.E)
    assert st["route"]["flops"] == pytest.approx(router, rel=1e-12)
    assert st["gemm_gate_up_swiglu"]["flops"] == pytest.approx(gate_up, rel=1e-12)
    assert st["gemm_down"]["flops"] == pytest.approx(down, rel=1e-12)


def test_algorithmic_bytes_count_active_experts_only():
    wl = W.WORKLOADS["coarse_bf16"]
    full = bench.algorithmic(wl, [1] * wl.E)["gemm_down"]["bytes"]
    half = bench.algorithmic(wl, [1] * (wl.E // 2) + [0] * (wl.E // 2))["gemm_down"]["bytes"]
    # the down weights of an expert: H x I bf16
    assert full - half == (wl.E // 2) * wl.H * wl.I * 2


def test_padding_waste():
    assert bench.padding_waste([256, 512], bm=256) == 0.0
    assert bench.padding_waste([257], bm=256) == pytest.approx(1 - 257 / 512)
    assert bench.padding_waste([0, 1, 0], bm=256) == pytest.approx(1 - 1 / 256)
    assert bench.padding_waste([0, 0], bm=256) == 0.0


def test_workload_key_matches_traffic_entries():
    assert bench.workload_key("coarse_bf16") == "coarse_bf16"
    assert bench.workload_key("coarse_bf16", mx=True) == "coarse_bf16+mxfp8"
    assert bench.workload_key("coarse_bf16", train=True) == "coarse_bf16+train"
    assert bench.workload_key("coarse_bf16", train=True, cache=False) == "coarse_bf16+train_recompute"
    assert bench.workload_key("fine_bf16", Is=2048) == "fine_bf16+shared2048"
    assert bench.workload_key("vfine_bf16", round_tile=256) == "vfine_bf16+round256"
    # every counted entry is a key a record can carry, for a workload that exists
    with open(bench.TRAFFIC_FILE) as f:
        keys = [k for k in json.load(f) if not k.startswith("_")]
    assert keys
    for k in keys:
        base, *variant = k.split("+")
        assert base in W.WORKLOADS
        assert variant in ([], ["mxfp8"], ["train"], ["train_recompute"]) or variant[0].startswith(("shared", "round"))
