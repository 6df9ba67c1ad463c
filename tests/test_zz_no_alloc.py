"""The allocation-free permutation (moe_permute_static) against moe_permute:
same counts, offsets, permutation, inverse and gathered rows, bit for bit, on
two calls in a row (the second smaller, so stale entries of the shared device
scratch would show), and its size limit reported as an error before launch."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_19_amd import binding as B
from moe_test_utils import log

pytestmark = pytest.mark.gpu


def _ids(T, E, k, seed, skew=False):
    g = torch.Generator().manual_seed(seed)
    if skew:   # a few experts take most rows, some none
        p = torch.tensor([0.5 ** (e % 12) for e in range(E)])
        rows = [torch.multinomial(p, k, replacement=False, generator=g) for _ in range(T)]
    else:
        rows = [torch.randperm(E, generator=g)[:k] for _ in range(T)]
    return torch.stack(rows).int().cuda()


@pytest.mark.parametrize("with_x", [False, True])
def test_permute_static_matches_permute(with_x):
    cases = [(20000, 2048, 128, 8, 1, False), (3000, 1024, 64, 4, 2, True)]   # second call smaller
    for T, H, E, k, seed, skew in cases:
        log(f"permute_static T={T} H={H} E={E} k={k} x={with_x}")
        ids = _ids(T, E, k, seed, skew)
        x = torch.randn(T, H, device="cuda").bfloat16() if with_x else None
        want = B.moe_permute(ids, E, x=x)
        got = B.moe_permute_static(ids, E, x=x)
        torch.cuda.synchronize()
        for name, a, b in zip(("counts", "offsets", "perm", "inv_perm"), got[:4], want[:4]):
            assert torch.equal(a, b), name
        if with_x:
            assert torch.equal(got[4].view(torch.int16), want[4].view(torch.int16))
        assert int(got[1][-1]) == T * k


def test_permute_static_size_limit():
    E, k = 256, 8
    T = (1 << 22) // k + 1024           # ceil(T*k/1024) * E beyond 2^20 entries
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_permute_static(ids, E)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    log(f"size limit: {ei.value}")
