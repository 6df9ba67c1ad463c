"""The C ABI library without a GPU: it loads, exports every declared symbol,
sizes its workspaces and rejects bad arguments before touching the device."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

from sparse_mixture_experts_19_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libmoe_mi355x.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_grouped_swiglu_gemm", "moe_combine", "moe_forward"):
        assert n in names


def test_every_declared_symbol_is_exported():
    L = B.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                             text=True).stdout
        exported = set(re.findall(r"\sT\s(moe_\w+)$", out, flags=re.M))
        assert set(declared_functions()) <= exported


def test_version_and_status_strings():
    L = B.lib()
    assert L.moe_version() == 106
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(3) == b"MOE_ERR_WORKSPACE"
    assert L.moe_status_string(99) == b"MOE_ERR_UNKNOWN"


def test_workspace_sizes_and_layout():
    T, H, I, E, k = 4096, 4096, 14336, 8, 2
    for entry in range(5):
        assert B.workspace_size(entry, T, H, I, E, k, B.MOE_DTYPE_BF16) >= 0
    Lay = B.forward_layout(T, H, I, E, k, B.MOE_DTYPE_BF16)
    offs = [Lay.topk_ids, Lay.topk_weights, Lay.expert_counts, Lay.expert_offsets, Lay.perm,
            Lay.inv_perm, Lay.h, Lay.y, Lay.scratch, Lay.total]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and len(set(offs)) == len(offs)
    M = T * k
    assert Lay.y - Lay.h >= M * I * 2 and Lay.scratch - Lay.y >= M * H * 2
    assert Lay.total == B.workspace_size(B.ENTRY_FORWARD, T, H, I, E, k, B.MOE_DTYPE_BF16)


FAKE = 0x10000   # aligned, never dereferenced: validation fails first


def _route(**kw):
    a = dict(x=FAKE, w=FAKE, b=None, T=16, H=64, E=8, k=2, dt=1, ren=0, ids=FAKE, wts=FAKE,
             ws=FAKE, wsb=1 << 30, s=None)
    a.update(kw)
    return B.lib().moe_route(a["x"], a["w"], a["b"], a["T"], a["H"], a["E"], a["k"], a["dt"],
                             a["ren"], a["ids"], a["wts"], a["ws"], a["wsb"], a["s"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=9, E=8), B.MOE_ERR_INVALID_ARG),       # k > E
    (dict(k=0), B.MOE_ERR_INVALID_ARG),
    (dict(T=-1), B.MOE_ERR_INVALID_ARG),
    (dict(E=300, k=2), B.MOE_ERR_UNSUPPORTED),     # E > 256
    (dict(E=16, k=9), B.MOE_ERR_UNSUPPORTED),      # k > 8
    (dict(H=100), B.MOE_ERR_UNSUPPORTED),          # H % 64
    (dict(dt=7), B.MOE_ERR_UNSUPPORTED),
    (dict(x=None), B.MOE_ERR_INVALID_ARG),
    (dict(x=FAKE + 8), B.MOE_ERR_INVALID_ARG),     # misaligned
    (dict(ids=None), B.MOE_ERR_INVALID_ARG),
    (dict(wsb=16), B.MOE_ERR_WORKSPACE),
    (dict(ws=None), B.MOE_ERR_WORKSPACE),
    (dict(T=0, x=None, ids=None), B.MOE_OK),       # T == 0: valid no-op
])
def test_route_argument_errors(kw, status):
    assert _route(**kw) == status
    if status != B.MOE_OK:
        assert len(B.lib().moe_last_error()) > 0


def test_other_entries_argument_errors():
    L = B.lib()
    # permute: x and x_perm must come together
    assert L.moe_permute(FAKE, FAKE, 8, 64, 4, 2, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
                         None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_permute(FAKE, None, 8, 64, 4, 2, 1, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 20,
                         None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_permute(FAKE, None, 8, 64, 4, 2, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4,
                         None) == B.MOE_ERR_WORKSPACE
    # grouped gemm: I must be a multiple of 64, workspace large enough
    assert L.moe_grouped_swiglu_gemm(FAKE, FAKE, FAKE, FAKE, 64, 64, 100, 4, 1, FAKE, FAKE, FAKE,
                                     1 << 20, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_grouped_swiglu_gemm(FAKE, FAKE, FAKE, FAKE, 64, 64, 128, 4, 1, FAKE, FAKE, FAKE,
                                     8, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_grouped_swiglu_gemm(FAKE, FAKE, FAKE, FAKE, 0, 64, 128, 4, 1, None, None, None,
                                     0, None) == B.MOE_OK
    # combine
    assert L.moe_combine(FAKE, FAKE, FAKE, 8, 64, 2, 1, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(FAKE, FAKE, FAKE, 8, 64, 0, 1, FAKE, None) == B.MOE_ERR_INVALID_ARG
    # forward
    assert L.moe_forward(FAKE, FAKE, None, FAKE, FAKE, 8, 64, 128, 4, 5, 1, 0, FAKE, FAKE, 1 << 30,
                         None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward(FAKE, FAKE, None, FAKE, FAKE, 8, 64, 128, 4, 2, 1, 0, FAKE, FAKE, 64,
                         None) == B.MOE_ERR_WORKSPACE
    assert L.moe_forward(FAKE, FAKE, None, FAKE, FAKE, 0, 64, 128, 4, 2, 1, 0, None, None, 0,
                         None) == B.MOE_OK
    size = ctypes.c_size_t(0)
    assert L.moe_workspace_size(9, 8, 64, 64, 4, 2, 1, ctypes.byref(size)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_size(0, 8, 64, 64, 4, 2, 1, None) == B.MOE_ERR_INVALID_ARG


def test_shared_expert_layout_and_argument_errors():
    T, H, I, Is, E, k = 4096, 4096, 14336, 5632, 8, 2
    S = B.shared_layout(T, H, I, Is, E, k, B.MOE_DTYPE_BF16)
    R = B.forward_layout(T, H, I, E, k, B.MOE_DTYPE_BF16)
    # the routed part is laid out exactly as moe_forward's, the shared regions follow it
    for f, _ in B.ForwardLayout._fields_:
        assert getattr(S.routed, f) == getattr(R, f), f
    offs = [R.total, S.h_shared, S.y_shared, S.scratch, S.total]
    assert S.h_shared >= R.total and all(o % 256 == 0 for o in offs[1:])
    assert S.y_shared - S.h_shared >= T * Is * 2 and S.scratch - S.y_shared >= T * H * 2
    L = B.lib()
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("x", FAKE), ("wr", FAKE), ("b", None), ("w13", FAKE), ("w2", FAKE), ("ws13", FAKE),
        ("ws2", FAKE), ("T", 8), ("H", 64), ("I", 128), ("Is", 128), ("E", 4), ("k", 2),
        ("dt", 1), ("ren", 0), ("out", FAKE), ("ws", FAKE), ("wsb", 1 << 30), ("s", None))]
    assert L.moe_forward_shared(*args(ws13=None)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward_shared(*args(ws2=FAKE + 4)) == B.MOE_ERR_INVALID_ARG   # misaligned
    assert L.moe_forward_shared(*args(Is=100)) == B.MOE_ERR_UNSUPPORTED          # Is % 64
    assert L.moe_forward_shared(*args(Is=0)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward_shared(*args(wsb=1024)) == B.MOE_ERR_WORKSPACE
    assert L.moe_forward_shared(*args(T=0, x=None, out=None, ws=None, wsb=0)) == B.MOE_OK
    lay = B.SharedLayout()
    assert L.moe_forward_shared_layout(8, 64, 128, 96, 4, 2, 1, ctypes.byref(lay)) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_forward_shared_layout(8, 64, 128, 128, 4, 2, 1, None) == B.MOE_ERR_INVALID_ARG


def test_rounded_layout_and_argument_errors():
    T, H, I, E, k = 16384, 2048, 768, 128, 8
    R = B.forward_layout(T, H, I, E, k, B.MOE_DTYPE_BF16)
    Q = B.rounded_layout(T, H, I, E, k, B.MOE_DTYPE_BF16)
    # same intermediates at the same offsets, a larger scratch region
    for f, _ in B.ForwardLayout._fields_:
        if f != "total":
            assert getattr(Q, f) == getattr(R, f), f
    assert Q.total > R.total and Q.total % 256 == 0
    assert B.gemm_tile_rows(B.MOE_DTYPE_BF16) == 256 and B.gemm_tile_rows(B.MOE_DTYPE_F32) == 64
    L = B.lib()
    assert L.moe_gemm_tile_rows(7) == 0 and len(L.moe_last_error()) > 0
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("x", FAKE), ("wr", FAKE), ("b", None), ("w13", FAKE), ("w2", FAKE), ("T", 8), ("H", 64),
        ("I", 128), ("E", 4), ("k", 2), ("dt", 1), ("ren", 0), ("B", 256), ("out", FAKE),
        ("ws", FAKE), ("wsb", 1 << 30), ("s", None))]
    assert L.moe_forward_rounded(*args(B=0)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward_rounded(*args(B=-5)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward_rounded(*args(k=5)) == B.MOE_ERR_INVALID_ARG            # k > E
    assert L.moe_forward_rounded(*args(w13=None)) == B.MOE_ERR_INVALID_ARG
    # the rounded path needs more workspace than moe_forward's
    small = B.forward_layout(8, 64, 128, 4, 2, B.MOE_DTYPE_BF16).total
    assert L.moe_forward_rounded(*args(wsb=small)) == B.MOE_ERR_WORKSPACE
    assert L.moe_forward_rounded(*args(T=0, x=None, out=None, ws=None, wsb=0)) == B.MOE_OK
    assert L.moe_forward_rounded_profiled(*args()[:-1], None, 0, None) == B.MOE_ERR_INVALID_ARG
    ev = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    assert L.moe_forward_rounded_profiled(*args()[:-1], ev, B.PROFILE_EVENTS_ROUNDED - 1, None) == B.MOE_ERR_INVALID_ARG
    lay = B.ForwardLayout()
    assert L.moe_forward_rounded_layout(8, 64, 100, 4, 2, 1, ctypes.byref(lay)) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_forward_rounded_layout(8, 64, 128, 4, 2, 1, None) == B.MOE_ERR_INVALID_ARG


def test_mxfp8_layout_and_argument_errors():
    T, H, I, E, k = 4096, 4096, 14336, 8, 2
    M = T * k
    X = B.mxfp8_layout(T, H, I, E, k)
    offs = [X.topk_ids, X.topk_weights, X.expert_counts, X.expert_offsets, X.perm, X.inv_perm,
            X.x_codes, X.x_scales, X.h_codes, X.h_scales, X.y, X.x_scale_words, X.w13_scale_words,
            X.w2_scale_words, X.scratch, X.total]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and len(set(offs)) == len(offs)
    assert X.x_scales - X.x_codes >= T * H and X.h_codes - X.x_scales >= T * H // 32
    assert X.h_scales - X.h_codes >= M * I and X.y - X.h_scales >= M * I // 32
    assert X.x_scale_words - X.y >= M * H * 2
    assert X.w13_scale_words - X.x_scale_words >= M * H // 32
    assert X.w2_scale_words - X.w13_scale_words >= E * 2 * I * H // 32
    assert X.scratch - X.w2_scale_words >= E * H * I // 32
    L = B.lib()
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("x", FAKE), ("wr", FAKE), ("b", None), ("w13q", FAKE), ("w13s", FAKE), ("w2q", FAKE),
        ("w2s", FAKE), ("T", 8), ("H", 128), ("I", 128), ("E", 4), ("k", 2), ("dt", 1), ("ren", 0),
        ("out", FAKE), ("ws", FAKE), ("wsb", 1 << 30), ("s", None))]
    assert L.moe_forward_mxfp8(*args(dt=0)) == B.MOE_ERR_UNSUPPORTED             # bf16 only
    assert L.moe_forward_mxfp8(*args(H=64)) == B.MOE_ERR_UNSUPPORTED             # H % 128
    assert L.moe_forward_mxfp8(*args(I=192)) == B.MOE_ERR_UNSUPPORTED            # I % 128
    assert L.moe_forward_mxfp8(*args(k=5)) == B.MOE_ERR_INVALID_ARG              # k > E
    assert L.moe_forward_mxfp8(*args(w2s=None)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward_mxfp8(*args(w13q=FAKE + 4)) == B.MOE_ERR_INVALID_ARG    # misaligned
    assert L.moe_forward_mxfp8(*args(wsb=1024)) == B.MOE_ERR_WORKSPACE
    assert L.moe_forward_mxfp8(*args(T=1 << 22, H=2048)) == B.MOE_ERR_UNSUPPORTED  # T*H > 2^32
    assert L.moe_forward_mxfp8(*args(T=0, x=None, out=None, ws=None, wsb=0)) == B.MOE_OK
    assert L.moe_forward_mxfp8_profiled(*args()[:-1], None, 0, None) == B.MOE_ERR_INVALID_ARG
    ev = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    assert L.moe_forward_mxfp8_profiled(*args()[:-1], ev, B.PROFILE_EVENTS_MXFP8 - 1, None) == B.MOE_ERR_INVALID_ARG
    lay = B.Mxfp8Layout()
    assert L.moe_forward_mxfp8_layout(8, 128, 100, 4, 2, 1, ctypes.byref(lay)) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_forward_mxfp8_layout(8, 128, 128, 4, 2, 1, None) == B.MOE_ERR_INVALID_ARG
    # quantize: cols a positive multiple of 32, known dtype, aligned pointers
    assert L.moe_mx_quantize(FAKE, 4, 48, 1, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_mx_quantize(FAKE, 4, 0, 1, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_mx_quantize(FAKE, -1, 32, 1, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_mx_quantize(FAKE, 4, 32, 5, FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_mx_quantize(FAKE, 4, 32, 1, FAKE, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_mx_quantize(FAKE + 8, 4, 32, 1, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_mx_quantize(None, 0, 32, 1, None, None, None) == B.MOE_OK


def test_backward_layout_and_argument_errors():
    T, H, I, E, k = 4096, 4096, 14336, 8, 2
    M = T * k
    Lb = B.backward_layout(T, H, I, E, k)
    assert Lb.ld % 64 == 0 and Lb.ld >= M + 64 * E
    offs = [Lb.dw, Lb.dlogits, Lb.dx_router, Lb.gu, Lb.dh, Lb.dgdu, Lb.h, Lb.dx_slots,
            Lb.padded_offsets, Lb.dyT, Lb.hT, Lb.dgduT, Lb.xT, Lb.scratch, Lb.total]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and len(set(offs)) == len(offs)
    assert Lb.dh - Lb.gu >= M * 2 * I * 2
    assert Lb.scratch - Lb.xT >= H * Lb.ld * 2
    L = B.lib()
    fw = B.forward_layout(8, 128, 128, 4, 2, B.MOE_DTYPE_BF16).total
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("x", FAKE), ("wr", FAKE), ("b", None), ("w13", FAKE), ("w2", FAKE), ("T", 8), ("H", 128),
        ("I", 128), ("E", 4), ("k", 2), ("dt", 1), ("ren", 0), ("fws", FAKE), ("fwsb", fw),
        ("gu", None), ("dout", FAKE), ("dx", FAKE), ("dwr", FAKE), ("db", None), ("dw13", FAKE), ("dw2", FAKE),
        ("ws", FAKE), ("wsb", 1 << 30), ("s", None))]
    assert L.moe_backward(*args(dt=0)) == B.MOE_ERR_UNSUPPORTED             # bf16 only
    assert L.moe_backward(*args(k=5)) == B.MOE_ERR_INVALID_ARG              # k > E
    assert L.moe_backward(*args(I=100)) == B.MOE_ERR_UNSUPPORTED            # I % 64
    assert L.moe_backward(*args(dout=None)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_backward(*args(dw2=FAKE + 4)) == B.MOE_ERR_INVALID_ARG     # misaligned
    assert L.moe_backward(*args(fwsb=fw - 1)) == B.MOE_ERR_WORKSPACE        # forward workspace too small
    assert L.moe_backward(*args(fws=None)) == B.MOE_ERR_WORKSPACE
    assert L.moe_backward(*args(gu=FAKE + 2)) == B.MOE_ERR_INVALID_ARG       # misaligned gate_up
    # the training forward: bf16 only, gate_up required, events count checked
    targs = lambda **kw: [kw.get(n, d) for n, d in (
        ("x", FAKE), ("wr", FAKE), ("b", None), ("w13", FAKE), ("w2", FAKE), ("T", 8), ("H", 128),
        ("I", 128), ("E", 4), ("k", 2), ("dt", 1), ("ren", 0), ("out", FAKE), ("gu", FAKE),
        ("ws", FAKE), ("wsb", 1 << 30), ("ev", None), ("nev", 0), ("s", None))]
    assert L.moe_forward_train(*targs(dt=0)) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_forward_train(*targs(gu=None)) == B.MOE_ERR_INVALID_ARG
    nev = B.PROFILE_EVENTS
    assert L.moe_forward_train(*targs(ev=(ctypes.c_void_p * nev)(*([FAKE] * nev)), nev=nev - 1)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward_train(*targs(wsb=64)) == B.MOE_ERR_WORKSPACE
    assert L.moe_backward(*args(wsb=1024)) == B.MOE_ERR_WORKSPACE
    assert L.moe_backward(*args(T=0, x=None, dout=None, dx=None, fws=None, fwsb=0, ws=None,
                                wsb=0)) == B.MOE_OK
    assert L.moe_backward_profiled(*args()[:-1], None, 0, None) == B.MOE_ERR_INVALID_ARG
    ev = (ctypes.c_void_p * B.PROFILE_EVENTS_BACKWARD)(*([FAKE] * B.PROFILE_EVENTS_BACKWARD))
    assert L.moe_backward_profiled(*args()[:-1], ev, B.PROFILE_EVENTS_BACKWARD - 1, None) == B.MOE_ERR_INVALID_ARG
    lay = B.BackwardLayout()
    assert L.moe_backward_workspace_layout(8, 128, 128, 4, 2, 0, ctypes.byref(lay)) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_backward_workspace_layout(8, 128, 128, 4, 2, 1, None) == B.MOE_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_gpu_is_unsupported():
    assert _route() == B.MOE_ERR_UNSUPPORTED
