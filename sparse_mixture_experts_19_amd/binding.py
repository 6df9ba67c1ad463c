"""ctypes binding of libmoe_mi355x (the C ABI in include/moe_mi355x.h).

Argument marshalling only: torch tensors supply device pointers, the current
HIP stream supplies the stream, and every step of the block runs in the HIP
kernels of the library.  There is no fallback: if the library is missing or
the device is not gfx950 the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
ENTRY_ROUTE, ENTRY_PERMUTE, ENTRY_GROUPED_GEMM, ENTRY_COMBINE, ENTRY_FORWARD = range(5)

_c_i32, _c_i64, _c_sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} [{status}]")
        self.status = status


class ForwardLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "topk_ids", "topk_weights", "expert_counts", "expert_offsets", "perm", "inv_perm",
        "h", "y", "scratch", "total")]


class SharedLayout(ctypes.Structure):
    _fields_ = [("routed", ForwardLayout)] + [(n, ctypes.c_size_t) for n in (
        "h_shared", "y_shared", "scratch", "total")]


class BackwardLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "dw", "dlogits", "dx_router", "gu", "dh", "dgdu", "h", "dx_slots",
        "padded_offsets", "dyT", "hT", "dgduT", "xT", "ld", "scratch", "total")]


class Mxfp8Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "topk_ids", "topk_weights", "expert_counts", "expert_offsets", "perm", "inv_perm",
        "x_codes", "x_scales", "h_codes", "h_scales", "y", "x_scale_words", "w13_scale_words",
        "w2_scale_words", "scratch", "total")]


_SIGS = {
    "moe_route": [_vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _c_sz, _vp],
    "moe_permute": [_vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp],
    "moe_permute_static": [_vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_grouped_swiglu_gemm": [_vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _c_sz, _vp],
    "moe_combine": [_vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _vp, _vp],
    "moe_forward": [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, _vp],
    "moe_forward_profiled": [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, ctypes.POINTER(ctypes.c_void_p), _c_i32, _vp],
    "moe_forward_shared": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, _vp],
    "moe_forward_shared_profiled": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, ctypes.POINTER(ctypes.c_void_p), _c_i32, _vp],
    "moe_forward_shared_layout": [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(SharedLayout)],
    "moe_forward_rounded": [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, _vp],
    "moe_forward_rounded_profiled": [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, ctypes.POINTER(ctypes.c_void_p), _c_i32, _vp],
    "moe_forward_rounded_layout": [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(ForwardLayout)],
    "moe_gemm_tile_rows": [_c_i32],
    "moe_mx_quantize": [_vp, _c_i64, _c_i32, _c_i32, _vp, _vp, _vp],
    "moe_backward": [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _c_sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp],
    "moe_backward_profiled": [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _c_sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_sz, ctypes.POINTER(ctypes.c_void_p), _c_i32, _vp],
    "moe_forward_train": [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _c_sz, ctypes.POINTER(ctypes.c_void_p), _c_i32, _vp],
    "moe_backward_workspace_layout": [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(BackwardLayout)],
    "moe_forward_mxfp8": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, _vp],
    "moe_forward_mxfp8_profiled": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _c_sz, ctypes.POINTER(ctypes.c_void_p), _c_i32, _vp],
    "moe_forward_mxfp8_layout": [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(Mxfp8Layout)],
    "moe_workspace_size": [_c_i32, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(ctypes.c_size_t)],
    "moe_forward_workspace_layout": [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(ForwardLayout)],
    "moe_status_string": [_c_i32],
    "moe_last_error": [],
    "moe_version": [],
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once (torch first, so its HIP runtime is the one used)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_mixture_experts_19_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name in ("moe_status_string", "moe_last_error") else ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != MOE_OK:
        L = lib()
        raise MoeError(status, f"{L.moe_status_string(status).decode()}: {L.moe_last_error().decode()}")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MOE_DTYPE_BF16
    if t == torch.float32:
        return MOE_DTYPE_F32
    raise TypeError(f"unsupported dtype {t}")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == MOE_DTYPE_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def version() -> int:
    return lib().moe_version()


def workspace_size(entry: int, T: int, H: int, I: int, E: int, k: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(entry, T, H, I, E, k, dtype, ctypes.byref(n)))
    return n.value


def forward_layout(T: int, H: int, I: int, E: int, k: int, dtype: int) -> ForwardLayout:
    L = ForwardLayout()
    _check(lib().moe_forward_workspace_layout(T, H, I, E, k, dtype, ctypes.byref(L)))
    return L


def _workspace(nbytes: int, dev, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


def moe_route(x, w_router, router_bias, k: int, renormalize: bool, topk_ids=None,
              topk_weights=None, workspace=None):
    """Router logits, softmax over all experts, top-k -> (ids [T,k] int32, weights [T,k] f32)."""
    T, H = x.shape
    E = w_router.shape[0]
    dt = _dtype_code(x.dtype)
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws = _workspace(workspace_size(ENTRY_ROUTE, T, H, 64, E, k, dt), dev, workspace)
    _check(lib().moe_route(_ptr(x), _ptr(w_router), _ptr(router_bias), T, H, E, k, dt,
                           int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_weights), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(dev)))
    return topk_ids, topk_weights


def moe_permute(topk_ids, E: int, x=None, workspace=None, out=None):
    """Expert histogram, offsets, stable expert-sorted permutation and its inverse;
    with ``x`` also the reordered rows.  ``out``: optional (counts, offsets, perm,
    inv, x_perm) tensors to write.  Returns (counts, offsets, perm, inv, x_perm)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    H = x.shape[1] if x is not None else 64
    dt = _dtype_code(x.dtype) if x is not None else MOE_DTYPE_BF16
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty((T * k, H), dtype=x.dtype, device=dev) if x is not None else None)
    counts, offsets, perm, inv, x_perm = out
    ws = _workspace(workspace_size(ENTRY_PERMUTE, T, H, 64, E, k, dt), dev, workspace)
    _check(lib().moe_permute(_ptr(topk_ids), _ptr(x), T, H, E, k, dt, _ptr(counts), _ptr(offsets),
                             _ptr(perm), _ptr(inv), _ptr(x_perm), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(dev)))
    return counts, offsets, perm, inv, x_perm


def moe_permute_static(topk_ids, E: int, x=None, out=None):
    """moe_permute without a workspace (the library's own device scratch).
    ``out``: optional (counts, offsets, perm, inv, x_perm) tensors to write.
    Returns (counts, offsets, perm, inv, x_perm)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    H = x.shape[1] if x is not None else 64
    dt = _dtype_code(x.dtype) if x is not None else MOE_DTYPE_BF16
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty((T * k, H), dtype=x.dtype, device=dev) if x is not None else None)
    counts, offsets, perm, inv, x_perm = out
    _check(lib().moe_permute_static(_ptr(topk_ids), _ptr(x), T, H, E, k, dt, _ptr(counts),
                                    _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(x_perm),
                                    _stream(dev)))
    return counts, offsets, perm, inv, x_perm


def moe_grouped_swiglu_gemm(x_perm, expert_offsets, w13, w2, h=None, y=None, workspace=None):
    """Every expert's SwiGLU MLP over its rows of ``x_perm`` -> (h [M,I], y [M,H])."""
    M, H = x_perm.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    dt = _dtype_code(x_perm.dtype)
    dev = x_perm.device
    if h is None:
        h = torch.empty((M, I), dtype=x_perm.dtype, device=dev)
    if y is None:
        y = torch.empty((M, H), dtype=x_perm.dtype, device=dev)
    ws = _workspace(workspace_size(ENTRY_GROUPED_GEMM, M, H, I, E, 1, dt), dev, workspace)
    _check(lib().moe_grouped_swiglu_gemm(_ptr(x_perm), _ptr(expert_offsets), _ptr(w13), _ptr(w2),
                                         M, H, I, E, dt, _ptr(h), _ptr(y), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(dev)))
    return h, y


def moe_combine(y, inv_perm, topk_weights, out=None):
    """out[t] = sum_j w[t,j] * y[inv_perm[t*k+j]]."""
    T, k = topk_weights.shape
    H = y.shape[1]
    dev = y.device
    if out is None:
        out = torch.empty((T, H), dtype=y.dtype, device=dev)
    _check(lib().moe_combine(_ptr(y), _ptr(inv_perm), _ptr(topk_weights), T, H, k,
                             _dtype_code(y.dtype), _ptr(out), _stream(dev)))
    return out


def moe_forward(x, w_router, router_bias, w13, w2, k: int, renormalize: bool, out=None,
                workspace=None):
    """The whole MoE block forward.  Returns (out, workspace); the intermediates
    can be read from the workspace with ``forward_intermediates``."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    dt = _dtype_code(x.dtype)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    ws = _workspace(workspace_size(ENTRY_FORWARD, T, H, I, E, k, dt), dev, workspace)
    _check(lib().moe_forward(_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w13), _ptr(w2), T, H,
                             I, E, k, dt, int(bool(renormalize)), _ptr(out), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(dev)))
    return out, ws


PROFILE_EVENTS = 6
PROFILE_STAGES = ("route", "permute", "gemm_gate_up_swiglu", "gemm_down", "combine")


def moe_forward_profiled(x, w_router, router_bias, w13, w2, k: int, renormalize: bool, out,
                         workspace, events):
    """moe_forward recording ``events`` (PROFILE_EVENTS torch.cuda.Event, timing enabled) on the
    current stream before each stage and after the last; see PROFILE_STAGES."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    dt = _dtype_code(x.dtype)
    dev = x.device
    if len(events) != PROFILE_EVENTS:
        raise ValueError(f"need {PROFILE_EVENTS} events")
    handles = (ctypes.c_void_p * PROFILE_EVENTS)(*[ev.cuda_event for ev in events])
    _check(lib().moe_forward_profiled(_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w13), _ptr(w2),
                                      T, H, I, E, k, dt, int(bool(renormalize)), _ptr(out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      handles, PROFILE_EVENTS, _stream(dev)))
    return out


def shared_layout(T: int, H: int, I: int, Is: int, E: int, k: int, dtype: int) -> SharedLayout:
    L = SharedLayout()
    _check(lib().moe_forward_shared_layout(T, H, I, Is, E, k, dtype, ctypes.byref(L)))
    return L


PROFILE_EVENTS_SHARED = 7
PROFILE_STAGES_SHARED = ("route", "permute", "gemm_gate_up_swiglu", "gemm_down",
                         "shared_expert", "combine")


def moe_forward_shared(x, w_router, router_bias, w13, w2, ws13, ws2, k: int, renormalize: bool,
                       out=None, workspace=None, events=None):
    """The MoE block with a shared expert (ws13 [2Is,H], ws2 [H,Is]) added to every token.
    Returns (out, workspace); with ``events`` (8 timing events) the stages are recorded
    as PROFILE_STAGES_SHARED."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    Is = ws13.shape[0] // 2
    dt = _dtype_code(x.dtype)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    ws = _workspace(shared_layout(T, H, I, Is, E, k, dt).total, dev, workspace)
    args = [_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w13), _ptr(w2), _ptr(ws13), _ptr(ws2),
            T, H, I, Is, E, k, dt, int(bool(renormalize)), _ptr(out), _ptr(ws),
            ws.numel() * ws.element_size()]
    if events is None:
        _check(lib().moe_forward_shared(*args, _stream(dev)))
    else:
        if len(events) != PROFILE_EVENTS_SHARED:
            raise ValueError(f"need {PROFILE_EVENTS_SHARED} events")
        handles = (ctypes.c_void_p * PROFILE_EVENTS_SHARED)(*[ev.cuda_event for ev in events])
        _check(lib().moe_forward_shared_profiled(*args, handles, PROFILE_EVENTS_SHARED, _stream(dev)))
    return out, ws


def shared_intermediates(ws: torch.Tensor, T: int, H: int, I: int, Is: int, E: int, k: int,
                         dtype: int):
    """forward_intermediates plus the shared expert's h_shared [T,Is] and y_shared [T,H]."""
    S = shared_layout(T, H, I, Is, E, k, dtype)
    eb = 2 if dtype == MOE_DTYPE_BF16 else 4
    tdt = _torch_dtype(dtype)
    mid = forward_intermediates(ws, T, H, I, E, k, dtype)
    mid["h_shared"] = ws[S.h_shared:S.h_shared + T * Is * eb].view(tdt).view(T, Is)
    mid["y_shared"] = ws[S.y_shared:S.y_shared + T * H * eb].view(tdt).view(T, H)
    return mid


def rounded_layout(T: int, H: int, I: int, E: int, k: int, dtype: int) -> ForwardLayout:
    L = ForwardLayout()
    _check(lib().moe_forward_rounded_layout(T, H, I, E, k, dtype, ctypes.byref(L)))
    return L


def gemm_tile_rows(dtype: int) -> int:
    """Rows per tile of the grouped GEMM (the token-rounding tile that removes its padding)."""
    n = lib().moe_gemm_tile_rows(dtype)
    if n <= 0:
        _check(MOE_ERR_UNSUPPORTED)
    return n


PROFILE_EVENTS_ROUNDED = 7
PROFILE_STAGES_ROUNDED = ("route", "token_round", "permute", "gemm_gate_up_swiglu",
                          "gemm_down", "combine")


def moe_forward_rounded(x, w_router, router_bias, w13, w2, k: int, renormalize: bool,
                        tile_rows: Optional[int] = None, out=None, workspace=None, events=None):
    """The MoE block with token rounding to ``tile_rows`` rows (default: the grouped
    GEMM's row tile).  Returns (out, workspace); the workspace holds the rounded
    routing at the moe_forward offsets (``forward_intermediates``).  With ``events``
    (8 timing events) the stages are recorded as PROFILE_STAGES_ROUNDED."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    dt = _dtype_code(x.dtype)
    dev = x.device
    B = gemm_tile_rows(dt) if tile_rows is None else int(tile_rows)
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    ws = _workspace(rounded_layout(T, H, I, E, k, dt).total, dev, workspace)
    args = [_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w13), _ptr(w2), T, H, I, E, k, dt,
            int(bool(renormalize)), B, _ptr(out), _ptr(ws), ws.numel() * ws.element_size()]
    if events is None:
        _check(lib().moe_forward_rounded(*args, _stream(dev)))
    else:
        if len(events) != PROFILE_EVENTS_ROUNDED:
            raise ValueError(f"need {PROFILE_EVENTS_ROUNDED} events")
        handles = (ctypes.c_void_p * PROFILE_EVENTS_ROUNDED)(*[ev.cuda_event for ev in events])
        _check(lib().moe_forward_rounded_profiled(*args, handles, PROFILE_EVENTS_ROUNDED,
                                                  _stream(dev)))
    return out, ws


def forward_intermediates(ws: torch.Tensor, T: int, H: int, I: int, E: int, k: int, dtype: int):
    """Typed views of the intermediates moe_forward leaves in its workspace."""
    L = forward_layout(T, H, I, E, k, dtype)
    M = T * k
    eb = 2 if dtype == MOE_DTYPE_BF16 else 4

    def view(off, n, dt, esz, shape):
        return ws[off:off + n * esz].view(dt).view(shape)

    tdt = _torch_dtype(dtype)
    return dict(
        ids=view(L.topk_ids, M, torch.int32, 4, (T, k)),
        weights=view(L.topk_weights, M, torch.float32, 4, (T, k)),
        counts=view(L.expert_counts, E, torch.int32, 4, (E,)),
        offsets=view(L.expert_offsets, E + 1, torch.int32, 4, (E + 1,)),
        perm=view(L.perm, M, torch.int32, 4, (M,)),
        inv_perm=view(L.inv_perm, M, torch.int32, 4, (M,)),
        h=view(L.h, M * I, tdt, eb, (M, I)),
        y=view(L.y, M * H, tdt, eb, (M, H)),
    )


def mx_quantize(src, codes=None, scales=None):
    """MXFP8 codes [..., C] and E8M0 scales [..., C/32] (uint8) of ``src`` (bf16 or
    fp32, last dimension C a multiple of 32) along its last dimension."""
    C = src.shape[-1]
    rows = src.numel() // C if C else 0
    dev = src.device
    if codes is None:
        codes = torch.empty(src.shape, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(tuple(src.shape[:-1]) + (C // 32,), dtype=torch.uint8, device=dev)
    _check(lib().moe_mx_quantize(_ptr(src), rows, C, _dtype_code(src.dtype), _ptr(codes),
                                 _ptr(scales), _stream(dev)))
    return codes, scales


def mxfp8_layout(T: int, H: int, I: int, E: int, k: int,
                 dtype: int = MOE_DTYPE_BF16) -> Mxfp8Layout:
    L = Mxfp8Layout()
    _check(lib().moe_forward_mxfp8_layout(T, H, I, E, k, dtype, ctypes.byref(L)))
    return L


PROFILE_EVENTS_MXFP8 = 7
PROFILE_STAGES_MXFP8 = ("route", "permute", "quantize_x", "gemm_gate_up_swiglu",
                        "gemm_down", "combine")


def moe_forward_mxfp8(x, w_router, router_bias, w13q, w13s, w2q, w2s, k: int,
                      renormalize: bool, out=None, workspace=None, events=None):
    """The MoE block with MXFP8 expert GEMMs (weights from ``mx_quantize``).
    Returns (out, workspace); ``mxfp8_intermediates`` reads the workspace.  With
    ``events`` (8 timing events) the stages are recorded as PROFILE_STAGES_MXFP8."""
    T, H = x.shape
    E, I2, _ = w13q.shape
    I = I2 // 2
    dt = _dtype_code(x.dtype)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    ws = _workspace(mxfp8_layout(T, H, I, E, k, dt).total, dev, workspace)
    args = [_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w13q), _ptr(w13s), _ptr(w2q),
            _ptr(w2s), T, H, I, E, k, dt, int(bool(renormalize)), _ptr(out), _ptr(ws),
            ws.numel() * ws.element_size()]
    if events is None:
        _check(lib().moe_forward_mxfp8(*args, _stream(dev)))
    else:
        if len(events) != PROFILE_EVENTS_MXFP8:
            raise ValueError(f"need {PROFILE_EVENTS_MXFP8} events")
        handles = (ctypes.c_void_p * PROFILE_EVENTS_MXFP8)(*[ev.cuda_event for ev in events])
        _check(lib().moe_forward_mxfp8_profiled(*args, handles, PROFILE_EVENTS_MXFP8,
                                                _stream(dev)))
    return out, ws


def mxfp8_intermediates(ws: torch.Tensor, T: int, H: int, I: int, E: int, k: int):
    """Typed views of the intermediates moe_forward_mxfp8 leaves in its workspace."""
    L = mxfp8_layout(T, H, I, E, k)
    M = T * k

    def view(off, n, dt, esz, shape):
        return ws[off:off + n * esz].view(dt).view(shape)

    return dict(
        ids=view(L.topk_ids, M, torch.int32, 4, (T, k)),
        weights=view(L.topk_weights, M, torch.float32, 4, (T, k)),
        counts=view(L.expert_counts, E, torch.int32, 4, (E,)),
        offsets=view(L.expert_offsets, E + 1, torch.int32, 4, (E + 1,)),
        perm=view(L.perm, M, torch.int32, 4, (M,)),
        inv_perm=view(L.inv_perm, M, torch.int32, 4, (M,)),
        x_codes=view(L.x_codes, T * H, torch.uint8, 1, (T, H)),
        x_scales=view(L.x_scales, T * H // 32, torch.uint8, 1, (T, H // 32)),
        h_codes=view(L.h_codes, M * I, torch.uint8, 1, (M, I)),
        # stage-major words [I/128, M] of 4 scale bytes -> [M, I/32]
        h_scales=view(L.h_scales, M * I // 32, torch.uint8, 1, (I // 128, M, 4))
        .permute(1, 0, 2).reshape(M, I // 32),
        y=view(L.y, M * H, torch.bfloat16, 2, (M, H)),
        x_scale_words=view(L.x_scale_words, M * H // 128, torch.int32, 4, (H // 128, M)),
    )


def backward_layout(T: int, H: int, I: int, E: int, k: int,
                    dtype: int = MOE_DTYPE_BF16) -> BackwardLayout:
    L = BackwardLayout()
    _check(lib().moe_backward_workspace_layout(T, H, I, E, k, dtype, ctypes.byref(L)))
    return L


PROFILE_EVENTS_BACKWARD = 8
PROFILE_STAGES_BACKWARD = ("router_grads", "recompute_gate_up", "dgrad_down_swiglu",
                           "dgrad_gate_up", "wgrad_transpose", "wgrad_down", "wgrad_gate_up")


def moe_forward_train(x, w_router, router_bias, w13, w2, k: int, renormalize: bool, out=None,
                      gate_up=None, workspace=None, events=None):
    """moe_forward that also keeps the gate and up sums [T*k, 2I] (bf16) for the
    caching variant of the backward.  Returns (out, gate_up, workspace); with
    ``events`` (7 timing events) the stages are recorded as PROFILE_STAGES."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    dt = _dtype_code(x.dtype)
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    if gate_up is None:
        gate_up = torch.empty((T * k, I2), dtype=x.dtype, device=dev)
    ws = _workspace(workspace_size(ENTRY_FORWARD, T, H, I, E, k, dt), dev, workspace)
    handles, n = None, 0
    if events is not None:
        if len(events) != PROFILE_EVENTS:
            raise ValueError(f"need {PROFILE_EVENTS} events")
        handles = (ctypes.c_void_p * PROFILE_EVENTS)(*[ev.cuda_event for ev in events])
        n = PROFILE_EVENTS
    _check(lib().moe_forward_train(_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w13), _ptr(w2),
                                   T, H, I, E, k, dt, int(bool(renormalize)), _ptr(out),
                                   _ptr(gate_up), _ptr(ws), ws.numel() * ws.element_size(), handles,
                                   n, _stream(dev)))
    return out, gate_up, ws


def moe_backward(x, w_router, router_bias, w13, w2, k: int, renormalize: bool, forward_ws, dout,
                 dx=None, dw_router=None, dbias=None, dw13=None, dw2=None, workspace=None,
                 events=None, want_dbias: bool = True, gate_up=None):
    """Gradients of sum(dout * out) for the moe_forward (or moe_forward_train)
    call that left ``forward_ws``; ``gate_up`` (from moe_forward_train) skips
    the recompute of g and u.  Returns (dx, dw_router, dbias, dw13, dw2,
    workspace); the weight gradients are float32.  With ``events`` (9 timing
    events) the stages are recorded as PROFILE_STAGES_BACKWARD."""
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    dt = _dtype_code(x.dtype)
    dev = x.device
    if dx is None:
        dx = torch.empty((T, H), dtype=x.dtype, device=dev)
    if dw_router is None:
        dw_router = torch.empty((E, H), dtype=torch.float32, device=dev)
    if dbias is None and want_dbias:
        dbias = torch.empty(E, dtype=torch.float32, device=dev)
    if dw13 is None:
        dw13 = torch.empty((E, I2, H), dtype=torch.float32, device=dev)
    if dw2 is None:
        dw2 = torch.empty((E, H, I), dtype=torch.float32, device=dev)
    ws = _workspace(backward_layout(T, H, I, E, k, dt).total, dev, workspace)
    args = [_ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w13), _ptr(w2), T, H, I, E, k, dt,
            int(bool(renormalize)), _ptr(forward_ws), forward_ws.numel() * forward_ws.element_size(),
            _ptr(gate_up), _ptr(dout), _ptr(dx), _ptr(dw_router), _ptr(dbias), _ptr(dw13), _ptr(dw2),
            _ptr(ws),
            ws.numel() * ws.element_size()]
    if events is None:
        _check(lib().moe_backward(*args, _stream(dev)))
    else:
        if len(events) != PROFILE_EVENTS_BACKWARD:
            raise ValueError(f"need {PROFILE_EVENTS_BACKWARD} events")
        handles = (ctypes.c_void_p * PROFILE_EVENTS_BACKWARD)(*[ev.cuda_event for ev in events])
        _check(lib().moe_backward_profiled(*args, handles, PROFILE_EVENTS_BACKWARD, _stream(dev)))
    return dx, dw_router, dbias, dw13, dw2, ws


def backward_intermediates(ws: torch.Tensor, T: int, H: int, I: int, E: int, k: int):
    """Typed views of the intermediates moe_backward leaves in its workspace."""
    L = backward_layout(T, H, I, E, k)
    M = T * k

    def view(off, n, dt, esz, shape):
        return ws[off:off + n * esz].view(dt).view(shape)

    bf = torch.bfloat16
    return dict(
        dw=view(L.dw, M, torch.float32, 4, (T, k)),
        dlogits=view(L.dlogits, T * E, torch.float32, 4, (T, E)),
        dx_router=view(L.dx_router, T * H, bf, 2, (T, H)),
        gu=view(L.gu, M * 2 * I, bf, 2, (M, 2 * I)),
        dh=view(L.dh, M * I, bf, 2, (M, I)),
        dgdu=view(L.dgdu, M * 2 * I, bf, 2, (M, 2 * I)),
        h=view(L.h, M * I, bf, 2, (M, I)),
        dx_slots=view(L.dx_slots, M * H, bf, 2, (M, H)),
        padded_offsets=view(L.padded_offsets, E + 1, torch.int32, 4, (E + 1,)),
    )
