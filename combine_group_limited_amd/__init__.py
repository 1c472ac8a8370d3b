"""MI355X-native MoE dispatch/combine: thin Python binding of ``libcgl_moe.so``.

The four calls of the C ABI in ``include/moe.h`` -- ``route_topk``,
``get_layout``, ``dispatch``, ``combine`` -- the backward pair, the one-launch
decode path ``route_dispatch``, the expert MLP ``expert_up`` / ``expert_down``,
and ``quantize_e4m3``.  This
module only marshals arguments: it checks tensor shapes, dtypes and devices,
allocates outputs with torch (device memory and the current stream are all
torch provides here) and passes raw pointers to the library.  Every step of
the path runs in the HIP kernels; if the library is missing this module raises
instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcgl_moe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, 1, 2, 4, 5
SCORE_FNS = {"sigmoid": 0, "softmax": 1}
DISPATCH_DTYPES = {"fp8": 0, "bf16": 1, "fp8_pow2": 2, "fp8_ue8m0": 3}
FP8_DTYPES = ("fp8", "fp8_pow2", "fp8_ue8m0")
FLAG_CAPACITY_OVERFLOW, FLAG_BAD_INDEX, FLAG_INCOMPLETE, FLAG_BAD_SCALE = 1, 2, 4, 8


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class RouteCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "num_experts", "num_groups", "topk_group", "topk", "group_topn", "score_fn",
        "renormalize")]


class LayoutCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "num_experts", "topk", "num_ranks", "capacity", "align_rows")]


class DispatchCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "hidden", "topk", "num_recv_rows", "dtype", "units_per_wave")]


class MlpCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_rows", "hidden", "inter", "num_experts", "capacity")]


class CombineCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "hidden", "topk", "num_recv_rows", "units_per_wave")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m combine_group_limited_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        L.moe_route_topk.argtypes = [ctypes.POINTER(RouteCfg), P, P, P, P]
        L.moe_layout_workspace_bytes.argtypes = [ctypes.POINTER(LayoutCfg)]
        L.moe_layout_workspace_bytes.restype = S
        L.moe_get_layout.argtypes = [ctypes.POINTER(LayoutCfg)] + [P] * 9 + [S, P]
        L.moe_get_layout_noalloc.argtypes = [ctypes.POINTER(LayoutCfg)] + [P] * 9
        L.moe_dispatch.argtypes = [ctypes.POINTER(DispatchCfg), P, P, P, P, P]
        L.moe_combine.argtypes = [ctypes.POINTER(CombineCfg), P, P, P, P, P]
        L.moe_quantize_e4m3.argtypes = [P, P, ctypes.c_int64, P]
        L.moe_check_pow2_scales.argtypes = [P, ctypes.c_int64, P, P]
        L.moe_dispatch_backward.argtypes = [ctypes.POINTER(CombineCfg), P, P, P, P]
        L.moe_combine_backward.argtypes = [ctypes.POINTER(CombineCfg), P, P, P, P, P, P, P]
        L.moe_route_dispatch_workspace_bytes.argtypes = []
        L.moe_route_dispatch_workspace_bytes.restype = S
        L.moe_route_dispatch.argtypes = ([ctypes.POINTER(RouteCfg), ctypes.POINTER(LayoutCfg),
                                          ctypes.POINTER(DispatchCfg)] + [P] * 13 + [P, S, P])
        L.moe_expert_up.argtypes = [ctypes.POINTER(MlpCfg)] + [P] * 9
        L.moe_expert_down.argtypes = [ctypes.POINTER(MlpCfg)] + [P] * 8
        L.moe_layer_workspace_bytes.argtypes = []
        L.moe_layer_workspace_bytes.restype = S
        L.moe_layer_forward.argtypes = ([ctypes.POINTER(MlpCfg), ctypes.c_int, ctypes.c_int] + [P] * 16 +
                                        [S, P])
        for f in ("moe_route_topk", "moe_get_layout", "moe_get_layout_noalloc", "moe_dispatch", "moe_combine", "moe_quantize_e4m3",
                  "moe_check_pow2_scales",
                  "moe_dispatch_backward", "moe_combine_backward", "moe_route_dispatch", "moe_expert_up",
                  "moe_expert_down", "moe_layer_forward"):
            getattr(L, f).restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(status: int):
    if status != MOE_OK:
        L = lib()
        raise MoeError(status, f"{L.moe_status_string(status).decode()}: {L.moe_last_error().decode()}")


_torch_mod = None


def _torch():
    """torch, imported on first use (the module imports without it) and then kept."""
    global _torch_mod
    if _torch_mod is None:
        import torch
        _torch_mod = torch
    return _torch_mod


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


_raw_stream = None


def _stream(device) -> int:
    """The raw handle of the current stream on `device`.  torch's raw-stream
    accessor costs 0.06 us per call against 2 us for building a Stream object,
    which matters when a decode loop calls this path several times a step."""
    global _raw_stream
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    index = device.index if getattr(device, "index", None) is not None else torch.cuda.current_device()
    if _raw_stream:
        return _raw_stream(index)
    return torch.cuda.current_stream(index).cuda_stream


def _need(t, name, dtype, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and t.shape != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def route_topk(logits, num_groups: int, topk_group: int, topk: int, score_fn: str = "sigmoid",
               renormalize: bool = True, group_topn: int = 0, out=None):
    """Group-limited top-k gating.  logits fp32 [T,E] -> (idx int32 [T,k], w fp32 [T,k])."""
    torch = _torch()
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    if out is None:
        idx = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
        w = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    else:
        idx, w = out
        _need(idx, "idx", torch.int32, (T, topk), logits.device)
        _need(w, "w", torch.float32, (T, topk), logits.device)
    cfg = RouteCfg(T, E, num_groups, topk_group, topk, group_topn, SCORE_FNS[score_fn], int(renormalize))
    _check(lib().moe_route_topk(ctypes.byref(cfg), _ptr(logits), _ptr(idx), _ptr(w), _stream(logits.device)))
    return idx, w


class Layout(NamedTuple):
    cnt_e: object      # int32 [E]
    cnt_r: object      # int32 [R]
    off_e: object      # int32 [E+1]
    off_r: object      # int32 [R+1]
    pos: object        # int32 [T,k]
    recv_src: object   # int32 [N]
    flags: object      # int32 [1]
    num_recv_rows: int


def layout_workspace_bytes(num_tokens: int, num_experts: int, topk: int, num_ranks: int,
                           capacity: int = 0, align_rows: int = 0) -> int:
    cfg = LayoutCfg(num_tokens, num_experts, topk, num_ranks, capacity, align_rows)
    n = lib().moe_layout_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise MoeError(MOE_ERR_INVALID, lib().moe_last_error().decode())
    return n


def recv_rows(num_tokens, num_experts, topk, capacity=0, align_rows=0) -> int:
    """Rows of the receive buffer: E*C padded, T*k + E*(A-1) aligned, T*k packed."""
    if capacity > 0:
        return num_experts * capacity
    return num_tokens * topk + (num_experts * (align_rows - 1) if align_rows > 1 else 0)


def alloc_layout(num_tokens, num_experts, topk, num_ranks, capacity=0, device="cuda", align_rows=0):
    """Output tensors and workspace for get_layout (reusable across calls)."""
    torch = _torch()
    N = recv_rows(num_tokens, num_experts, topk, capacity, align_rows)
    i32 = dict(dtype=torch.int32, device=device)
    lay = Layout(torch.empty(num_experts, **i32), torch.empty(num_ranks, **i32),
                 torch.empty(num_experts + 1, **i32), torch.empty(num_ranks + 1, **i32),
                 torch.empty((num_tokens, topk), **i32), torch.empty(N, **i32), torch.empty(1, **i32), N)
    ws = torch.empty(layout_workspace_bytes(num_tokens, num_experts, topk, num_ranks, capacity, align_rows),
                     dtype=torch.uint8, device=device)
    return lay, ws


def get_layout(topk_idx, num_experts: int, num_ranks: int, capacity: int = 0, out=None,
               align_rows: int = 0) -> Layout:
    """Routing layout (counts, offsets, receive rows).  out = (Layout, workspace) to reuse buffers."""
    torch = _torch()
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    if out is None:
        out = alloc_layout(T, num_experts, k, num_ranks, capacity, topk_idx.device, align_rows)
    lay, ws = out
    cfg = LayoutCfg(T, num_experts, k, num_ranks, capacity, align_rows)
    _check(lib().moe_get_layout(ctypes.byref(cfg), _ptr(topk_idx), _ptr(lay.cnt_e), _ptr(lay.cnt_r),
                                _ptr(lay.off_e), _ptr(lay.off_r), _ptr(lay.pos), _ptr(lay.recv_src),
                                _ptr(lay.flags), _ptr(ws), ws.numel(), _stream(topk_idx.device)))
    return lay


def get_layout_noalloc(topk_idx, num_experts: int, num_ranks: int, layout: Layout, capacity: int = 0,
                       align_rows: int = 0) -> Layout:
    """get_layout into caller-provided buffers (alloc_layout's Layout) with no
    workspace: the library's own per-GPU count table is used, so nothing is
    allocated.  Calls that may overlap on one GPU race on that table."""
    torch = _torch()
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    dev = topk_idx.device
    N = recv_rows(T, num_experts, k, capacity, align_rows)
    for name, t, shape in (("cnt_e", layout.cnt_e, (num_experts,)), ("cnt_r", layout.cnt_r, (num_ranks,)),
                           ("off_e", layout.off_e, (num_experts + 1,)), ("off_r", layout.off_r, (num_ranks + 1,)),
                           ("pos", layout.pos, (T, k)), ("recv_src", layout.recv_src, (N,)),
                           ("flags", layout.flags, (1,))):
        _need(t, name, torch.int32, shape, dev)
    cfg = LayoutCfg(T, num_experts, k, num_ranks, capacity, align_rows)
    _check(lib().moe_get_layout_noalloc(ctypes.byref(cfg), _ptr(topk_idx), _ptr(layout.cnt_e), _ptr(layout.cnt_r),
                                        _ptr(layout.off_e), _ptr(layout.off_r), _ptr(layout.pos),
                                        _ptr(layout.recv_src), _ptr(layout.flags), _stream(dev)))
    return layout


def dispatch(x, pos, num_recv_rows: int, dtype: str = "fp8", recv_x=None, recv_scales=None,
             units_per_wave: int = 0):
    """x bf16 [T,H] -> (recv_x uint8 [N,H] or bf16 [N,H], recv_scales [N,H/128] or None):
    fp32 scales for "fp8" and "fp8_pow2", uint8 E8M0 exponent bytes for "fp8_ue8m0"."""
    torch = _torch()
    _need(x, "x", torch.bfloat16)
    _need(pos, "pos", torch.int32, device=x.device)
    T, H = x.shape
    k = pos.shape[1]
    if pos.shape[0] != T:
        raise ValueError("pos must be [T, k]")
    fp8 = dtype in FP8_DTYPES
    sdt = torch.uint8 if dtype == "fp8_ue8m0" else torch.float32
    if recv_x is None:
        recv_x = torch.empty((num_recv_rows, H), dtype=torch.uint8 if fp8 else torch.bfloat16,
                             device=x.device)
    else:
        _need(recv_x, "recv_x", torch.uint8 if fp8 else torch.bfloat16, (num_recv_rows, H), x.device)
    if fp8 and recv_scales is None:
        recv_scales = torch.empty((num_recv_rows, H // 128), dtype=sdt, device=x.device)
    elif fp8:
        _need(recv_scales, "recv_scales", sdt, (num_recv_rows, H // 128), x.device)
    cfg = DispatchCfg(T, H, k, num_recv_rows, DISPATCH_DTYPES[dtype], units_per_wave)
    _check(lib().moe_dispatch(ctypes.byref(cfg), _ptr(x), _ptr(pos), _ptr(recv_x),
                              _ptr(recv_scales) if fp8 else None, _stream(x.device)))
    return recv_x, (recv_scales if fp8 else None)


_route_dispatch_ws = {}


def route_dispatch_workspace(device):
    """A zeroed barrier workspace for route_dispatch (one per device is cached
    and used by default; calls that may overlap on different streams need
    their own)."""
    torch = _torch()
    n = lib().moe_route_dispatch_workspace_bytes()
    return torch.zeros(n, dtype=torch.uint8, device=device)


def route_dispatch(logits, x, num_groups: int, topk_group: int, topk: int, num_ranks: int,
                   capacity: int = 0, dtype: str = "fp8", score_fn: str = "sigmoid",
                   renormalize: bool = True, group_topn: int = 0, align_rows: int = 0,
                   out=None, workspace=None):
    """Route + layout + dispatch in one launch (small batches, T <= 1024).

    logits fp32 [T,E], x bf16 [T,H] -> (idx, w, Layout, recv_x, recv_scales), the
    same tensors route_topk, get_layout and dispatch return.  out = (idx, w,
    Layout, recv_x, recv_scales) reuses buffers."""
    torch = _torch()
    _need(logits, "logits", torch.float32)
    _need(x, "x", torch.bfloat16, device=logits.device)
    T, E = logits.shape
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x must be [T, H] with the T of logits")
    dev = logits.device
    N = recv_rows(T, E, topk, capacity, align_rows)
    fp8 = dtype in FP8_DTYPES
    sdt = torch.uint8 if dtype == "fp8_ue8m0" else torch.float32
    if out is None:
        idx = torch.empty((T, topk), dtype=torch.int32, device=dev)
        w = torch.empty((T, topk), dtype=torch.float32, device=dev)
        lay = alloc_layout(T, E, topk, num_ranks, capacity, dev, align_rows)[0]
        recv_x = torch.empty((N, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        recv_scales = torch.empty((N, H // 128), dtype=sdt, device=dev) if fp8 else None
    else:
        idx, w, lay, recv_x, recv_scales = out
        _need(idx, "idx", torch.int32, (T, topk), dev)
        _need(w, "w", torch.float32, (T, topk), dev)
        _need(recv_x, "recv_x", torch.uint8 if fp8 else torch.bfloat16, (N, H), dev)
        if fp8:
            _need(recv_scales, "recv_scales", sdt, (N, H // 128), dev)
        if lay.num_recv_rows != N:
            raise ValueError("layout buffers were sized for another receive layout")
    if workspace is None:
        key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
        if key not in _route_dispatch_ws:
            _route_dispatch_ws[key] = route_dispatch_workspace(dev)
        workspace = _route_dispatch_ws[key]
    rc = RouteCfg(T, E, num_groups, topk_group, topk, group_topn, SCORE_FNS[score_fn], int(renormalize))
    lc = LayoutCfg(T, E, topk, num_ranks, capacity, align_rows)
    dc = DispatchCfg(T, H, topk, N, DISPATCH_DTYPES[dtype], 0)
    _check(lib().moe_route_dispatch(
        ctypes.byref(rc), ctypes.byref(lc), ctypes.byref(dc), _ptr(logits), _ptr(x), _ptr(idx), _ptr(w),
        _ptr(lay.cnt_e), _ptr(lay.cnt_r), _ptr(lay.off_e), _ptr(lay.off_r), _ptr(lay.pos), _ptr(lay.recv_src),
        _ptr(lay.flags), _ptr(recv_x), _ptr(recv_scales) if fp8 else None, _ptr(workspace), workspace.numel(),
        _stream(dev)))
    return idx, w, lay, recv_x, (recv_scales if fp8 else None)


def expert_up(x, x_scales, w1, w1_scales, cnt_e, off_e, capacity: int = 0, act=None, act_scales=None):
    """First expert layer + SwiGLU + FP8 requantisation.  x uint8 [N,H] with
    power-of-two scales fp32 [N,H/128]; w1 uint8 [E,2I,H], w1_scales fp32
    [E,2I/128,H/128]; cnt_e/off_e from get_layout -> (act uint8 [N,I],
    act_scales fp32 [N,I/128])."""
    torch = _torch()
    _need(x, "x", torch.uint8)
    dev = x.device
    N, H = x.shape
    E, I2, H2 = w1.shape
    I = I2 // 2
    if H2 != H:
        raise ValueError("w1 must be [E, 2I, H]")
    _need(x_scales, "x_scales", torch.float32, (N, H // 128), dev)
    _need(w1, "w1", torch.uint8, device=dev)
    _need(w1_scales, "w1_scales", torch.float32, (E, I2 // 128, H // 128), dev)
    _need(cnt_e, "cnt_e", torch.int32, (E,), dev)
    if capacity == 0:
        _need(off_e, "off_e", torch.int32, (E + 1,), dev)
    if act is None:
        act = torch.empty((N, I), dtype=torch.uint8, device=dev)
        act_scales = torch.empty((N, I // 128), dtype=torch.float32, device=dev)
    else:
        _need(act, "act", torch.uint8, (N, I), dev)
        _need(act_scales, "act_scales", torch.float32, (N, I // 128), dev)
    cfg = MlpCfg(N, H, I, E, capacity)
    _check(lib().moe_expert_up(ctypes.byref(cfg), _ptr(cnt_e), _ptr(off_e), _ptr(x), _ptr(x_scales), _ptr(w1),
                               _ptr(w1_scales), _ptr(act), _ptr(act_scales), _stream(dev)))
    return act, act_scales


def expert_down(act, act_scales, w2, w2_scales, cnt_e, off_e, capacity: int = 0, y=None):
    """Second expert layer: act uint8 [N,I] (power-of-two scales [N,I/128]),
    w2 uint8 [E,H,I], w2_scales [E,H/128,I/128] -> y bf16 [N,H]."""
    torch = _torch()
    _need(act, "act", torch.uint8)
    dev = act.device
    N, I = act.shape
    E, H, I2 = w2.shape
    if I2 != I:
        raise ValueError("w2 must be [E, H, I]")
    _need(act_scales, "act_scales", torch.float32, (N, I // 128), dev)
    _need(w2, "w2", torch.uint8, device=dev)
    _need(w2_scales, "w2_scales", torch.float32, (E, H // 128, I // 128), dev)
    _need(cnt_e, "cnt_e", torch.int32, (E,), dev)
    if capacity == 0:
        _need(off_e, "off_e", torch.int32, (E + 1,), dev)
    if y is None:
        y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(y, "y", torch.bfloat16, (N, H), dev)
    cfg = MlpCfg(N, H, I, E, capacity)
    _check(lib().moe_expert_down(ctypes.byref(cfg), _ptr(cnt_e), _ptr(off_e), _ptr(act), _ptr(act_scales),
                                 _ptr(w2), _ptr(w2_scales), _ptr(y), _stream(dev)))
    return y


def layer_workspace(device):
    """A zeroed barrier workspace for layer_forward (calls that may overlap on
    different streams need their own)."""
    torch = _torch()
    return torch.zeros(lib().moe_layer_workspace_bytes(), dtype=torch.uint8, device=device)


def layer_forward(x, pos, topk_w, cnt_e, off_e, w1, w1_scales, w2, w2_scales, num_recv_rows: int,
                  capacity: int = 0, workspace=None, out=None, buffers=None):
    """The MoE layer after routing in one launch: FP8 (power-of-two) dispatch
    of x bf16 [T,H] by pos int32 [T,k] -> expert up (w1 uint8 [E,2I,H]) ->
    expert down (w2 uint8 [E,H,I]) -> combine with topk_w fp32 [T,k] ->
    out bf16 [T,H].  cnt_e/off_e from get_layout.  buffers: optional
    (recv_x, recv_scales, act, act_scales, y) to write the intermediates
    into; returns (out, buffers).  workspace: the barrier workspace; by
    default one zeroed workspace per device is cached and shared, so calls
    that may run at the same time on different streams must each pass their
    own (layer_workspace)."""
    torch = _torch()
    _need(x, "x", torch.bfloat16)
    dev = x.device
    T, H = x.shape
    _need(pos, "pos", torch.int32, device=dev)
    k = pos.shape[1] if pos.dim() == 2 else 0
    _need(pos, "pos", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    E, I2, H2 = w1.shape
    I = I2 // 2
    if H2 != H:
        raise ValueError("w1 must be [E, 2I, H]")
    N = num_recv_rows
    _need(w1, "w1", torch.uint8, device=dev)
    _need(w1_scales, "w1_scales", torch.float32, (E, I2 // 128, H // 128), dev)
    _need(w2, "w2", torch.uint8, (E, H, I), dev)
    _need(w2_scales, "w2_scales", torch.float32, (E, H // 128, I // 128), dev)
    _need(cnt_e, "cnt_e", torch.int32, (E,), dev)
    if capacity == 0:
        _need(off_e, "off_e", torch.int32, (E + 1,), dev)
    if buffers is None:
        buffers = (torch.empty((N, H), dtype=torch.uint8, device=dev),
                   torch.empty((N, H // 128), dtype=torch.float32, device=dev),
                   torch.empty((N, I), dtype=torch.uint8, device=dev),
                   torch.empty((N, I // 128), dtype=torch.float32, device=dev),
                   torch.empty((N, H), dtype=torch.bfloat16, device=dev))
    rx, rs, act, act_s, y = buffers
    _need(rx, "recv_x", torch.uint8, (N, H), dev)
    _need(rs, "recv_scales", torch.float32, (N, H // 128), dev)
    _need(act, "act", torch.uint8, (N, I), dev)
    _need(act_s, "act_scales", torch.float32, (N, I // 128), dev)
    _need(y, "y", torch.bfloat16, (N, H), dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, (T, H), dev)
    if workspace is None:
        key = (dev.type, dev.index)
        if key not in _layer_ws:
            _layer_ws[key] = layer_workspace(dev)
        workspace = _layer_ws[key]
    cfg = MlpCfg(N, H, I, E, capacity)
    _check(lib().moe_layer_forward(ctypes.byref(cfg), T, k, _ptr(pos), _ptr(topk_w), _ptr(cnt_e), _ptr(off_e),
                                   _ptr(x), _ptr(w1), _ptr(w1_scales), _ptr(w2), _ptr(w2_scales), _ptr(rx),
                                   _ptr(rs), _ptr(act), _ptr(act_s), _ptr(y), _ptr(out), _ptr(workspace),
                                   workspace.numel(), _stream(dev)))
    return out, buffers


_layer_ws = {}


def barrier_gave_up(workspace) -> int:
    """Word 2 of a route_dispatch or layer_forward barrier workspace (waits for
    the device): the number of blocks that stopped waiting at a barrier.
    Nonzero means the outputs of the call that raised it, and of every later
    call on that workspace, are incomplete until reset_barrier_workspace()."""
    return int(workspace.view(_torch().int32)[2].item())


def reset_barrier_workspace(workspace):
    """Zero a barrier workspace (on the current stream) so that it can be used
    again after a give-up."""
    workspace.zero_()
    return workspace


def combine(y, pos, topk_w, out=None, units_per_wave: int = 0):
    """y bf16 [N,H], pos int32 [T,k], topk_w fp32 [T,k] -> out bf16 [T,H]."""
    torch = _torch()
    _need(y, "y", torch.bfloat16)
    _need(pos, "pos", torch.int32, device=y.device)
    T, k = pos.shape
    _need(topk_w, "topk_w", torch.float32, (T, k), y.device)
    N, H = y.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    else:
        _need(out, "out", torch.bfloat16, (T, H), y.device)
    cfg = CombineCfg(T, H, k, N, units_per_wave)
    _check(lib().moe_combine(ctypes.byref(cfg), _ptr(y), _ptr(pos), _ptr(topk_w), _ptr(out),
                             _stream(y.device)))
    return out


def dispatch_backward(grad_recv, pos, out=None, units_per_wave: int = 0):
    """Backward of dispatch: grad_recv bf16 [N,H], pos int32 [T,k] -> grad_x bf16 [T,H]."""
    torch = _torch()
    _need(grad_recv, "grad_recv", torch.bfloat16)
    _need(pos, "pos", torch.int32, device=grad_recv.device)
    T, k = pos.shape
    N, H = grad_recv.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=grad_recv.device)
    else:
        _need(out, "out", torch.bfloat16, (T, H), grad_recv.device)
    cfg = CombineCfg(T, H, k, N, units_per_wave)
    _check(lib().moe_dispatch_backward(ctypes.byref(cfg), _ptr(grad_recv), _ptr(pos), _ptr(out),
                                       _stream(grad_recv.device)))
    return out


def combine_backward(grad_out, y, pos, topk_w, grad_y=None, grad_w=None, units_per_wave: int = 0):
    """Backward of combine -> (grad_y bf16 [N,H], grad_w fp32 [T,k])."""
    torch = _torch()
    _need(grad_out, "grad_out", torch.bfloat16)
    dev = grad_out.device
    _need(y, "y", torch.bfloat16, device=dev)
    _need(pos, "pos", torch.int32, device=dev)
    T, k = pos.shape
    N, H = y.shape
    _need(grad_out, "grad_out", torch.bfloat16, (T, H), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    if grad_y is None:
        grad_y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(grad_y, "grad_y", torch.bfloat16, (N, H), dev)
    if grad_w is None:
        grad_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    else:
        _need(grad_w, "grad_w", torch.float32, (T, k), dev)
    cfg = CombineCfg(T, H, k, N, units_per_wave)
    _check(lib().moe_combine_backward(ctypes.byref(cfg), _ptr(grad_out), _ptr(y), _ptr(pos), _ptr(topk_w),
                                      _ptr(grad_y), _ptr(grad_w), _stream(dev)))
    return grad_y, grad_w


def check_pow2_scales(*scales) -> bool:
    """True if every element of the given fp32 GPU tensors is a positive normal
    power of two, the precondition of expert_up, expert_down and layer_forward
    on their block scales (waits for the device)."""
    torch = _torch()
    if not scales:
        return True
    dev = scales[0].device
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for i, t in enumerate(scales):
        _need(t, f"scales[{i}]", torch.float32, device=dev)
        _check(lib().moe_check_pow2_scales(_ptr(t), t.numel(), _ptr(status), _stream(dev)))
    return int(status.item()) & FLAG_BAD_SCALE == 0


def quantize_e4m3(x, out=None):
    """fp32 tensor -> uint8 E4M3FN codes of the same shape."""
    torch = _torch()
    _need(x, "x", torch.float32)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    else:
        _need(out, "out", torch.uint8, x.shape, x.device)
    _check(lib().moe_quantize_e4m3(_ptr(x), _ptr(out), x.numel(), _stream(x.device)))
    return out


__all__ = ["lib", "MoeError", "Layout", "route_topk", "get_layout", "get_layout_noalloc", "alloc_layout",
           "layout_workspace_bytes", "recv_rows", "dispatch", "combine", "dispatch_backward", "combine_backward",
           "route_dispatch", "route_dispatch_workspace", "expert_up", "expert_down", "layer_forward",
           "layer_workspace", "barrier_gave_up", "reset_barrier_workspace", "check_pow2_scales", "quantize_e4m3",
           "FLAG_CAPACITY_OVERFLOW", "FLAG_BAD_INDEX", "FLAG_INCOMPLETE", "FLAG_BAD_SCALE"]
