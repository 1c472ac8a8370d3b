"""CPU oracle for MoE dispatch/combine (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
single-threaded) with ctypes over NumPy arrays and shares nothing with the HIP
library in ``combine_group_limited_amd``.

Which passage each function follows is stated in ``moe_oracle.c``:
route -- Perplexity "Efficient and Portable Mixture-of-Experts Communication",
section "Introduction", and the GeekNews DeepEP digest (group-limited gating);
layout/dispatch -- same Perplexity page, sections "Portable kernels" and
"Dispatch"; combine -- section "Combine"; the expert MLP -- the Mega MoE news
page and the TileKernels news page, "functions".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The compiled oracle.  CGL_ORACLE_LIB names another build of the same
    source to load instead (the mutation test points it at deliberately
    broken copies to show that the pins catch them)."""
    global _lib
    if _lib is None:
        path = os.environ.get("CGL_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.orc_exp_r.restype = ctypes.c_float
        L.orc_exp_r.argtypes = [ctypes.c_float]
        L.orc_sigmoid.restype = ctypes.c_float
        L.orc_sigmoid.argtypes = [ctypes.c_float]
        for name in ("orc_exp_r_array", "orc_sigmoid_array", "orc_e4m3_from_f32_array",
                     "orc_bf16_from_f64_array"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [P, P, i64]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_route.restype = i32
        L.orc_route.argtypes = [i32] * 8 + [P, P, P]
        L.orc_layout.restype = i32
        L.orc_layout.argtypes = [i32] * 6 + [P] * 8
        L.orc_dispatch.restype = i32
        L.orc_dispatch.argtypes = [i32] * 5 + [P] * 4
        L.orc_combine.restype = i32
        L.orc_combine.argtypes = [i32] * 4 + [P] * 4
        L.orc_dispatch_backward.restype = i32
        L.orc_dispatch_backward.argtypes = [i32] * 4 + [P] * 3
        L.orc_combine_backward.restype = i32
        L.orc_combine_backward.argtypes = [i32] * 4 + [P] * 6
        for name in ("orc_mlp_up", "orc_mlp_down"):
            getattr(L, name).restype = i32
        L.orc_mlp_up.argtypes = [i32] * 4 + [P, P, i32] + [P] * 8
        L.orc_mlp_down.argtypes = [i32] * 4 + [P, P, i32] + [P] * 6
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def exp_r(z) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32)
    out = np.empty_like(z)
    lib().orc_exp_r_array(_p(z), _p(out), z.size)
    return out


def sigmoid(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().orc_sigmoid_array(_p(x), _p(out), x.size)
    return out


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_from_f32(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().orc_e4m3_from_f32_array(_p(y), _p(out), y.size)
    return out


def bf16_from_f64(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_bf16_from_f64_array(_p(v), _p(out), v.size)
    return out


SIGMOID, SOFTMAX = 0, 1


def route(logits: np.ndarray, num_groups: int, topk_group: int, topk: int,
          score_fn: int = SIGMOID, renormalize: bool = True, group_topn: int = 0):
    """Returns (idx int32 [T,k], w float32 [T,k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, topk), dtype=np.int32)
    w = np.empty((T, topk), dtype=np.float32)
    rc = lib().orc_route(T, E, num_groups, topk_group, topk, group_topn, score_fn,
                         int(renormalize), _p(logits), _p(idx), _p(w))
    if rc != 0:
        raise ValueError("oracle route: invalid arguments")
    return idx, w


def layout(idx: np.ndarray, num_experts: int, num_ranks: int, capacity: int = 0, align: int = 0):
    """Returns a dict with cnt_e, cnt_r, off_e, off_r, pos, recv_src, flags."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    E, R = num_experts, num_ranks
    N = E * capacity if capacity > 0 else T * k + (E * (align - 1) if align > 1 else 0)
    out = dict(
        cnt_e=np.zeros(E, np.int32), cnt_r=np.zeros(R, np.int32),
        off_e=np.zeros(E + 1, np.int32), off_r=np.zeros(R + 1, np.int32),
        pos=np.zeros((T, k), np.int32), recv_src=np.zeros(N, np.int32),
        flags=np.zeros(1, np.int32),
    )
    rc = lib().orc_layout(T, E, k, R, capacity, align, _p(idx), _p(out["cnt_e"]), _p(out["cnt_r"]),
                          _p(out["off_e"]), _p(out["off_r"]), _p(out["pos"]),
                          _p(out["recv_src"]), _p(out["flags"]))
    if rc != 0:
        raise ValueError("oracle layout: invalid arguments")
    out["flags"] = int(out["flags"][0])
    return out


FP8, BF16, FP8_POW2, FP8_UE8M0 = 0, 1, 2, 3


def dispatch(x_bits: np.ndarray, pos: np.ndarray, num_recv_rows: int, dtype: int = FP8,
             recv_x: np.ndarray | None = None, recv_scales: np.ndarray | None = None):
    """x_bits: uint16 [T,H] bf16 patterns.  Returns (recv_x, recv_scales).

    recv_x is uint8 [N,H] (FP8 codes) or uint16 [N,H] (BF16); recv_scales is
    float32 [N,H/128], or uint8 [N,H/128] E8M0 bytes for FP8_UE8M0; rows that
    no pair addresses keep the contents of the arrays passed in (zeros by
    default)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    T, H = x_bits.shape
    k = pos.shape[1]
    N = num_recv_rows
    if recv_x is None:
        recv_x = np.zeros((N, H), dtype=np.uint16 if dtype == BF16 else np.uint8)
    sdt = np.uint8 if dtype == FP8_UE8M0 else np.float32
    if dtype != BF16 and recv_scales is None:
        recv_scales = np.zeros((N, H // 128), dtype=sdt)
    if recv_scales is not None:
        assert recv_scales.dtype == sdt and recv_scales.shape == (N, H // 128)
    sc = _p(recv_scales) if recv_scales is not None else None
    rc = lib().orc_dispatch(T, H, k, N, dtype, _p(x_bits), _p(pos), _p(recv_x), sc)
    if rc != 0:
        raise ValueError("oracle dispatch: invalid arguments")
    return recv_x, recv_scales


def combine(y_bits: np.ndarray, pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y_bits: uint16 [N,H] bf16 patterns.  Returns uint16 [T,H] bf16 patterns."""
    y_bits = np.ascontiguousarray(y_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, H = y_bits.shape
    T, k = pos.shape
    out = np.empty((T, H), dtype=np.uint16)
    rc = lib().orc_combine(T, H, k, N, _p(y_bits), _p(pos), _p(w), _p(out))
    if rc != 0:
        raise ValueError("oracle combine: invalid arguments")
    return out


def dispatch_backward(grad_recv_bits: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """grad_recv uint16 [N,H] bf16 patterns -> grad_x uint16 [T,H]."""
    g = np.ascontiguousarray(grad_recv_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    N, H = g.shape
    T, k = pos.shape
    out = np.empty((T, H), dtype=np.uint16)
    if lib().orc_dispatch_backward(T, H, k, N, _p(g), _p(pos), _p(out)) != 0:
        raise ValueError("oracle dispatch_backward: invalid arguments")
    return out


def combine_backward(grad_out_bits: np.ndarray, y_bits: np.ndarray, pos: np.ndarray, w: np.ndarray,
                     grad_y: np.ndarray | None = None):
    """Returns (grad_y uint16 [N,H], grad_w float32 [T,k]); unaddressed rows of
    grad_y keep the array passed in (zeros by default)."""
    g = np.ascontiguousarray(grad_out_bits, dtype=np.uint16)
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, H = y.shape
    T, k = pos.shape
    if grad_y is None:
        grad_y = np.zeros((N, H), dtype=np.uint16)
    grad_w = np.empty((T, k), dtype=np.float32)
    if lib().orc_combine_backward(T, H, k, N, _p(g), _p(y), _p(pos), _p(w), _p(grad_y), _p(grad_w)) != 0:
        raise ValueError("oracle combine_backward: invalid arguments")
    return grad_y, grad_w


def _ranges(start, count):
    return (np.ascontiguousarray(start, dtype=np.int32), np.ascontiguousarray(count, dtype=np.int32))


def mlp_up(x, xs, w1, w1s, start, count, rows=None, act=None, act_s=None, want_f64=False, act_f64=None):
    """Expert up projection + SwiGLU + FP8 (power-of-two scale) quantisation.

    x uint8 [N,H], xs f32 [N,H/128], w1 uint8 [E,2I,H], w1s f32 [E,2I/128,H/128];
    start/count int32 [E].  Returns (act uint8 [N,I], act_s f32 [N,I/128],
    act_f64 [N,I] or None): the unrounded SwiGLU output, when want_f64 or an
    act_f64 array is given; rows not computed keep the arrays passed in."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    w1 = np.ascontiguousarray(w1, dtype=np.uint8)
    w1s = np.ascontiguousarray(w1s, dtype=np.float32)
    N, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    st, ct = _ranges(start, count)
    act = np.zeros((N, I), np.uint8) if act is None else act
    act_s = np.zeros((N, I // 128), np.float32) if act_s is None else act_s
    f64 = act_f64 if act_f64 is not None else (np.full((N, I), np.nan) if want_f64 else None)
    if f64 is not None:
        assert f64.shape == (N, I) and f64.dtype == np.float64 and f64.flags["C_CONTIGUOUS"]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    rc = lib().orc_mlp_up(N, H, I, E, _p(st), _p(ct), 0 if r is None else r.size,
                          None if r is None else _p(r), _p(x), _p(xs), _p(w1), _p(w1s), _p(act),
                          _p(act_s), None if f64 is None else _p(f64))
    if rc != 0:
        raise ValueError("oracle mlp_up: invalid arguments")
    return act, act_s, f64


def mlp_down(act, act_s, w2, w2s, start, count, rows=None, y=None):
    """Expert down projection: y bf16 bits [N,H] = bf16(act @ w2[e]^T) per row."""
    act = np.ascontiguousarray(act, dtype=np.uint8)
    act_s = np.ascontiguousarray(act_s, dtype=np.float32)
    w2 = np.ascontiguousarray(w2, dtype=np.uint8)
    w2s = np.ascontiguousarray(w2s, dtype=np.float32)
    N, I = act.shape
    E, H, _ = w2.shape
    st, ct = _ranges(start, count)
    y = np.zeros((N, H), np.uint16) if y is None else y
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    rc = lib().orc_mlp_down(N, H, I, E, _p(st), _p(ct), 0 if r is None else r.size,
                            None if r is None else _p(r), _p(act), _p(act_s), _p(w2), _p(w2s), _p(y))
    if rc != 0:
        raise ValueError("oracle mlp_down: invalid arguments")
    return y
