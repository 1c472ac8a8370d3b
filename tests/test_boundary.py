"""The C ABI on the host: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments before touching a GPU.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

import combine_group_limited_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"moe_route_topk", "moe_get_layout", "moe_dispatch", "moe_combine"} <= set(names)
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n


def test_no_undefined_symbols_beyond_runtime():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (moe_[a-z0-9_]+)", out))
    assert exported == set(declared_functions())


def test_status_strings_and_version():
    L = moe.lib()
    assert L.moe_abi_version() == 8
    for s in (0, 1, 2, 4, 5):
        assert L.moe_status_string(s)


def _route(cfg_vals, logits=None, idx=None, w=None):
    L = moe.lib()
    cfg = moe.RouteCfg(*cfg_vals)
    return L.moe_route_topk(ctypes.byref(cfg), logits, idx, w, None)


@pytest.mark.parametrize("vals", [
    (-1, 256, 8, 4, 8, 0, 0, 1),      # negative T
    (4, 0, 1, 1, 1, 0, 0, 1),         # no experts
    (4, 1024, 8, 4, 8, 0, 0, 1),      # E above the limit
    (4, 256, 7, 4, 8, 0, 0, 1),       # G does not divide E
    (4, 256, 8, 9, 8, 0, 0, 1),       # g > G
    (4, 256, 8, 0, 8, 0, 0, 1),       # g = 0
    (4, 256, 8, 1, 33, 0, 0, 1),      # k > g*E/G
    (4, 256, 8, 4, 8, 33, 0, 1),      # group_topn > E/G
    (4, 256, 8, 4, 8, -1, 0, 1),      # negative group_topn
    (4, 256, 8, 4, 8, 0, 2, 1),       # unknown score fn
    (4, 256, 8, 4, 8, 0, 0, 3),       # renormalize not 0/1
    (4, 512, 128, 4, 8, 0, 0, 1),     # more than 64 groups
    (4, 256, 8, 4, 8, 0, 0, 1),       # valid shape, NULL arrays
])
def test_route_rejects(vals):
    assert _route(vals) == moe.MOE_ERR_INVALID
    assert moe.lib().moe_last_error()


def test_route_zero_tokens_is_noop():
    assert _route((0, 256, 8, 4, 8, 0, 0, 1)) == moe.MOE_OK


def test_layout_workspace_and_rejects():
    L = moe.lib()
    ok = moe.LayoutCfg(4096, 256, 8, 32, 0)
    assert L.moe_layout_workspace_bytes(ctypes.byref(ok)) >= 4 * 16 * (256 + 32 + 1)
    for vals in [(4, 256, 8, 33, 0), (4, 256, 0, 32, 0), (4, 256, 8, 32, -1), (-1, 256, 8, 32, 0),
                 (4, 600, 8, 8, 0), (4, 256, 8, 512, 0), (4, 256, 8, 32, 0, -1),
                 (4, 256, 8, 32, 4, 64), (4, 256, 8, 32, 0, 5000)]:
        cfg = moe.LayoutCfg(*vals)
        assert L.moe_layout_workspace_bytes(ctypes.byref(cfg)) == 0
        st = L.moe_get_layout(ctypes.byref(cfg), *([None] * 9), 0, None)
        assert st == moe.MOE_ERR_INVALID
    # valid shape: missing arrays, then missing workspace
    st = L.moe_get_layout(ctypes.byref(ok), *([None] * 9), 0, None)
    assert st == moe.MOE_ERR_INVALID
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    args = [fake] * 8
    st = L.moe_get_layout(ctypes.byref(ok), *args, None, 0, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = L.moe_get_layout(ctypes.byref(ok), *args, fake, 16, None)
    assert st == moe.MOE_ERR_WORKSPACE


def test_layout_noalloc_rejects_before_any_hip_call():
    """Bad configurations, missing arrays and shapes whose count table is
    larger than the library's fixed array fail on the host."""
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)
    for vals in [(4, 256, 8, 33, 0, 0), (-1, 256, 8, 32, 0, 0), (4, 256, 8, 32, 4, 64)]:
        cfg = moe.LayoutCfg(*vals)
        assert L.moe_get_layout_noalloc(ctypes.byref(cfg), *([fake] * 8), None) == moe.MOE_ERR_INVALID
    ok = moe.LayoutCfg(4096, 256, 8, 32, 0, 0)
    assert L.moe_get_layout_noalloc(ctypes.byref(ok), *([None] * 8), None) == moe.MOE_ERR_INVALID
    big = moe.LayoutCfg(231937, 256, 8, 32, 0, 0)
    assert L.moe_layout_workspace_bytes(ctypes.byref(big)) > 1 << 20
    assert L.moe_get_layout_noalloc(ctypes.byref(big), *([fake] * 8), None) == moe.MOE_ERR_WORKSPACE
    assert b"count table" in L.moe_last_error()
    fits = moe.LayoutCfg(231936, 256, 8, 32, 0, 0)
    assert L.moe_layout_workspace_bytes(ctypes.byref(fits)) <= 1 << 20


def test_check_pow2_scales_rejects():
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)
    L.moe_check_pow2_scales.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert L.moe_check_pow2_scales(fake, -1, fake, None) == moe.MOE_ERR_INVALID
    assert L.moe_check_pow2_scales(fake, 10, None, None) == moe.MOE_ERR_INVALID
    assert L.moe_check_pow2_scales(None, 10, fake, None) == moe.MOE_ERR_INVALID
    assert L.moe_check_pow2_scales(ctypes.c_void_p((1 << 20) + 2), 10, fake, None) == moe.MOE_ERR_INVALID
    assert L.moe_check_pow2_scales(None, 0, fake, None) == moe.MOE_OK


def test_dispatch_rejects():
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)
    for vals in [(4, 7168, 0, 32, 0, 0), (4, 100, 8, 32, 0, 0), (4, 7168, 8, 32, 4, 0),
                 (4, 12, 8, 32, 1, 0), (4, 7168, 8, 32, 0, 5), (-1, 7168, 8, 32, 0, 0)]:
        cfg = moe.DispatchCfg(*vals)
        assert L.moe_dispatch(ctypes.byref(cfg), fake, fake, fake, fake, None) == moe.MOE_ERR_INVALID
    cfg = moe.DispatchCfg(4, 7168, 8, 32, 0, 0)
    assert L.moe_dispatch(ctypes.byref(cfg), None, fake, fake, fake, None) == moe.MOE_ERR_INVALID
    assert L.moe_dispatch(ctypes.byref(cfg), fake, fake, fake, None, None) == moe.MOE_ERR_INVALID
    mis = ctypes.c_void_p((1 << 20) + 8)   # not 16-byte aligned
    assert L.moe_dispatch(ctypes.byref(cfg), mis, fake, fake, fake, None) == moe.MOE_ERR_INVALID
    zero = moe.DispatchCfg(0, 7168, 8, 0, 0, 0)
    assert L.moe_dispatch(ctypes.byref(zero), None, None, None, None, None) == moe.MOE_OK


def test_combine_rejects():
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)
    for vals in [(4, 7168, 0, 32, 0), (4, 7, 8, 32, 0), (4, 7168, 8, 32, 3), (4, 7168, 65, 32, 0)]:
        cfg = moe.CombineCfg(*vals)
        assert L.moe_combine(ctypes.byref(cfg), fake, fake, fake, fake, None) == moe.MOE_ERR_INVALID
    cfg = moe.CombineCfg(4, 7168, 8, 32, 0)
    assert L.moe_combine(ctypes.byref(cfg), fake, fake, None, fake, None) == moe.MOE_ERR_INVALID
    zero = moe.CombineCfg(0, 7168, 8, 0, 0)
    assert L.moe_combine(ctypes.byref(zero), None, None, None, None, None) == moe.MOE_OK


def test_quantize_rejects():
    L = moe.lib()
    assert L.moe_quantize_e4m3(None, None, -1, None) == moe.MOE_ERR_INVALID
    assert L.moe_quantize_e4m3(None, None, 0, None) == moe.MOE_OK
    assert L.moe_quantize_e4m3(None, None, 10, None) == moe.MOE_ERR_INVALID


def test_binding_has_no_fallback(tmp_path, monkeypatch):
    """Without the built library the binding raises; it never computes on the CPU."""
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(ImportError):
        moe.lib()


def _route_dispatch(rc, lc, dc, ws_bytes=256, fake=None):
    """Calls moe_route_dispatch with host-side configurations only; `fake` is
    a non-NULL dummy pointer for the arrays (never dereferenced: every case
    here fails validation before any launch)."""
    L = moe.lib()
    r, l, d = moe.RouteCfg(*rc), moe.LayoutCfg(*lc), moe.DispatchCfg(*dc)
    p = fake
    return L.moe_route_dispatch(ctypes.byref(r), ctypes.byref(l), ctypes.byref(d), p, p, p, p, p, p, p, p, p,
                                p, p, p, p, p, ws_bytes, None)


DECODE_RC = (128, 256, 8, 4, 8, 0, 0, 1)
DECODE_LC = (128, 256, 8, 32, 128, 0)
DECODE_DC = (128, 7168, 8, 256 * 128, 0, 0)


def test_route_dispatch_workspace_size():
    assert moe.lib().moe_route_dispatch_workspace_bytes() >= 12


@pytest.mark.parametrize("rc,lc,dc,status", [
    # configurations that disagree with each other
    ((128, 256, 8, 4, 8, 0, 0, 1), (64, 256, 8, 32, 128, 0), DECODE_DC, moe.MOE_ERR_INVALID),
    ((128, 256, 8, 4, 8, 0, 0, 1), (128, 128, 8, 32, 128, 0), DECODE_DC, moe.MOE_ERR_INVALID),
    ((128, 256, 8, 4, 8, 0, 0, 1), (128, 256, 4, 32, 128, 0), DECODE_DC, moe.MOE_ERR_INVALID),
    (DECODE_RC, DECODE_LC, (128, 7168, 8, 128 * 8, 0, 0), moe.MOE_ERR_INVALID),   # N of the compact layout
    (DECODE_RC, DECODE_LC, (128, 7168, 8, 256 * 128, 0, 2), moe.MOE_ERR_INVALID),  # launch-shape override
    (DECODE_RC, DECODE_LC, (128, 7000, 8, 256 * 128, 0, 0), moe.MOE_ERR_INVALID),  # H % 128 for FP8
    ((128, 256, 8, 9, 8, 0, 0, 1), DECODE_LC, DECODE_DC, moe.MOE_ERR_INVALID),     # bad routing cfg
    # valid but beyond the one-launch limits
    ((2048, 256, 8, 4, 8, 0, 0, 1), (2048, 256, 8, 32, 0, 0), (2048, 7168, 8, 2048 * 8, 0, 0),
     moe.MOE_ERR_UNSUPPORTED),
    ((1024, 512, 8, 4, 32, 0, 0, 1), (1024, 512, 32, 512, 0, 0), (1024, 7168, 32, 1024 * 32, 0, 0),
     moe.MOE_ERR_UNSUPPORTED),
    # valid shape, NULL arrays
    (DECODE_RC, DECODE_LC, DECODE_DC, moe.MOE_ERR_INVALID),
])
def test_route_dispatch_rejects(rc, lc, dc, status):
    assert _route_dispatch(rc, lc, dc) == status
    assert moe.lib().moe_last_error()


def _mlp(fn, cfg_vals, n_args):
    L = moe.lib()
    cfg = moe.MlpCfg(*cfg_vals)
    return getattr(L, fn)(ctypes.byref(cfg), *([None] * n_args))


@pytest.mark.parametrize("fn,n_args", [("moe_expert_up", 9), ("moe_expert_down", 8)])
@pytest.mark.parametrize("vals", [
    (100, 7000, 2048, 8, 0),      # hidden not a multiple of 128
    (100, 7168, 2000, 8, 0),      # inter not a multiple of 128
    (100, 7168, 2048, 0, 0),      # no experts
    (100, 7168, 2048, 513, 0),    # too many experts
    (100, 7168, 2048, 8, -1),     # negative capacity
    (-1, 7168, 2048, 8, 0),       # negative rows
    (100, 7168, 16384, 8, 0),     # inter above 8192
    (100, 7168, 2048, 8, 0),      # valid shape, NULL arrays
])
def test_expert_mlp_rejects(fn, n_args, vals):
    assert _mlp(fn, vals, n_args) == moe.MOE_ERR_INVALID
    assert moe.lib().moe_last_error()


def test_expert_up_rejects_hidden_above_8192():
    assert _mlp("moe_expert_up", (100, 16384, 2048, 8, 0), 9) == moe.MOE_ERR_INVALID


@pytest.mark.parametrize("fn,n_args", [("moe_expert_up", 9), ("moe_expert_down", 8)])
def test_expert_mlp_zero_rows_is_noop(fn, n_args):
    assert _mlp(fn, (0, 7168, 2048, 8, 0), n_args) == moe.MOE_OK


@pytest.mark.parametrize("fn,n_args,vals", [
    ("moe_expert_up", 9, (600000, 8192, 2048, 8, 0)),     # N*H above 2^32
    ("moe_expert_down", 8, (600000, 7168, 8192, 8, 0)),   # N*I above 2^32
])
def test_expert_mlp_32bit_offsets(fn, n_args, vals):
    """Row offsets inside the kernels are 32-bit: larger receive buffers are
    refused before any array is looked at."""
    assert _mlp(fn, vals, n_args) == moe.MOE_ERR_UNSUPPORTED
    assert moe.lib().moe_last_error()


def _layer(cfg_vals, T, k, ws_bytes=4096, ws=None):
    L = moe.lib()
    cfg = moe.MlpCfg(*cfg_vals)
    return L.moe_layer_forward(ctypes.byref(cfg), T, k, *([None] * 15), ws, ws_bytes, None)


def test_layer_workspace_size():
    assert moe.lib().moe_layer_workspace_bytes() == 4096


@pytest.mark.parametrize("cfg,T,k,status", [
    ((100, 7000, 2048, 8, 0), 50, 2, moe.MOE_ERR_INVALID),       # hidden not a multiple of 128
    ((100, 7168, 2048, 0, 0), 50, 2, moe.MOE_ERR_INVALID),       # no experts
    ((100, 7168, 2048, 8, 0), -1, 2, moe.MOE_ERR_INVALID),       # negative tokens
    ((100, 7168, 2048, 8, 0), 50, 0, moe.MOE_ERR_INVALID),       # topk 0
    ((100, 7168, 2048, 8, 0), 50, 65, moe.MOE_ERR_INVALID),      # topk above 64
    ((100, 16384, 2048, 8, 0), 50, 2, moe.MOE_ERR_INVALID),      # hidden above 8192
    ((600000, 8192, 2048, 8, 0), 50, 2, moe.MOE_ERR_UNSUPPORTED),  # N*H above 2^32
    ((100, 7168, 2048, 8, 0), 50, 2, moe.MOE_ERR_INVALID),       # valid shape, NULL arrays
    ((100, 7168, 2048, 8, 0), 1 << 27, 2, moe.MOE_ERR_INVALID),  # item indices beyond 32 bits
])
def test_layer_rejects(cfg, T, k, status):
    assert _layer(cfg, T, k) == status
    assert moe.lib().moe_last_error()


def test_layer_zero_tokens_or_rows_is_noop():
    assert _layer((100, 7168, 2048, 8, 0), 0, 2) == moe.MOE_OK
    assert _layer((0, 7168, 2048, 8, 0), 50, 2) == moe.MOE_OK
