"""moe_get_layout_noalloc against moe_get_layout, through the C ABI.

The no-allocation entry point keeps its count table in a static device array
of the library; every output must equal, bit for bit, what moe_get_layout
writes with a caller workspace.  Two calls in a row on the same array, the
second smaller than the first, so the second starts from the first's
leftovers; a third in the padded layout.
"""
import ctypes
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import combine_group_limited_amd as moe  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def random_idx(T, E, k, seed):
    """k distinct experts per token (a seeded permutation prefix per row)."""
    rng = np.random.default_rng(seed)
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


def buffers(T, E, k, R, C, sentinel):
    N = moe.recv_rows(T, E, k, C)
    i32 = dict(dtype=torch.int32, device=DEV)
    f = lambda *shape: torch.full(shape, sentinel, **i32)
    return moe.Layout(f(E), f(R), f(E + 1), f(R + 1), f(T, k), f(N), f(1), N)


def call_noalloc(idx, E, R, C, lay):
    T, k = idx.shape
    cfg = moe.LayoutCfg(T, E, k, R, C, 0)
    st = moe.lib().moe_get_layout_noalloc(
        ctypes.byref(cfg), idx.data_ptr(), lay.cnt_e.data_ptr(), lay.cnt_r.data_ptr(), lay.off_e.data_ptr(),
        lay.off_r.data_ptr(), lay.pos.data_ptr(), lay.recv_src.data_ptr(), lay.flags.data_ptr(),
        torch.cuda.current_stream(DEV).cuda_stream)
    assert st == moe.MOE_OK, moe.lib().moe_last_error()


def call_workspace(idx, E, R, C, lay):
    T, k = idx.shape
    cfg = moe.LayoutCfg(T, E, k, R, C, 0)
    nbytes = moe.lib().moe_layout_workspace_bytes(ctypes.byref(cfg))
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=DEV)
    st = moe.lib().moe_get_layout(
        ctypes.byref(cfg), idx.data_ptr(), lay.cnt_e.data_ptr(), lay.cnt_r.data_ptr(), lay.off_e.data_ptr(),
        lay.off_r.data_ptr(), lay.pos.data_ptr(), lay.recv_src.data_ptr(), lay.flags.data_ptr(),
        ws.data_ptr(), nbytes, torch.cuda.current_stream(DEV).cuda_stream)
    assert st == moe.MOE_OK, moe.lib().moe_last_error()
    return ws


# (T, E, k, R, capacity): the first call fills most of the count table, the
# second is smaller and starts from the first's contents, the third is padded
CALLS = [(4096, 256, 8, 32, 0), (1000, 256, 8, 32, 0), (300, 64, 6, 8, 40)]


def test_noalloc_matches_workspace_layout():
    for n, (T, E, k, R, C) in enumerate(CALLS):
        say(f"[gpu] layout_noalloc call {n}: T={T} E={E} k={k} R={R} C={C}")
        idx = torch.from_numpy(random_idx(T, E, k, 100 + n)).to(DEV)
        a = buffers(T, E, k, R, C, -77)
        b = buffers(T, E, k, R, C, -55)
        call_noalloc(idx, E, R, C, a)
        ws = call_workspace(idx, E, R, C, b)
        torch.cuda.synchronize()
        for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src", "flags"):
            ga, gb = getattr(a, name).cpu().numpy(), getattr(b, name).cpu().numpy()
            assert np.array_equal(ga, gb), (n, name)
        # every pair was placed (neither sentinel survives where a pair lives)
        assert int(a.flags.cpu()[0]) == (1 if C and int(a.cnt_e.max()) > C else 0)
        assert int(a.cnt_e.sum()) == T * k
        del ws


def test_noalloc_binding_and_reuse():
    """The binding's get_layout_noalloc on two calls in a row (large, then
    small) equals get_layout."""
    for n, (T, E, k, R) in enumerate([(2048, 256, 8, 32), (77, 256, 8, 32)]):
        say(f"[gpu] layout_noalloc binding call {n}: T={T}")
        idx = torch.from_numpy(random_idx(T, E, k, 200 + n)).to(DEV)
        got = moe.get_layout_noalloc(idx, E, R, moe.alloc_layout(T, E, k, R, 0, DEV)[0])
        ref = moe.get_layout(idx, E, R)
        torch.cuda.synchronize()
        for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src", "flags"):
            assert torch.equal(getattr(got, name), getattr(ref, name)), (n, name)


def test_noalloc_rejects_beyond_its_table():
    T, E, k, R = 300000, 256, 8, 32
    cfg = moe.LayoutCfg(T, E, k, R, 0, 0)
    fake = ctypes.c_void_p(1 << 20)
    st = moe.lib().moe_get_layout_noalloc(ctypes.byref(cfg), *([fake] * 8), None)
    assert st == moe.MOE_ERR_WORKSPACE
    assert b"count table" in moe.lib().moe_last_error()
