"""GPU parity of the one-launch decode path (moe_route_dispatch) through the
C ABI: every output -- indices, weights, counts, offsets, receive rows,
recv_src, flags, FP8 codes and scales or BF16 copies -- bit-identical to the
oracle's route -> layout -> dispatch, for decode-sized batches, ragged shapes,
every routing path (grouped, general groups, no groups, softmax), padded,
compact and aligned layouts, all three dispatch dtypes, and repeated calls
on one barrier workspace; a workspace marked as given up (set from the
host, so no block ever waits) is refused and reported in flags."""
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import combine_group_limited_amd as moe  # noqa: E402
import oracle  # noqa: E402

DEV = torch.device("cuda:0")
FILL8, FILL16, FILLS = 0xAB, -21555, -7.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_from_dev(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sf(wl):
    return oracle.SOFTMAX if wl.score == "softmax" else oracle.SIGMOID


ODT = {"fp8": oracle.FP8, "bf16": oracle.BF16, "fp8_pow2": oracle.FP8_POW2, "fp8_ue8m0": oracle.FP8_UE8M0}


def reference(wl, logits, x, align=0, dtype=None):
    """The oracle's route -> layout -> dispatch into prefilled receive buffers."""
    dtype = dtype or wl.dtype
    idx, w = oracle.route(logits, wl.G, wl.g, wl.k, score_fn=sf(wl))
    lay = oracle.layout(idx, wl.E, wl.R, wl.capacity, align)
    N = moe.recv_rows(wl.T, wl.E, wl.k, wl.capacity, align)
    fp8 = dtype != "bf16"
    rx = np.full((N, wl.H), FILL8 if fp8 else np.uint16(FILL16 & 0xFFFF), np.uint8 if fp8 else np.uint16)
    if dtype == "fp8_ue8m0":
        rs = np.full((N, wl.S), 0xEE, np.uint8)
    else:
        rs = np.full((N, wl.S), FILLS, np.float32) if fp8 else None
    rx, rs = oracle.dispatch(x, lay["pos"], N, ODT[dtype], rx, rs)
    return idx, w, lay, rx, rs, N


def prefilled_out(wl, N, dtype, align=0):
    fp8 = dtype != "bf16"
    idx = torch.full((wl.T, wl.k), -5, dtype=torch.int32, device=DEV)
    w = torch.full((wl.T, wl.k), -5.0, dtype=torch.float32, device=DEV)
    lay = moe.alloc_layout(wl.T, wl.E, wl.k, wl.R, wl.capacity, DEV, align)[0]
    for t in lay[:7]:
        t.fill_(-9)
    rx = torch.full((N, wl.H), FILL8 if fp8 else FILL16, dtype=torch.uint8 if fp8 else torch.int16, device=DEV)
    if not fp8:
        rx = rx.view(torch.bfloat16)
    if dtype == "fp8_ue8m0":
        rs = torch.full((N, wl.S), 0xEE, dtype=torch.uint8, device=DEV)
    else:
        rs = torch.full((N, wl.S), FILLS, dtype=torch.float32, device=DEV) if fp8 else None
    return idx, w, lay, rx, rs


def check(wl, got, ref, dtype):
    idx, w, lay, rx, rs = got
    ridx, rw, rlay, rrx, rrs, N = ref
    assert np.array_equal(idx.cpu().numpy(), ridx), "idx"
    assert np.array_equal(w.cpu().numpy().view(np.uint32), rw.view(np.uint32)), "w"
    for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, name).cpu().numpy(), rlay[name]), name
    assert int(lay.flags.item()) == rlay["flags"], "flags"
    if dtype == "bf16":
        assert np.array_equal(bf16_from_dev(rx), rrx), "recv_x"
    else:
        assert np.array_equal(rx.cpu().numpy(), rrx), "recv_x"
        assert np.array_equal(rs.cpu().numpy().view(np.uint8), rrs.view(np.uint8)), "recv_scales"


def run_case(wl, align=0, dtype=None, logits=None, x=None, ws=None):
    dtype = dtype or wl.dtype
    logits = W.gen_logits(wl) if logits is None else logits
    x = W.gen_x(wl) if x is None else x
    ref = reference(wl, logits, x, align, dtype)
    out = prefilled_out(wl, ref[5], dtype, align)
    ws = moe.route_dispatch_workspace(DEV) if ws is None else ws
    got = moe.route_dispatch(torch.from_numpy(logits).to(DEV), bf16_to_dev(x), wl.G, wl.g, wl.k, wl.R,
                             wl.capacity, dtype, wl.score, align_rows=align, out=out, workspace=ws)
    torch.cuda.synchronize()
    words = ws.view(torch.int32).cpu().numpy()
    assert words[0] == 0 and words[2] == 0, f"barrier workspace words {words[:3]}"
    check(wl, got, ref, dtype)
    return got, ref


CASES = [
    W.get("ll_decode"),
    W.get("tiny"),
    W.get("dsv3_prefill").replace(T=256),
    W.get("dsv3_prefill").replace(T=768),
    W.get("dsv3_prefill").replace(T=1),
    W.get("mixtral").replace(T=300),
    W.custom("ragged_b", T=301, H=1152, E=96, G=4, g=2, k=6, score="sigmoid", R=8, dtype="fp8"),
    W.custom("ragged_f", T=65, H=7168, E=256, G=8, g=4, k=8, score="sigmoid", R=32, dtype="fp8", capacity=3),
    W.custom("ragged_g", T=200, H=512, E=512, G=16, g=3, k=12, score="sigmoid", R=64, dtype="fp8"),
    W.custom("ragged_h", T=130, H=1024, E=128, G=8, g=2, k=4, score="softmax", R=4, dtype="fp8", capacity=40),
    W.custom("ragged_e", T=257, H=2048, E=64, G=64, g=8, k=8, score="sigmoid", R=16, dtype="fp8"),
    W.custom("ragged_bf16", T=97, H=264, E=8, G=1, g=1, k=2, score="softmax", R=2, dtype="bf16", capacity=30),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: f"{w.name}_T{w.T}")
def test_route_dispatch_parity(wl):
    say(f"[gpu] route_dispatch {W.describe(wl)}")
    run_case(wl)


@pytest.mark.parametrize("dtype", ["fp8_pow2", "fp8_ue8m0", "bf16"])
def test_route_dispatch_dtypes(dtype):
    wl = W.get("ll_decode")
    say(f"[gpu] route_dispatch ll_decode {dtype}")
    run_case(wl, dtype=dtype)


@pytest.mark.parametrize("T,A", [(200, 8), (128, 128), (64, 4)])
def test_route_dispatch_aligned(T, A):
    wl = W.get("dsv3_prefill").replace(T=T)
    say(f"[gpu] route_dispatch aligned T={T} A={A}")
    run_case(wl, align=A)


def test_route_dispatch_zero_tokens():
    wl = W.get("ll_decode").replace(T=0)
    say("[gpu] route_dispatch T=0")
    ws = moe.route_dispatch_workspace(DEV)
    out = prefilled_out(wl, wl.E * wl.capacity, "fp8")
    _, _, lay, _, _ = moe.route_dispatch(torch.zeros((0, wl.E), dtype=torch.float32, device=DEV),
                                         torch.zeros((0, wl.H), dtype=torch.bfloat16, device=DEV), wl.G, wl.g,
                                         wl.k, wl.R, wl.capacity, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert (lay.cnt_e == 0).all() and (lay.cnt_r == 0).all() and (lay.off_e == 0).all()
    assert (lay.off_r == 0).all() and (lay.recv_src == -1).all() and int(lay.flags.item()) == 0


def test_route_dispatch_repeated_calls_share_the_barrier():
    """Five calls in a row on one workspace, each with new inputs and a
    different grid size, each checked: the barrier resets itself."""
    ws = moe.route_dispatch_workspace(DEV)
    for i, T in enumerate([128, 37, 128, 500, 3]):
        wl = W.get("ll_decode").replace(T=T, seed=100 + i)
        say(f"[gpu] route_dispatch repeat {i} T={T}")
        run_case(wl, ws=ws)


def test_route_dispatch_equals_separate_calls():
    """Same outputs as route_topk -> get_layout -> dispatch on the GPU,
    whole receive buffers included, then the combine on top."""
    wl = W.get("ll_decode")
    say("[gpu] route_dispatch vs separate calls")
    logits = torch.from_numpy(W.gen_logits(wl)).to(DEV)
    x = bf16_to_dev(W.gen_x(wl))
    N = wl.N
    f_out = prefilled_out(wl, N, "fp8")
    idx, w, lay, rx, rs = moe.route_dispatch(logits, x, wl.G, wl.g, wl.k, wl.R, wl.capacity, out=f_out)
    s_idx, s_w = moe.route_topk(logits, wl.G, wl.g, wl.k, wl.score)
    s_lay = moe.get_layout(s_idx, wl.E, wl.R, wl.capacity)
    _, _, _, s_rx, s_rs = prefilled_out(wl, N, "fp8")
    moe.dispatch(x, s_lay.pos, N, "fp8", s_rx, s_rs)
    torch.cuda.synchronize()
    assert torch.equal(idx, s_idx) and torch.equal(w.view(torch.int32), s_w.view(torch.int32))
    for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src", "flags"):
        assert torch.equal(getattr(lay, name), getattr(s_lay, name)), name
    assert torch.equal(rx, s_rx) and torch.equal(rs.view(torch.int32), s_rs.view(torch.int32))
    y = torch.randn((N, wl.H), device=DEV).to(torch.bfloat16)
    assert torch.equal(moe.combine(y, lay.pos, w), moe.combine(y, s_lay.pos, s_w))


def test_route_dispatch_rejects_large_batches():
    wl = W.get("dsv3_prefill").replace(T=2048)
    with pytest.raises(moe.MoeError) as e:
        moe.route_dispatch(torch.zeros((wl.T, wl.E), dtype=torch.float32, device=DEV),
                           torch.zeros((wl.T, wl.H), dtype=torch.bfloat16, device=DEV), wl.G, wl.g, wl.k, wl.R)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED


def test_route_dispatch_refused_workspace():
    """A workspace whose give-up word is nonzero (set here from the host: no
    block is ever made to wait) is refused: the call reports
    MOE_FLAG_INCOMPLETE and leaves the barrier words as they were; zeroed
    again, the workspace works."""
    wl = W.get("ll_decode")
    say("[gpu] route_dispatch on a refused workspace")
    ws = moe.route_dispatch_workspace(DEV)
    ws.view(torch.int32)[2] = 1
    before = ws.clone()
    out = prefilled_out(wl, wl.N, "fp8")
    _, _, lay, _, _ = moe.route_dispatch(torch.from_numpy(W.gen_logits(wl)).to(DEV), bf16_to_dev(W.gen_x(wl)),
                                         wl.G, wl.g, wl.k, wl.R, wl.capacity, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert int(lay.flags.item()) == moe.FLAG_INCOMPLETE
    assert torch.equal(ws, before)
    assert moe.barrier_gave_up(ws) == 1
    moe.reset_barrier_workspace(ws)
    run_case(wl, ws=ws)
