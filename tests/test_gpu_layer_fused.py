"""The MoE layer after routing in one launch (moe_layer_forward): dispatch
(FP8, power-of-two scales) -> expert up -> expert down -> combine in a
persistent grid with grid-wide barriers.  Every array it writes (receive
codes and scales, act codes and scales, expert outputs y, combined output)
must equal, bit for bit, what the four separate calls write on the same
inputs: compact, tile-aligned and padded layouts, 256-row and 128-row expert
tiles, and several calls in a row on one barrier workspace, which must be
left at rest."""
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import combine_group_limited_amd as moe  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def fresh(N, H, I):
    return (torch.full((N, H), 0x11, dtype=torch.uint8, device=DEV),
            torch.full((N, H // 128), 3.0, dtype=torch.float32, device=DEV),
            torch.full((N, I), 0x22, dtype=torch.uint8, device=DEV),
            torch.full((N, I // 128), 5.0, dtype=torch.float32, device=DEV),
            torch.full((N, H), 77, dtype=torch.int16, device=DEV).view(torch.bfloat16))


@pytest.mark.parametrize("T,H,I,E,G,g,k,R,A,C", [
    (256, 512, 256, 16, 4, 2, 4, 4, 128, 0),      # aligned regions, 128-row tiles
    (300, 1024, 384, 32, 8, 4, 8, 8, 0, 0),       # compact, ragged tails
    (128, 7168, 128, 256, 8, 4, 8, 32, 128, 0),   # decode-sized, 256 experts
    (2048, 1024, 512, 8, 4, 2, 2, 8, 0, 0),       # 256-row tiles
    (512, 1024, 256, 16, 4, 2, 4, 4, 0, 160),     # padded (capacity) layout, drops
    (16384, 7168, 2048, 8, 1, 1, 2, 8, 0, 0),     # one rank's layer, the benchmark's shape
    (200, 640, 256, 8, 2, 1, 3, 4, 0, 0),         # H not a multiple of 512: a partial unit
    # more items per wave than one routing batch of the combine phase (64 / k
    # items) on a 1024-wave grid: two batches at k = 8; at k = 2 a partial
    # second batch and an odd item count per wave
    (16384, 512, 128, 16, 4, 2, 8, 4, 0, 0),
    (40000, 512, 128, 8, 4, 2, 2, 8, 0, 0),
])
def test_layer_one_launch_matches_four_calls(T, H, I, E, G, g, k, R, A, C):
    say(f"[gpu] one-launch layer T={T} H={H} I={I} E={E} k={k} align={A} capacity={C}")
    wl = W.custom("layer1", T=T, H=H, E=E, G=G, g=g, k=k, score="sigmoid", R=R, dtype="fp8")
    mw = W.MlpWorkload("layer1_mlp", N=1, H=H, I=I, E=E, seed=7)
    w1, w1s = W.gen_mlp_weights(mw, "w1")
    w2, w2s = W.gen_mlp_weights(mw, "w2")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    w1, w1s, w2, w2s = d(w1), d(w1s), d(w2), d(w2s)
    ws = moe.layer_workspace(DEV)
    for rep, seed in enumerate([0, 1, 2]):
        wl2 = wl.replace(seed=seed)
        x = bf16_to_dev(W.gen_x(wl2))
        idx, w = moe.route_topk(d(W.gen_logits(wl2)), G, g, k)
        lay = moe.get_layout(idx, E, R, C, align_rows=A)
        N = lay.num_recv_rows
        # the four calls
        rx, rs, act, act_s, y = fresh(N, H, I)
        moe.dispatch(x, lay.pos, N, "fp8_pow2", rx, rs)
        moe.expert_up(rx, rs, w1, w1s, lay.cnt_e, lay.off_e, C, act, act_s)
        moe.expert_down(act, act_s, w2, w2s, lay.cnt_e, lay.off_e, C, y)
        out = moe.combine(y, lay.pos, w)
        # one launch
        bufs = fresh(N, H, I)
        out1, _ = moe.layer_forward(x, lay.pos, w, lay.cnt_e, lay.off_e, w1, w1s, w2, w2s, N, C,
                                    workspace=ws, buffers=bufs)
        torch.cuda.synchronize()
        for name, a, b in zip(("recv_x", "recv_scales", "act", "act_scales", "y"), (rx, rs, act, act_s, y), bufs):
            assert same(a, b), (rep, name)
        assert same(out, out1), (rep, "out")
        words = ws.view(torch.int32).cpu().numpy()
        assert words[0] == 0 and words[2] == 0, words[:3]
        say(f"   call {rep} (seed {seed}): every array identical to the four calls")


def test_layer_rejects_small_workspace():
    """A workspace below moe_layer_workspace_bytes() is reported, not used."""
    T, H, I, E, k = 64, 512, 256, 4, 2
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    w = torch.zeros((T, k), dtype=torch.float32, device=DEV)
    cnt = torch.zeros((E,), dtype=torch.int32, device=DEV)
    off = torch.zeros((E + 1,), dtype=torch.int32, device=DEV)
    w1 = torch.zeros((E, 2 * I, H), dtype=torch.uint8, device=DEV)
    w1s = torch.ones((E, 2 * I // 128, H // 128), dtype=torch.float32, device=DEV)
    w2 = torch.zeros((E, H, I), dtype=torch.uint8, device=DEV)
    w2s = torch.ones((E, H // 128, I // 128), dtype=torch.float32, device=DEV)
    small = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError, match="workspace"):
        moe.layer_forward(x, pos, w, cnt, off, w1, w1s, w2, w2s, T * k, workspace=small)


def test_layer_graph_replays():
    """moe_layer_forward captured once in a HIP graph and replayed with new
    tokens and routing weights copied into the captured buffers: every replay
    equals an eager call on the same inputs (nothing in the launch allocates,
    synchronises or records a memset node, and the barrier workspace resets
    itself)."""
    T, H, I, E, G, g, k, R = 512, 1024, 256, 16, 4, 2, 4, 4
    wl = W.custom("layer_graph", T=T, H=H, E=E, G=G, g=g, k=k, score="sigmoid", R=R, dtype="fp8")
    mw = W.MlpWorkload("layer_graph_mlp", N=1, H=H, I=I, E=E, seed=7)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    w1, w1s = map(d, W.gen_mlp_weights(mw, "w1"))
    w2, w2s = map(d, W.gen_mlp_weights(mw, "w2"))
    x_s = bf16_to_dev(W.gen_x(wl))
    idx, w_s = moe.route_topk(d(W.gen_logits(wl)), G, g, k)
    lay = moe.get_layout(idx, E, R)
    N = lay.num_recv_rows
    bufs = fresh(N, H, I)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = moe.layer_workspace(DEV)

    def step():
        moe.layer_forward(x_s, lay.pos, w_s, lay.cnt_e, lay.off_e, w1, w1s, w2, w2s, N, 0, workspace=ws,
                          out=out, buffers=bufs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep, seed in enumerate([5, 6, 7]):
        wl2 = wl.replace(seed=seed)
        x_s.copy_(bf16_to_dev(W.gen_x(wl2)))
        w_s.copy_(torch.rand((T, k), dtype=torch.float32, device=DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref, rbufs = moe.layer_forward(x_s, lay.pos, w_s, lay.cnt_e, lay.off_e, w1, w1s, w2, w2s, N, 0,
                                       buffers=fresh(N, H, I))
        torch.cuda.synchronize()
        assert same(out, ref), rep
        assert same(bufs[4], rbufs[4]), rep
        words = ws.view(torch.int32).cpu().numpy()
        assert words[0] == 0 and words[2] == 0, words[:3]
        say(f"   replay {rep} (seed {seed}) identical to an eager call")
