"""The decode step under HIP graph capture: route -> layout -> dispatch ->
combine (separate launches) and moe_route_dispatch -> combine (one launch)
captured once and replayed with new inputs copied into the captured buffers,
every replay checked against eager calls on the same inputs.  Nothing in these
paths allocates, synchronises or clears memory with a memset node, and the
one-launch path's barrier workspace resets itself, so replays need no
preparation."""
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


def inputs(wl, seed):
    w2 = wl.replace(seed=seed)
    x = torch.from_numpy(W.gen_x(w2).view(np.int16)).to(DEV).view(torch.bfloat16)
    logits = torch.from_numpy(W.gen_logits(w2)).to(DEV)
    y = torch.from_numpy(W.gen_y(w2).view(np.int16)).to(DEV).view(torch.bfloat16)
    return x, logits, y


def eager(wl, x, logits, y):
    idx, w = moe.route_topk(logits, wl.G, wl.g, wl.k, wl.score)
    lay = moe.get_layout(idx, wl.E, wl.R, wl.capacity)
    rx, rs = moe.dispatch(x, lay.pos, wl.N, wl.dtype,
                          torch.zeros((wl.N, wl.H), dtype=torch.uint8, device=DEV),
                          torch.zeros((wl.N, wl.S), dtype=torch.float32, device=DEV))
    out = moe.combine(y, lay.pos, w)
    return idx, w, lay, rx, rs, out


@pytest.mark.parametrize("one_launch", [False, True])
def test_decode_step_graph_replays(one_launch):
    wl = W.get("ll_decode")
    say(f"[gpu] graph capture of the decode step, one_launch={one_launch}")
    x_s, l_s, y_s = inputs(wl, 0)
    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=DEV)
    lay_out = moe.alloc_layout(wl.T, wl.E, wl.k, wl.R, wl.capacity, DEV)
    rx = torch.zeros((wl.N, wl.H), dtype=torch.uint8, device=DEV)
    rs = torch.zeros((wl.N, wl.S), dtype=torch.float32, device=DEV)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    ws = moe.route_dispatch_workspace(DEV)

    def step():
        if one_launch:
            moe.route_dispatch(l_s, x_s, wl.G, wl.g, wl.k, wl.R, wl.capacity, wl.dtype, wl.score,
                               out=(idx, w, lay_out[0], rx, rs), workspace=ws)
        else:
            moe.route_topk(l_s, wl.G, wl.g, wl.k, wl.score, out=(idx, w))
            moe.get_layout(idx, wl.E, wl.R, wl.capacity, out=lay_out)
            moe.dispatch(x_s, lay_out[0].pos, wl.N, wl.dtype, rx, rs)
        moe.combine(y_s, lay_out[0].pos, w, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep, seed in enumerate([11, 12, 0, 13]):
        x, logits, y = inputs(wl, seed)
        x_s.copy_(x)
        l_s.copy_(logits)
        y_s.copy_(y)
        rx.zero_()
        rs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e_idx, e_w, e_lay, e_rx, e_rs, e_out = eager(wl, x, logits, y)
        torch.cuda.synchronize()
        assert torch.equal(idx, e_idx) and torch.equal(w.view(torch.int32), e_w.view(torch.int32)), rep
        for name in ("cnt_e", "off_e", "pos", "recv_src", "flags"):
            assert torch.equal(getattr(lay_out[0], name), getattr(e_lay, name)), (rep, name)
        assert torch.equal(rx, e_rx) and torch.equal(rs.view(torch.int32), e_rs.view(torch.int32)), rep
        assert torch.equal(out.view(torch.int16), e_out.view(torch.int16)), rep
        if one_launch:
            words = ws.view(torch.int32).cpu().numpy()
            assert words[0] == 0 and words[2] == 0, words[:3]
        say(f"   replay {rep} (seed {seed}) identical to eager")
