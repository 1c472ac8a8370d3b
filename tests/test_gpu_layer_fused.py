"""The MoE layer after routing in one launch (moe_layer_forward): dispatch
(FP8, power-of-two scales) -> expert up -> expert down -> combine in a
persistent grid with grid-wide barriers.

Two checks.  Against the oracle: the receive codes and scales bit for bit,
act and its scales and the expert outputs y within the expert-MLP bounds on
one row of every 128-row tile of every expert, and the combined output within
the combine bound of the oracle's combine of the returned y -- on the shapes
below, up to one rank's layer at the benchmark's size.  Against the four
separate calls: every array bit for bit, with different sentinels in the two
sets of buffers so that a row neither path writes cannot pass unseen.  Both
also check compact, tile-aligned and padded layouts, 256-row and 128-row
expert tiles, and several calls in a row on one barrier workspace, which must
be left at rest; a workspace marked as given up (from the host: no block is
ever made to wait) is refused without touching the barrier's words."""
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
from bounds import check_down, check_up, combine_check, tile_rows  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


# sentinels per buffer set: recv_x, recv_scales, act, act_scales, y (bf16 bits)
SENTINELS = [(0x11, 3.0, 0x22, 5.0, 77), (0x33, 6.0, 0x44, 9.0, 99),
             (0x7F, -1.0, 0x7F, -1.0, 0x7FC1)]   # E4M3 NaN codes, negative scales, bf16 NaN


def fresh(N, H, I, variant=0):
    a, b, c, d, e = SENTINELS[variant]
    return (torch.full((N, H), a, dtype=torch.uint8, device=DEV),
            torch.full((N, H // 128), b, dtype=torch.float32, device=DEV),
            torch.full((N, I), c, dtype=torch.uint8, device=DEV),
            torch.full((N, I // 128), d, dtype=torch.float32, device=DEV),
            torch.full((N, H), e, dtype=torch.int16, device=DEV).view(torch.bfloat16))


def bits(t):
    return t.contiguous().view(torch.uint8) if t.dtype != torch.bfloat16 else t.contiguous().view(torch.int16)


SHAPES = [
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
]


def expert_ranges(lay, E, C):
    """Each expert's receive rows [start, start + count) as the MLP reads them."""
    cnt = lay.cnt_e.cpu().numpy().astype(np.int64)
    if C > 0:
        return (np.arange(E) * C).astype(np.int32), np.minimum(cnt, C).astype(np.int32)
    return lay.off_e.cpu().numpy()[:E].astype(np.int32), cnt.astype(np.int32)


@pytest.mark.parametrize("T,H,I,E,G,g,k,R,A,C", SHAPES)
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
        rx, rs, act, act_s, y = fresh(N, H, I, 0)
        moe.dispatch(x, lay.pos, N, "fp8_pow2", rx, rs)
        moe.expert_up(rx, rs, w1, w1s, lay.cnt_e, lay.off_e, C, act, act_s)
        moe.expert_down(act, act_s, w2, w2s, lay.cnt_e, lay.off_e, C, y)
        out = moe.combine(y, lay.pos, w)
        # one launch, into buffers holding other sentinels
        bufs = fresh(N, H, I, 1)
        out1, _ = moe.layer_forward(x, lay.pos, w, lay.cnt_e, lay.off_e, w1, w1s, w2, w2s, N, C,
                                    workspace=ws, buffers=bufs)
        torch.cuda.synchronize()
        # rows some pair fills (recv_src >= 0) are exactly the rows of the
        # expert ranges: they must agree; every other row keeps its own sentinel
        filled = lay.recv_src >= 0
        for i, (name, a, b) in enumerate(zip(("recv_x", "recv_scales", "act", "act_scales", "y"),
                                             (rx, rs, act, act_s, y), bufs)):
            assert torch.equal(bits(a)[filled], bits(b)[filled]), (rep, name)
            for t, v in ((a, 0), (b, 1)):
                ref = fresh(1, H, I, v)[i]
                assert torch.equal(bits(t)[~filled], bits(ref).expand(int((~filled).sum()), -1)), (rep, name, v)
        assert same(out, out1), (rep, "out")
        words = ws.view(torch.int32).cpu().numpy()
        assert words[0] == 0 and words[2] == 0, words[:3]
        say(f"   call {rep} (seed {seed}): every array identical to the four calls")


@pytest.mark.parametrize("T,H,I,E,G,g,k,R,A,C", SHAPES)
def test_layer_one_launch_against_oracle(T, H, I, E, G, g, k, R, A, C):
    say(f"[gpu] one-launch layer vs oracle T={T} H={H} I={I} E={E} k={k} align={A} capacity={C}")
    wl = W.custom("layer_o", T=T, H=H, E=E, G=G, g=g, k=k, score="sigmoid", R=R, dtype="fp8")
    mw = W.MlpWorkload("layer_o_mlp", N=1, H=H, I=I, E=E, seed=7)
    w1h, w1sh = W.gen_mlp_weights(mw, "w1")
    w2h, w2sh = W.gen_mlp_weights(mw, "w2")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    w1, w1s, w2, w2s = d(w1h), d(w1sh), d(w2h), d(w2sh)
    xh, logits = W.gen_x(wl), W.gen_logits(wl)
    # routing and layout: the oracle's, which the GPU's equal bit for bit
    idx_o, w_o = oracle.route(logits, G, g, k)
    lay_o = oracle.layout(idx_o, E, R, C, A)
    idx, w = moe.route_topk(d(logits), G, g, k)
    lay = moe.get_layout(idx, E, R, C, align_rows=A)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
    for name in ("cnt_e", "off_e", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, name).cpu().numpy(), lay_o[name]), name
    N = lay.num_recv_rows
    pos = lay_o["pos"]
    bufs = fresh(N, H, I, 2)
    out, _ = moe.layer_forward(bf16_to_dev(xh), lay.pos, w, lay.cnt_e, lay.off_e, w1, w1s, w2, w2s, N, C,
                               buffers=bufs)
    torch.cuda.synchronize()
    rx_g, rs_g, act_g, act_s_g = (t.cpu().numpy() for t in bufs[:4])
    y_g = bufs[4].view(torch.int16).cpu().numpy().view(np.uint16)
    # dispatch: bit-exact, unaddressed rows untouched
    rx_o, rs_o = oracle.dispatch(xh, pos, N, oracle.FP8_POW2, np.full((N, H), 0x7F, np.uint8),
                                 np.full((N, H // 128), -1.0, np.float32))
    assert np.array_equal(rx_g, rx_o)
    assert np.array_equal(rs_g.view(np.uint32), rs_o.view(np.uint32))
    # expert MLP: every row of every range written, others untouched; one row
    # of every 128-row tile of every expert within the bounds
    start, count = expert_ranges(lay, E, C)
    covered = np.zeros(N, bool)
    for s0, c0 in zip(start, count):
        covered[s0:s0 + c0] = True
    assert np.all(act_s_g[covered] > 0) and np.all(act_s_g[~covered] == -1.0)
    assert np.all(act_g[~covered] == 0x7F) and not np.any(act_g[covered] == 0x7F)
    assert np.all(y_g[~covered] == 0x7FC1) and not np.any(np.isnan(W.bf16_bits_to_f32(y_g[covered])))
    rows = tile_rows(start, count, 128, seed=T)
    nbad, code_eq, scale_eq = check_up(rx_o, rs_o, w1h, w1sh, start, count, act_g, act_s_g, rows)
    say(f"   up: {len(rows)} rows, codes equal {code_eq:.5f}, scales equal {scale_eq:.5f}, out of bound {nbad}")
    assert nbad == 0 and code_eq > 0.99
    nbad, exact = check_down(act_g, act_s_g, w2h, w2sh, start, count, y_g, rows)
    say(f"   down: exact {exact:.5f}, out of bound {nbad}")
    assert nbad == 0 and exact > 0.9
    # combine of the returned y
    out_o = oracle.combine(y_g, pos, w_o)
    out_g = out.view(torch.int16).cpu().numpy().view(np.uint16)
    nbad, maxrel, exact = combine_check(out_g, out_o, y_g, pos, w_o)
    say(f"   combine: out of bound {nbad}, max rel {maxrel:.2e}, exact {exact:.5f}")
    assert nbad == 0


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


def test_layer_refused_workspace():
    """Give-up word set from the host: the launch stops at its first barrier
    without arriving (barrier words unchanged) and barrier_gave_up reports it;
    after reset_barrier_workspace the same call equals the four calls."""
    T, H, I, E, G, g, k, R = 300, 1024, 384, 32, 8, 4, 8, 8
    say("[gpu] one-launch layer on a refused workspace")
    wl = W.custom("layer_ref", T=T, H=H, E=E, G=G, g=g, k=k, score="sigmoid", R=R, dtype="fp8")
    mw = W.MlpWorkload("layer_ref_mlp", N=1, H=H, I=I, E=E, seed=7)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    w1, w1s = map(d, W.gen_mlp_weights(mw, "w1"))
    w2, w2s = map(d, W.gen_mlp_weights(mw, "w2"))
    x = bf16_to_dev(W.gen_x(wl))
    idx, w = moe.route_topk(d(W.gen_logits(wl)), G, g, k)
    lay = moe.get_layout(idx, E, R)
    N = lay.num_recv_rows
    ws = moe.layer_workspace(DEV)
    ws.view(torch.int32)[2] = 3
    before = ws.view(torch.int32)[:768].clone()
    moe.layer_forward(x, lay.pos, w, lay.cnt_e, lay.off_e, w1, w1s, w2, w2s, N, workspace=ws,
                      buffers=fresh(N, H, I, 0))
    torch.cuda.synchronize()
    assert torch.equal(ws.view(torch.int32)[:768], before)
    assert moe.barrier_gave_up(ws) == 3
    moe.reset_barrier_workspace(ws)
    out1, b1 = moe.layer_forward(x, lay.pos, w, lay.cnt_e, lay.off_e, w1, w1s, w2, w2s, N, workspace=ws,
                                 buffers=fresh(N, H, I, 0))
    rx, rs, act, act_s, y = fresh(N, H, I, 1)
    moe.dispatch(x, lay.pos, N, "fp8_pow2", rx, rs)
    moe.expert_up(rx, rs, w1, w1s, lay.cnt_e, lay.off_e, 0, act, act_s)
    moe.expert_down(act, act_s, w2, w2s, lay.cnt_e, lay.off_e, 0, y)
    out = moe.combine(y, lay.pos, w)
    torch.cuda.synchronize()
    assert same(out, out1) and same(y, b1[4])
    assert moe.barrier_gave_up(ws) == 0
