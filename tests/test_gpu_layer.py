"""A whole MoE layer on the GPU through the C ABI: route -> layout (tile-
aligned expert regions) -> FP8 dispatch with power-of-two scales -> expert
up (SwiGLU, FP8 requantisation) -> expert down -> combine.  Every stage is
checked against the oracle on the GPU's own inputs to that stage, so the test
pins how the stages fit together (receive-row order, expert ranges, scale
formats) as well as each stage's arithmetic."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_from_dev(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("T,H,I,E,G,g,k,R,A", [
    (256, 512, 256, 16, 4, 2, 4, 4, 128),
    (300, 1024, 384, 32, 8, 4, 8, 8, 64),
    (128, 7168, 128, 256, 8, 4, 8, 32, 128),
])
def test_layer_stages_fit_together(T, H, I, E, G, g, k, R, A):
    say(f"[gpu] layer T={T} H={H} I={I} E={E} k={k} align={A}")
    wl = W.custom("layer", T=T, H=H, E=E, G=G, g=g, k=k, score="sigmoid", R=R, dtype="fp8")
    mw = W.MlpWorkload("layer_mlp", N=1, H=H, I=I, E=E, seed=7)
    x = W.gen_x(wl)
    logits = W.gen_logits(wl)
    w1, w1s = W.gen_mlp_weights(mw, "w1")
    w2, w2s = W.gen_mlp_weights(mw, "w2")

    # route + layout + dispatch: bit-exact
    idx, w = moe.route_topk(torch.from_numpy(logits).to(DEV), G, g, k)
    ridx, rw = oracle.route(logits, G, g, k)
    assert np.array_equal(idx.cpu().numpy(), ridx) and np.array_equal(w.cpu().numpy(), rw)
    lay = moe.get_layout(idx, E, R, align_rows=A)
    rlay = oracle.layout(ridx, E, R, align=A)
    for n in ("cnt_e", "off_e", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, n).cpu().numpy(), rlay[n]), n
    N = lay.num_recv_rows
    rx = torch.zeros((N, H), dtype=torch.uint8, device=DEV)
    rs = torch.ones((N, H // 128), dtype=torch.float32, device=DEV)
    moe.dispatch(bf16_to_dev(x), lay.pos, N, "fp8_pow2", rx, rs)
    ref_q, ref_s = oracle.dispatch(x, rlay["pos"], N, oracle.FP8_POW2,
                                   np.zeros((N, H), np.uint8), np.ones((N, H // 128), np.float32))
    assert np.array_equal(rx.cpu().numpy(), ref_q) and np.array_equal(rs.cpu().numpy(), ref_s)

    # expert MLP on the receive buffer, ranges from the layout
    cnt, off = rlay["cnt_e"], rlay["off_e"]
    assert np.all(off[:-1] % A == 0)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    act, act_s = moe.expert_up(rx, rs, d(w1), d(w1s), lay.cnt_e, lay.off_e)
    y = moe.expert_down(act, act_s, d(w2), d(w2s), lay.cnt_e, lay.off_e,
                        y=torch.zeros((N, H), dtype=torch.bfloat16, device=DEV))
    act_g, act_s_g = act.cpu().numpy(), act_s.cpu().numpy()
    # up against the oracle on sampled rows of every non-empty expert
    rows = np.array(sorted({int(off[e] + j) for e in range(E) if cnt[e] > 0
                            for j in (0, cnt[e] // 2, cnt[e] - 1)}), np.int32)
    ra, rsc, f64 = oracle.mlp_up(ref_q, ref_s, w1, w1s, off[:-1], cnt, rows=rows, want_f64=True)
    dq = np.array([oracle.e4m3_value(c) for c in range(256)])[act_g[rows]] * np.repeat(act_s_g[rows], 128, axis=1)
    ref = f64[rows]
    assert np.mean(act_g[rows] == ra[rows]) > 0.99
    assert np.all(np.abs(dq - ref) <= 0.0626 * np.abs(ref) + 2.0 ** -10 * np.repeat(act_s_g[rows], 128, axis=1)
                  + 1e-3 * np.abs(ref).max())
    # down on the GPU's act: within one bf16 step plus the fp32 sum
    ry = oracle.mlp_down(act_g, act_s_g, w2, w2s, off[:-1], cnt, rows=rows)
    yg = W.bf16_bits_to_f32(bf16_from_dev(y)[rows]).astype(np.float64)
    yr = W.bf16_bits_to_f32(ry[rows]).astype(np.float64)
    assert np.all(np.abs(yg - yr) <= 2.0 ** -7 * np.abs(yr) + 1e-3 * np.abs(yr).max())

    # combine of the GPU's expert outputs, against the oracle's combine of the same rows
    out = moe.combine(y, lay.pos, w)
    yb = bf16_from_dev(y)
    ref_out = oracle.combine(yb, rlay["pos"], rw)
    got = W.bf16_bits_to_f32(bf16_from_dev(out)).astype(np.float64)
    want = W.bf16_bits_to_f32(ref_out).astype(np.float64)
    mag = np.zeros_like(want)
    yf = W.bf16_bits_to_f32(yb).astype(np.float64)
    for j in range(k):
        mag += np.abs(rw[:, j:j + 1] * yf[rlay["pos"][:, j]])
    assert np.all(np.abs(got - want) <= 1e-2 * np.abs(want) + 2 * k * 2.0 ** -24 * mag)
    say(f"   layer ok: {N} receive rows, {len(rows)} sampled MLP rows")
