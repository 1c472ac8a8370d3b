"""GPU parity of the expert MLP (moe_expert_up, moe_expert_down) through the C
ABI against the oracle.

Both sides read the same FP8 codes and power-of-two scales.  The GPU sums on
the matrix cores, the oracle in double, so results are compared within
bounds derived from the arithmetic.  The matrix cores' FP8 dot product is not
sequential fp32: within one 64-deep step the products are aligned to the
largest and the bits below 2^-13 of it are dropped, toward zero (measured on
gfx950: a product 2^-14 of the largest vanishes, 1.5*2^-13 of it becomes
2^-13), so each step can lose up to 64 * 2^-13 * max|p|; the bounds add
al = K 2^-12 max_k |a_k w_k| per output (one bit of margin) to the fp32
terms below:
  up:   |dq_gpu - act| <= 2^-4 (|act| + d) + 2^-10 s_gpu + d, where
        d = 1.1 |u| dh + |silu(g)| dh + (|g| 2^-24 + 2^-20) |act| bounds the
        error of the activation (dh = K 2^-24 sum_k |x_k w_k| + al, the worst
        case of an fp32 sum of K terms plus the alignment loss; the last term
        covers SwiGLU itself,
        evaluated with the hardware exp2 and reciprocal, 1 ulp each, on the
        rounded product -g log2(e)) and the rest is the E4M3 rounding of a
        value with power-of-two scale s (half a step, 2^-10 s below the
        normals);
        scales must agree except where the fp32 row maximum crossed a power
        of two (then by exactly a factor 2);
  down: |y_gpu - y| <= 2^-8 |y| + 2^-8 |y_gpu| + 2 K 2^-24 sum_k |a_k w_k| + al
        (one bf16 rounding on each side, the fp32 sum and the alignment loss).
Rows outside every expert's range must stay untouched.
"""
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
E4M3 = np.array([oracle.e4m3_value(c) for c in range(256)])


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def deq(codes, scales, block_rows=1):
    v = E4M3[codes]
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=-1), block_rows, axis=-2)
    return v * s


def layout_arrays(start, count, capacity=0):
    E = len(count)
    off = np.zeros(E + 1, np.int32)
    if capacity == 0:
        off[:E] = start
        off[E] = start[-1] + count[-1]
    return count.astype(np.int32), off


def check_up(x, xs, w1, w1s, start, count, act_g, act_s_g, rows):
    """Bounds of the module docstring on the given rows (numpy for the bound
    terms only; the reference values are the oracle's)."""
    I = w1.shape[1] // 2
    H = x.shape[1]
    ref_a, ref_s, f64 = oracle.mlp_up(x, xs, w1, w1s, start, count, rows=rows, want_f64=True)
    xd = deq(x[rows], xs[rows])
    wd = {}
    e_of = np.array([np.nonzero((r >= start) & (r < start + count))[0][0] for r in rows])
    nbad = 0
    code_eq = 0
    scale_eq = 0
    for i, r in enumerate(rows):
        e = e_of[i]
        if e not in wd:
            wd[e] = deq(w1[e], w1s[e], block_rows=128)
        h = wd[e] @ xd[i]
        S = np.abs(wd[e]) @ np.abs(xd[i])
        al = H * 2.0 ** -12 * np.max(np.abs(wd[e]) * np.abs(xd[i])[None, :], axis=1)
        dh = H * 2.0 ** -24 * S + al
        g, u = h[:I], h[I:]
        silu = g / (1.0 + np.exp(-g))
        a = f64[r]
        d = 1.1 * np.abs(u) * dh[:I] + np.abs(silu) * dh[I:] + (np.abs(g) * 2.0 ** -24 + 2.0 ** -20) * np.abs(a)
        s_g = np.repeat(act_s_g[r].astype(np.float64), 128)
        dq = E4M3[act_g[r]] * s_g
        bound = 2.0 ** -4 * (np.abs(a) + d) + 2.0 ** -10 * s_g + d
        nbad += int(np.sum(np.abs(dq - a) > bound))
        ratio = act_s_g[r] / ref_s[r]
        assert np.all((ratio == 1.0) | (ratio == 2.0) | (ratio == 0.5)), (r, ratio)
        scale_eq += int(np.sum(ratio == 1.0))
        code_eq += int(np.sum(act_g[r] == ref_a[r]))
    n = len(rows)
    return nbad, code_eq / (n * I), scale_eq / (n * (I // 128))


def check_down(act, act_s, w2, w2s, start, count, y_g_bits, rows):
    K = act.shape[1]
    ref = oracle.mlp_down(act, act_s, w2, w2s, start, count, rows=rows)
    ad = deq(act[rows], act_s[rows])
    wd = {}
    nbad = 0
    exact = 0
    for i, r in enumerate(rows):
        e = np.nonzero((r >= start) & (r < start + count))[0][0]
        if e not in wd:
            wd[e] = deq(w2[e], w2s[e], block_rows=128)
        S = np.abs(wd[e]) @ np.abs(ad[i])
        al = K * 2.0 ** -12 * np.max(np.abs(wd[e]) * np.abs(ad[i])[None, :], axis=1)
        yr = W.bf16_bits_to_f32(ref[r]).astype(np.float64)
        yg = W.bf16_bits_to_f32(y_g_bits[r]).astype(np.float64)
        bound = 2.0 ** -8 * (np.abs(yr) + np.abs(yg)) + 2 * K * 2.0 ** -24 * S + al
        nbad += int(np.sum(np.abs(yg - yr) > bound))
        exact += int(np.sum(y_g_bits[r] == ref[r]))
    return nbad, exact / (len(rows) * y_g_bits.shape[1])


def run_mlp(wl, start, count, capacity=0, rows=None, cnt_override=None):
    x, xs = W.gen_mlp_x(wl)
    w1, w1s = W.gen_mlp_weights(wl, "w1")
    w2, w2s = W.gen_mlp_weights(wl, "w2")
    cnt, off = layout_arrays(start, count, capacity)
    if cnt_override is not None:
        cnt = cnt_override
    act = torch.full((wl.N, wl.I), 0xEE, dtype=torch.uint8, device=DEV)
    act_s = torch.full((wl.N, wl.I // 128), -3.0, dtype=torch.float32, device=DEV)
    moe.expert_up(dev(x), dev(xs), dev(w1), dev(w1s), dev(cnt), dev(off), capacity, act, act_s)
    act_g = act.cpu().numpy()
    act_s_g = act_s.cpu().numpy()
    covered = np.zeros(wl.N, bool)
    for s, c in zip(start, count):
        covered[s:s + c] = True
    all_rows = np.nonzero(covered)[0].astype(np.int32)
    rows = all_rows if rows is None else rows
    # untouched rows keep the sentinel
    assert np.all(act_g[~covered] == 0xEE) and np.all(act_s_g[~covered] == -3.0)
    nbad, code_eq, scale_eq = check_up(x, xs, w1, w1s, start, count, act_g, act_s_g, rows)
    say(f"   up {wl.name}: {len(rows)} rows, codes equal {code_eq:.5f}, scales equal {scale_eq:.5f}, "
        f"out of bound {nbad}")
    assert nbad == 0 and code_eq > 0.99
    # down on the GPU's own act (identical inputs on both sides)
    y = torch.full((wl.N, wl.H), 1234, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.expert_down(act, act_s, dev(w2), dev(w2s), dev(cnt), dev(off), capacity, y)
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(yb[~covered] == 1234)
    nbad, exact = check_down(act_g, act_s_g, w2, w2s, start, count, yb, rows)
    say(f"   down {wl.name}: exact {exact:.5f}, out of bound {nbad}")
    assert nbad == 0 and exact > 0.9


def test_mlp_tiny_packed():
    wl = W.MLP_WORKLOADS["mlp_tiny"]
    say(f"[gpu] mlp {wl}")
    start, count, _ = W.mlp_ranges(wl)
    run_mlp(wl, start, count)


def test_mlp_ragged_with_empty_expert_and_gaps():
    wl = W.MlpWorkload("gaps", N=700, H=384, I=256, E=5)
    say(f"[gpu] mlp {wl}")
    start = np.array([0, 130, 130, 400, 690], np.int32)
    count = np.array([129, 0, 200, 250, 10], np.int32)   # rows 330..399 belong to nobody
    run_mlp(wl, start, count)


def test_mlp_aligned_regions():
    wl = W.MLP_WORKLOADS["mlp_tiny"].replace(N=600, align=128, H=512, I=384, E=4)
    say(f"[gpu] mlp aligned {wl}")
    start, count, _ = W.mlp_ranges(wl)
    run_mlp(wl, start, count)


def test_mlp_padded_capacity_clips_counts():
    wl = W.MlpWorkload("pad", N=4 * 96, H=256, I=256, E=4)
    say(f"[gpu] mlp padded {wl}")
    C = 96
    cnt = np.array([50, 96, 120, 0], np.int32)         # expert 2 overflows: only 96 rows used
    start = np.arange(4, dtype=np.int32) * C
    count = np.minimum(cnt, C).astype(np.int32)
    run_mlp(wl, start, count, capacity=C, cnt_override=cnt)


@pytest.mark.parametrize("N,H,I,E", [
    (300, 128, 128, 2),     # one 128-deep stage in both layers, 128-row tiles
    (1100, 384, 128, 2),    # 256-row tiles (>= 512 rows per expert): three stages up, one down
    (1536, 640, 384, 3),    # 256-row tiles, five and three stages
])
def test_mlp_short_and_odd_k(N, H, I, E):
    wl = W.MlpWorkload("shortk", N=N, H=H, I=I, E=E, seed=5)
    say(f"[gpu] mlp short/odd K {wl}")
    start, count, _ = W.mlp_ranges(wl)
    run_mlp(wl, start, count)


def test_mlp_many_experts():
    wl = W.MlpWorkload("many", N=8192, H=1024, I=512, E=128, seed=3)
    say(f"[gpu] mlp many experts {wl}")
    start, count, _ = W.mlp_ranges(wl)
    rows = np.random.default_rng(0).choice(int(start[-1] + count[-1]), 256, replace=False).astype(np.int32)
    run_mlp(wl, start, count, rows=np.sort(rows))


def test_mlp_rank_full_size_sampled():
    """One expert-parallel rank of the DeepSeek-V3 shape (8 experts, 32768
    rows, H 7168, I 2048) in the benchmark's launch configuration; 24 rows
    spread over all experts checked against the oracle."""
    wl = W.MLP_WORKLOADS["mlp_rank"]
    say(f"[gpu] mlp full size {wl}")
    start, count, _ = W.mlp_ranges(wl)
    rng = np.random.default_rng(1)
    rows = []
    for s, c in zip(start, count):
        rows += [s, s + c - 1, int(rng.integers(s, s + c))]
    run_mlp(wl, start, count, rows=np.array(sorted(rows), np.int32))


@pytest.mark.parametrize("N,H,I,E", [(4096, 1024, 512, 2), (1100, 640, 256, 2)])
def test_mlp_unaligned_scales_match_aligned(N, H, I, E):
    """Row scales at a 4-byte offset take the single-scale preload instead of
    the 16-byte loads; both layouts must give bit-identical act, act scales
    and y (256-row and 128-row tiles)."""
    wl = W.MlpWorkload("unal", N=N, H=H, I=I, E=E, seed=9)
    say(f"[gpu] mlp unaligned scales {wl}")
    start, count, _ = W.mlp_ranges(wl)
    x, xs = W.gen_mlp_x(wl)
    w1, w1s = W.gen_mlp_weights(wl, "w1")
    w2, w2s = W.gen_mlp_weights(wl, "w2")
    cnt, off = layout_arrays(start, count)

    def shifted(a):
        buf = torch.empty(a.size + 1, dtype=torch.float32, device=DEV)
        v = buf[1:].view(a.shape)
        v.copy_(dev(a))
        assert v.data_ptr() % 16 == 4
        return v

    outs = []
    for xs_d, act_sd in ((dev(xs), None), (shifted(xs), "shift")):
        act = torch.full((N, I), 0xEE, dtype=torch.uint8, device=DEV)
        act_s = torch.full((N, I // 128), -3.0, dtype=torch.float32, device=DEV)
        if act_sd:
            act_s = shifted(act_s.cpu().numpy())
        moe.expert_up(dev(x), xs_d, dev(w1), dev(w1s), dev(cnt), dev(off), 0, act, act_s)
        y = torch.full((N, H), 1234, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        moe.expert_down(act, act_s, dev(w2), dev(w2s), dev(cnt), dev(off), 0, y)
        torch.cuda.synchronize()
        outs.append((act.cpu().numpy(), act_s.cpu().numpy(), y.view(torch.int16).cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


def test_mlp_zero_rows_is_noop():
    cfg = moe.MlpCfg(0, 7168, 2048, 8, 0)
    assert moe.lib().moe_expert_up(cfg, None, None, None, None, None, None, None, None, None) == moe.MOE_OK
