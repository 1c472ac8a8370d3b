"""Pins of the oracle's expert MLP (up projection + SwiGLU + FP8 requantisation,
down projection) to things other than itself: closed forms with identity
weights, NumPy matrix products on the dequantised operands, and the
invariants of the power-of-two quantiser.  CPU only."""
import numpy as np
import pytest

import oracle
import workloads as W

E4M3_VALUES = np.array([oracle.e4m3_value(c) for c in range(256)])


def deq(codes, scales, block_rows=1):
    """Dequantise codes [..., R, K] with scales [..., R/block_rows, K/128]."""
    v = E4M3_VALUES[codes]
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=-1), block_rows, axis=-2)
    return v * s


def silu_glu(h, I):
    g, u = h[..., :I], h[..., I:]
    return g / (1.0 + np.exp(-g)) * u


def test_up_identity_weights_closed_form():
    """Gate rows = identity, up rows = 2 x identity, expert e scaled by 2^e:
    act = silu(2^e x) * 2^(e+1) x, column for column."""
    wl = W.MlpWorkload("id", N=40, H=128, I=128, E=2)
    x, xs = W.gen_mlp_x(wl)
    w1 = np.zeros((2, 256, 128), np.uint8)
    for n in range(128):
        w1[:, n, n] = 0x38        # 1.0
        w1[:, 128 + n, n] = 0x40  # 2.0
    w1s = np.stack([np.full((2, 1), 1.0, np.float32), np.full((2, 1), 2.0, np.float32)])
    start, count = np.array([0, 25], np.int32), np.array([25, 15], np.int32)
    _, _, act = oracle.mlp_up(x, xs, w1, w1s, start, count, want_f64=True)
    xd = deq(x, xs)
    for p in range(40):
        e = 0 if p < 25 else 1
        g = xd[p] * 2.0 ** e
        want = g / (1.0 + np.exp(-g)) * (2.0 * g)
        np.testing.assert_allclose(act[p], want, rtol=1e-14, atol=1e-300)


def test_up_matches_numpy_matmul():
    wl = W.MlpWorkload("r", N=90, H=256, I=256, E=4)
    x, xs = W.gen_mlp_x(wl)
    w1, w1s = W.gen_mlp_weights(wl, "w1")
    # expert 2 is empty; rows 80..89 belong to nobody
    start = np.array([0, 30, 50, 50], np.int32)
    count = np.array([30, 20, 0, 30], np.int32)
    act, act_s, f64 = oracle.mlp_up(x, xs, w1, w1s, start, count, want_f64=True)
    xd = deq(x, xs)
    wd = deq(w1, w1s, block_rows=128)
    for e in range(4):
        rows = slice(start[e], start[e] + count[e])
        h = xd[rows] @ wd[e].T
        bound = 1e-12 * (np.abs(xd[rows]) @ np.abs(wd[e]).T)
        want = silu_glu(h, 256)
        assert np.all(np.abs(f64[rows] - want) <= 1e-12 * np.abs(want) + bound[:, :256] * 4 + 1e-300)
    assert np.isnan(f64[80:]).all() and not act[80:].any() and not act_s[80:].any()


def test_up_quantiser_invariants():
    """Every 128-column block: a power-of-two scale s, the smallest with
    amax <= 448 s; decoded codes within half an E4M3 step of the fp32 values."""
    wl = W.MlpWorkload("q", N=64, H=256, I=384, E=2)
    x, xs = W.gen_mlp_x(wl)
    w1, w1s = W.gen_mlp_weights(wl, "w1")
    start, count = np.array([0, 40], np.int32), np.array([40, 24], np.int32)
    act, act_s, f64 = oracle.mlp_up(x, xs, w1, w1s, start, count, want_f64=True)
    a32 = f64.astype(np.float32).astype(np.float64)
    m, ex = np.frexp(act_s.astype(np.float64))
    assert np.all(m == 0.5)                                   # powers of two
    amax = np.abs(a32).reshape(64, 3, 128).max(-1)
    a = np.maximum(amax, 2.0 ** -100)
    assert np.all(a <= 448.0 * act_s) and np.all(a > 224.0 * act_s)
    s = np.repeat(act_s.astype(np.float64), 128, axis=1)
    dq = E4M3_VALUES[act] * s
    assert np.all(np.abs(dq - a32) <= 2.0 ** -4 * np.abs(a32) + 2.0 ** -10 * s)


def test_down_matches_numpy_matmul():
    wl = W.MlpWorkload("d", N=70, H=384, I=256, E=3)
    rng = np.random.default_rng(5)
    act = rng.integers(0, 0x7F, (70, 256)).astype(np.uint8) | (rng.integers(0, 2, (70, 256)) << 7).astype(np.uint8)
    act_s = np.ldexp(np.float32(1.0), rng.integers(-9, -6, (70, 2))).astype(np.float32)
    w2, w2s = W.gen_mlp_weights(wl, "w2")
    start, count = np.array([0, 20, 45], np.int32), np.array([20, 25, 25], np.int32)
    y = oracle.mlp_down(act, act_s, w2, w2s, start, count)
    ad = deq(act, act_s)
    wd = deq(w2, w2s, block_rows=128)
    for e in range(3):
        rows = slice(start[e], start[e] + count[e])
        want = oracle.bf16_from_f64(ad[rows] @ wd[e].T)
        got = y[rows]
        exact = np.mean(got == want)
        assert exact >= 0.9999, exact
        assert np.all(np.abs(got.astype(np.int32) - want.astype(np.int32)) <= 1)


def test_row_list_equals_full_and_leaves_others():
    wl = W.MlpWorkload("l", N=50, H=128, I=128, E=2)
    x, xs = W.gen_mlp_x(wl)
    w1, w1s = W.gen_mlp_weights(wl, "w1")
    w2, w2s = W.gen_mlp_weights(wl, "w2")
    start, count = np.array([0, 20], np.int32), np.array([20, 30], np.int32)
    full_a, full_s, _ = oracle.mlp_up(x, xs, w1, w1s, start, count)
    rows = np.array([3, 19, 20, 49], np.int32)
    sa = np.full((50, 128), 0xEE, np.uint8)
    ss = np.full((50, 1), -1.0, np.float32)
    oracle.mlp_up(x, xs, w1, w1s, start, count, rows=rows, act=sa, act_s=ss)
    assert np.array_equal(sa[rows], full_a[rows]) and np.array_equal(ss[rows], full_s[rows])
    others = np.setdiff1d(np.arange(50), rows)
    assert np.all(sa[others] == 0xEE) and np.all(ss[others] == -1.0)
    yfull = oracle.mlp_down(full_a, full_s, w2, w2s, start, count)
    ys = np.full((50, 128), 0x1234, np.uint16)
    oracle.mlp_down(full_a, full_s, w2, w2s, start, count, rows=rows, y=ys)
    assert np.array_equal(ys[rows], yfull[rows]) and np.all(ys[others] == 0x1234)


def test_row_outside_every_expert_is_rejected():
    wl = W.MlpWorkload("o", N=10, H=128, I=128, E=1)
    x, xs = W.gen_mlp_x(wl)
    w1, w1s = W.gen_mlp_weights(wl, "w1")
    with pytest.raises(ValueError):
        oracle.mlp_up(x, xs, w1, w1s, np.array([0], np.int32), np.array([5], np.int32),
                      rows=np.array([7], np.int32))
