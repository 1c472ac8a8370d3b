"""Error bounds of the GPU's floating-point results against the oracle's
(shared by the GPU tests).

Combine: |gpu - oracle| <= 1e-2 |oracle| + 2 k 2^-24 sum_j |w_j y_j| per
element (the kernel accumulates in fp32 with one rounding per fma and rounds
to bf16 once; the oracle sums in double and rounds to bf16 once, so the two
differ by at most the bf16 rounding of each plus the fp32 accumulation error).

Expert MLP (double-precision oracle against the matrix cores):

The GPU sums on the matrix cores, the oracle in double, so results are
compared within bounds derived from the arithmetic.  The matrix cores' FP8
dot product is not sequential fp32: within one 64-deep step the products are
aligned to the largest and the bits below 2^-13 of it are dropped, toward
zero (measured on gfx950: a product 2^-14 of the largest vanishes,
1.5*2^-13 of it becomes 2^-13), so each step can lose up to
64 * 2^-13 * max|p|; the bounds add al = K 2^-12 max_k |a_k w_k| per output
(one bit of margin) to the fp32 terms below:
  up:   |dq_gpu - act| <= 2^-4 (|act| + d) + 2^-10 s_gpu + d, where
        d = 1.1 |u| dh + |silu(g)| dh + (|g| 2^-24 + 2^-20) |act| bounds the
        error of the activation (dh = K 2^-24 sum_k |x_k w_k| + al, the worst
        case of an fp32 sum of K terms plus the alignment loss; the last term
        covers SwiGLU itself, evaluated with the hardware exp2 and reciprocal,
        1 ulp each, on the rounded product -g log2(e)) and the rest is the
        E4M3 rounding of a value with power-of-two scale s (half a step,
        2^-10 s below the normals); scales must agree except where the fp32
        row maximum crossed a power of two (then by exactly a factor 2);
  down: |y_gpu - y| <= 2^-8 |y| + 2^-8 |y_gpu| + 2 K 2^-24 sum_k |a_k w_k| + al
        (one bf16 rounding on each side, the fp32 sum and the alignment loss).
"""
import concurrent.futures
import os

import numpy as np

import oracle
import workloads as W

E4M3 = np.array([oracle.e4m3_value(c) for c in range(256)])


def combine_check(got_bits, ref_bits, y_bits, pos, w):
    got = W.bf16_bits_to_f32(got_bits).astype(np.float64)
    ref = W.bf16_bits_to_f32(ref_bits).astype(np.float64)
    T, k = pos.shape
    yf = W.bf16_bits_to_f32(y_bits)
    mag = np.zeros_like(ref)
    for j in range(k):
        p = pos[:, j]
        ok = p >= 0
        mag[ok] += np.abs(w[ok, j:j + 1].astype(np.float64) * yf[p[ok]].astype(np.float64))
    bound = 1e-2 * np.abs(ref) + 2 * k * 2.0 ** -24 * mag
    bad = np.abs(got - ref) > bound
    big = np.abs(ref) >= 1e-2
    rel = np.abs(got - ref)[big] / np.abs(ref)[big]
    return int(bad.sum()), float(rel.max() if rel.size else 0.0), float(np.mean(got == ref))


def deq(codes, scales, block_rows=1):
    v = E4M3[codes]
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=-1), block_rows, axis=-2)
    return v * s


WORKERS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8))


def _parallel(fn, items):
    """fn over items on a thread pool (the C oracle and numpy's large array
    operations release the GIL); results in item order."""
    with concurrent.futures.ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(fn, items))


def _chunks(rows):
    return [c for c in np.array_split(np.asarray(rows, np.int32), max(1, min(len(rows), 4 * WORKERS))) if c.size]


def _expert_of(rows, start, count):
    return np.array([np.nonzero((r >= start) & (r < start + count))[0][0] for r in rows])


def oracle_up_rows(x, xs, w1, w1s, start, count, rows):
    """The oracle's up projection on the given rows, the rows split over
    threads that write disjoint rows of shared output arrays."""
    N, I = x.shape[0], w1.shape[1] // 2
    act = np.zeros((N, I), np.uint8)
    act_s = np.zeros((N, I // 128), np.float32)
    f64 = np.full((N, I), np.nan)
    _parallel(lambda r: oracle.mlp_up(x, xs, w1, w1s, start, count, rows=r, act=act, act_s=act_s, act_f64=f64),
              _chunks(rows))
    return act, act_s, f64


def oracle_down_rows(act, act_s, w2, w2s, start, count, rows):
    N, H = act.shape[0], w2.shape[1]
    y = np.zeros((N, H), np.uint16)
    _parallel(lambda r: oracle.mlp_down(act, act_s, w2, w2s, start, count, rows=r, y=y), _chunks(rows))
    return y


def check_up(x, xs, w1, w1s, start, count, act_g, act_s_g, rows):
    """Bounds of the module docstring on the given rows (numpy for the bound
    terms only; the reference values are the oracle's)."""
    I = w1.shape[1] // 2
    H = x.shape[1]
    ref_a, ref_s, f64 = oracle_up_rows(x, xs, w1, w1s, start, count, rows)
    e_of = _expert_of(rows, start, count)
    wd = dict(zip(sorted(set(e_of.tolist())),
                  _parallel(lambda e: deq(w1[e], w1s[e], block_rows=128), sorted(set(e_of.tolist())))))
    aw = {e: np.abs(v) for e, v in wd.items()}

    def one(i):
        r, e = rows[i], e_of[i]
        xd = deq(x[r:r + 1], xs[r:r + 1])[0]
        h = wd[e] @ xd
        S = aw[e] @ np.abs(xd)
        al = H * 2.0 ** -12 * np.max(aw[e] * np.abs(xd)[None, :], axis=1)
        dh = H * 2.0 ** -24 * S + al
        g, u = h[:I], h[I:]
        silu = g / (1.0 + np.exp(-g))
        a = f64[r]
        d = 1.1 * np.abs(u) * dh[:I] + np.abs(silu) * dh[I:] + (np.abs(g) * 2.0 ** -24 + 2.0 ** -20) * np.abs(a)
        s_g = np.repeat(act_s_g[r].astype(np.float64), 128)
        dq = E4M3[act_g[r]] * s_g
        bound = 2.0 ** -4 * (np.abs(a) + d) + 2.0 ** -10 * s_g + d
        ratio = act_s_g[r] / ref_s[r]
        assert np.all((ratio == 1.0) | (ratio == 2.0) | (ratio == 0.5)), (r, ratio)
        return (int(np.sum(np.abs(dq - a) > bound)), int(np.sum(act_g[r] == ref_a[r])), int(np.sum(ratio == 1.0)))

    res = np.array(_parallel(one, range(len(rows))))
    n = len(rows)
    return int(res[:, 0].sum()), res[:, 1].sum() / (n * I), res[:, 2].sum() / (n * (I // 128))


def check_down(act, act_s, w2, w2s, start, count, y_g_bits, rows):
    K = act.shape[1]
    ref = oracle_down_rows(act, act_s, w2, w2s, start, count, rows)
    e_of = _expert_of(rows, start, count)
    wd = dict(zip(sorted(set(e_of.tolist())),
                  _parallel(lambda e: deq(w2[e], w2s[e], block_rows=128), sorted(set(e_of.tolist())))))
    aw = {e: np.abs(v) for e, v in wd.items()}

    def one(i):
        r, e = rows[i], e_of[i]
        ad = np.abs(deq(act[r:r + 1], act_s[r:r + 1])[0])
        S = aw[e] @ ad
        al = K * 2.0 ** -12 * np.max(aw[e] * ad[None, :], axis=1)
        yr = W.bf16_bits_to_f32(ref[r]).astype(np.float64)
        yg = W.bf16_bits_to_f32(y_g_bits[r]).astype(np.float64)
        bound = 2.0 ** -8 * (np.abs(yr) + np.abs(yg)) + 2 * K * 2.0 ** -24 * S + al
        return int(np.sum(np.abs(yg - yr) > bound)), int(np.sum(y_g_bits[r] == ref[r]))

    res = np.array(_parallel(one, range(len(rows))))
    return int(res[:, 0].sum()), res[:, 1].sum() / (len(rows) * y_g_bits.shape[1])


def tile_rows(start, count, step=128, seed=0):
    """One row in every `step`-row tile of every expert's range [s, s + c),
    counted from the range's start (the expert-MLP kernels tile each expert
    from its first row, in 128- or 256-row tiles), plus each range's last row."""
    rng = np.random.default_rng(seed)
    rows = set()
    for s, c in zip(np.asarray(start).tolist(), np.asarray(count).tolist()):
        for t0 in range(s, s + c, step):
            rows.add(int(rng.integers(t0, min(t0 + step, s + c))))
        if c > 0:
            rows.add(s + c - 1)
    return np.array(sorted(rows), np.int32)
