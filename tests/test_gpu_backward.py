"""GPU parity of the backward pair against the CPU oracle, through the C ABI.

combine_backward: grad_y bit-exact (one rounding of the exact product on both
sides; rows no pair addresses untouched); grad_w within 1e-5 * sum_c |g_c y_c|
(the kernel sums fp32 products -- each exact, bf16 x bf16 -- lane by lane over
at most 112 terms and then over a 6-level tree, error <= 118 * 2^-24 of that
sum; the oracle sums in double).  dispatch_backward: the combine bound with
unit weights.
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def from_dev(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sum_bound(got_bits, ref_bits, rows_bits, pos, w):
    got = W.bf16_bits_to_f32(got_bits).astype(np.float64)
    ref = W.bf16_bits_to_f32(ref_bits).astype(np.float64)
    rf = W.bf16_bits_to_f32(rows_bits)
    k = pos.shape[1]
    mag = np.zeros_like(ref)
    for j in range(k):
        ok = pos[:, j] >= 0
        wj = np.abs(w[ok, j:j + 1].astype(np.float64)) if w is not None else 1.0
        mag[ok] += wj * np.abs(rf[pos[ok, j]].astype(np.float64))
    return int((np.abs(got - ref) > 1e-2 * np.abs(ref) + 2 * k * 2.0 ** -24 * mag).sum())


def case_inputs(wl):
    idx, w = oracle.route(W.gen_logits(wl), wl.G, wl.g, wl.k,
                          score_fn=oracle.SOFTMAX if wl.score == "softmax" else oracle.SIGMOID)
    lay = oracle.layout(idx, wl.E, wl.R, wl.capacity)
    rng = np.random.default_rng(wl.seed + 7)
    g = W.f32_to_bf16_bits(rng.standard_normal((wl.T, wl.H), dtype=np.float32))
    y = W.gen_y(wl)
    return lay["pos"], w, g, y


CASES = [W.get("dsv3_prefill"), W.get("mixtral"), W.get("ll_decode"), W.get("tiny"),
         W.custom("bw_ragged", T=77, H=640, E=16, G=4, g=2, k=3, score="sigmoid", R=4, dtype="fp8"),
         W.custom("bw_drop", T=65, H=1152, E=256, G=8, g=4, k=8, score="sigmoid", R=32, dtype="fp8",
                  capacity=3)]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_combine_backward_parity(wl):
    say(f"[gpu] combine_backward {W.describe(wl)}")
    pos, w, g, y = case_inputs(wl)
    fill = np.full((wl.N, wl.H), 0x7FC1, np.uint16)
    ref_gy, ref_gw = oracle.combine_backward(g, y, pos, w, grad_y=fill.copy())
    gy = to_dev(fill)
    gy2, gw = moe.combine_backward(to_dev(g), to_dev(y), torch.from_numpy(pos).to(DEV),
                                   torch.from_numpy(w).to(DEV), grad_y=gy)
    assert np.array_equal(from_dev(gy2), ref_gy)
    gwh = gw.cpu().numpy().astype(np.float64)
    gf = W.bf16_bits_to_f32(g).astype(np.float64)
    yf = W.bf16_bits_to_f32(y).astype(np.float64)
    mag = np.zeros(pos.shape)
    for j in range(pos.shape[1]):
        ok = pos[:, j] >= 0
        mag[ok, j] = np.abs(gf[ok] * yf[pos[ok, j]]).sum(1)
    err = np.abs(gwh - ref_gw.astype(np.float64))
    assert np.all(err <= 1e-5 * mag + 1e-30), float((err / np.maximum(mag, 1e-30)).max())
    assert np.all(gwh[pos < 0] == 0)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_dispatch_backward_parity(wl):
    say(f"[gpu] dispatch_backward {W.describe(wl)}")
    pos, _, _, y = case_inputs(wl)
    ref = oracle.dispatch_backward(y, pos)
    got = moe.dispatch_backward(to_dev(y), torch.from_numpy(pos).to(DEV))
    assert sum_bound(from_dev(got), ref, y, pos, None) == 0


def test_combine_backward_single_rounding_cases():
    cases = [(float.fromhex("0x1.419d0ap+0"), 1.859375), (float.fromhex("0x1.874a88p+0"), 1.234375),
             (1 + 2 ** -8, 1.0), (1 + 2 ** -8 + 2 ** -23, 1.0), (1 + 2 ** -8, 3.0)]
    T, H = len(cases), 64
    w = np.float32([[c[0]] for c in cases])
    g = W.f32_to_bf16_bits(np.float32([[c[1]] * (H // 2) + [-c[1]] * (H // 2) for c in cases]))
    y = np.zeros((T, H), np.uint16)
    pos = np.arange(T, dtype=np.int32)[:, None]
    ref_gy, _ = oracle.combine_backward(g, y, pos, w)
    gy, _ = moe.combine_backward(to_dev(g), to_dev(y), torch.from_numpy(pos).to(DEV), torch.from_numpy(w).to(DEV))
    assert np.array_equal(from_dev(gy), ref_gy)


def test_backward_launch_shapes_agree():
    wl = W.get("dsv3_prefill").replace(T=200)
    pos, w, g, y = case_inputs(wl)
    P, Wt, G, Y = (torch.from_numpy(pos).to(DEV), torch.from_numpy(w).to(DEV), to_dev(g), to_dev(y))
    ref = moe.combine_backward(G, Y, P, Wt, units_per_wave=1)
    for u in (2, 4, 7):
        got = moe.combine_backward(G, Y, P, Wt, units_per_wave=u)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), u
