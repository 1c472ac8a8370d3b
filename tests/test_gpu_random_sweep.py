"""Seeded random sweeps through the C ABI against the oracle.

Each case draws one configuration from the shapes the API accepts -- E up to
512 with any group count dividing it, k up to 16, a rank count dividing E,
compact, padded (often overflowing) and tile-aligned layouts, all four
dispatch dtypes, sigmoid and softmax scores with and without renormalisation,
tie-heavy logits, T from 0 to 1500 -- and runs route -> layout -> dispatch ->
combine on the GPU.  Every stage is checked against the oracle on the GPU's
own inputs to that stage: indices and weights, every layout array and the
flags, FP8 codes and scales (or BF16 copies, untouched rows included) bit for
bit, the combine within its bound (tests/bounds.py).  The same generator
also draws configurations for the one-launch route + layout + dispatch
(at most 1024 tokens, within its LDS limit) and for the backward pair."""
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bounds  # noqa: E402
import combine_group_limited_amd as moe  # noqa: E402
import oracle  # noqa: E402

DEV = torch.device("cuda:0")
N_CASES = 40
ODT = {"fp8": oracle.FP8, "bf16": oracle.BF16, "fp8_pow2": oracle.FP8_POW2, "fp8_ue8m0": oracle.FP8_UE8M0}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_from_dev(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def divisors(n, limit):
    return [d for d in range(1, min(n, limit) + 1) if n % d == 0]


def draw(case):
    """One configuration the API accepts, from a generator seeded by the case."""
    rng = np.random.default_rng(1000 + case)
    E = int(rng.choice([8, 16, 24, 32, 48, 64, 96, 128, 160, 256, 384, 512]))
    G = int(rng.choice(divisors(E, 64)))
    g = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, min(16, g * (E // G)) + 1))
    topn = int(rng.integers(1, E // G + 1)) if rng.random() < 0.2 else 0
    R = int(rng.choice(divisors(E, E)))
    T = 0 if rng.random() < 0.05 else int(rng.integers(1, 1501))
    dtype = str(rng.choice(["fp8", "fp8_pow2", "fp8_ue8m0", "bf16"]))
    H = int(rng.choice([128, 256, 512, 1024, 1536, 2048] if dtype != "bf16" else [8, 64, 264, 1024, 2000]))
    C = A = 0
    u = rng.random()
    if u < 0.3:
        C = int(rng.integers(1, max(2, 2 * T * k // E + 3)))
    elif u < 0.5:
        A = int(rng.choice([2, 4, 8, 16, 32]))
    score = "softmax" if rng.random() < 0.3 else "sigmoid"
    renorm = bool(rng.random() >= 0.2)
    ties = bool(rng.random() < 0.3)
    return dict(T=T, E=E, G=G, g=g, k=k, topn=topn, R=R, H=H, C=C, A=A, dtype=dtype, score=score,
                renorm=renorm, ties=ties, seed=2000 + case)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration(case):
    c = draw(case)
    say(f"[gpu] random sweep case {case}: {c}")
    T, E, G, g, k, R, H, C, A = (c[n] for n in ("T", "E", "G", "g", "k", "R", "H", "C", "A"))
    rng = np.random.default_rng(c["seed"])
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if c["ties"]:
        logits = W.tie_heavy(logits)
    sf = oracle.SOFTMAX if c["score"] == "softmax" else oracle.SIGMOID

    # route
    ridx, rw = oracle.route(logits, G, g, k, score_fn=sf, renormalize=c["renorm"], group_topn=c["topn"])
    idx, w = moe.route_topk(torch.from_numpy(logits).to(DEV), G, g, k, c["score"], c["renorm"], c["topn"])
    assert np.array_equal(idx.cpu().numpy(), ridx), "idx"
    assert np.array_equal(w.cpu().numpy().view(np.uint32), rw.view(np.uint32)), "w"

    # layout
    rlay = oracle.layout(ridx, E, R, C, A)
    lay = moe.get_layout(idx, E, R, C, align_rows=A)
    for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, name).cpu().numpy(), rlay[name]), name
    assert int(lay.flags.item()) == rlay["flags"], "flags"

    # dispatch into prefilled buffers (rows no pair fills must stay untouched)
    N = moe.recv_rows(T, E, k, C, A)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    fp8 = c["dtype"] != "bf16"
    S = H // 128
    if fp8:
        rrx = np.full((N, H), 0xA5, np.uint8)
        rrs = np.full((N, S), 0xEE, np.uint8) if c["dtype"] == "fp8_ue8m0" else np.full((N, S), -3.0, np.float32)
        rx = torch.from_numpy(rrx.copy()).to(DEV)
        rs = torch.from_numpy(rrs.copy()).to(DEV)
    else:
        rrx = np.full((N, H), 0x7A5A, np.uint16)
        rrs = None
        rx = bf16_to_dev(rrx.copy())
        rs = None
    rrx, rrs = oracle.dispatch(x, rlay["pos"], N, ODT[c["dtype"]], rrx, rrs)
    rx, rs = moe.dispatch(bf16_to_dev(x), lay.pos, N, c["dtype"], rx, rs)
    if fp8:
        assert np.array_equal(rx.cpu().numpy(), rrx), "recv_x"
        assert np.array_equal(rs.cpu().numpy().view(np.uint8), rrs.view(np.uint8)), "recv_scales"
    else:
        assert np.array_equal(bf16_from_dev(rx), rrx), "recv_x"

    # combine of synthetic expert outputs
    y = W.f32_to_bf16_bits(rng.standard_normal((max(N, 1), H), dtype=np.float32))[:N]
    ref = oracle.combine(y, rlay["pos"], rw)
    out = moe.combine(bf16_to_dev(y), lay.pos, w)
    if T == 0:
        assert tuple(out.shape) == (0, H)
        return
    bad, rel, _ = bounds.combine_check(bf16_from_dev(out), ref, y, rlay["pos"], rw)
    assert bad == 0, f"{bad} combine outputs outside the bound (max rel {rel:.3g})"


def fused_lds_bytes(T, E, k, R):
    """The one-launch decode path's LDS need, as include/moe.h states it."""
    return 8 * ((T + 63) // 64) * (E + R) + 4 * (2 * E + 1 + T * k + 2048)


@pytest.mark.parametrize("case", range(20))
def test_random_route_dispatch(case):
    """The one-launch route + layout + dispatch on drawn configurations of at
    most 1024 tokens: every output bit for bit against the oracle."""
    c = draw(500 + case)
    T = min(c["T"], 1024)
    E, G, g, k, R, H, C, A = (c[n] for n in ("E", "G", "g", "k", "R", "H", "C", "A"))
    if fused_lds_bytes(T, E, k, R) > 64512:
        pytest.skip("beyond the one-launch LDS limit")
    say(f"[gpu] random route_dispatch case {case}: {dict(c, T=T)}")
    rng = np.random.default_rng(c["seed"])
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if c["ties"]:
        logits = W.tie_heavy(logits)
    sf = oracle.SOFTMAX if c["score"] == "softmax" else oracle.SIGMOID
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    ridx, rw = oracle.route(logits, G, g, k, score_fn=sf, renormalize=c["renorm"], group_topn=c["topn"])
    rlay = oracle.layout(ridx, E, R, C, A)
    N = moe.recv_rows(T, E, k, C, A)
    fp8 = c["dtype"] != "bf16"
    S = H // 128
    if fp8:
        rrx = np.full((N, H), 0xA5, np.uint8)
        rrs = np.full((N, S), 0xEE, np.uint8) if c["dtype"] == "fp8_ue8m0" else np.full((N, S), -3.0, np.float32)
        rx, rs = torch.from_numpy(rrx.copy()).to(DEV), torch.from_numpy(rrs.copy()).to(DEV)
    else:
        rrx, rrs = np.full((N, H), 0x7A5A, np.uint16), None
        rx, rs = bf16_to_dev(rrx.copy()), None
    rrx, rrs = oracle.dispatch(x, rlay["pos"], N, ODT[c["dtype"]], rrx, rrs)
    lay = moe.alloc_layout(T, E, k, R, C, DEV, A)[0]
    idx = torch.full((T, k), -5, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), -5.0, dtype=torch.float32, device=DEV)
    idx, w, lay, rx, rs = moe.route_dispatch(torch.from_numpy(logits).to(DEV), bf16_to_dev(x), G, g, k, R, C,
                                             c["dtype"], c["score"], c["renorm"], c["topn"], A,
                                             out=(idx, w, lay, rx, rs))
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx), "idx"
    assert np.array_equal(w.cpu().numpy().view(np.uint32), rw.view(np.uint32)), "w"
    for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, name).cpu().numpy(), rlay[name]), name
    assert int(lay.flags.item()) == rlay["flags"], "flags"
    if fp8:
        assert np.array_equal(rx.cpu().numpy(), rrx), "recv_x"
        assert np.array_equal(rs.cpu().numpy().view(np.uint8), rrs.view(np.uint8)), "recv_scales"
    else:
        assert np.array_equal(bf16_from_dev(rx), rrx), "recv_x"


@pytest.mark.parametrize("case", range(20))
def test_random_backward(case):
    """combine_backward (grad_y bit for bit, grad_w within 1e-5 of the
    products' magnitude) and dispatch_backward (the combine bound with unit
    weights) on drawn configurations."""
    c = draw(800 + case)
    T, E, G, g, k, R, C, A = (c[n] for n in ("T", "E", "G", "g", "k", "R", "C", "A"))
    H = c["H"] if c["H"] % 8 == 0 else 8
    say(f"[gpu] random backward case {case}: {dict(c, H=H)}")
    rng = np.random.default_rng(c["seed"])
    logits = rng.standard_normal((T, E), dtype=np.float32)
    sf = oracle.SOFTMAX if c["score"] == "softmax" else oracle.SIGMOID
    ridx, rw = oracle.route(logits, G, g, k, score_fn=sf, renormalize=c["renorm"], group_topn=c["topn"])
    pos = oracle.layout(ridx, E, R, C, A)["pos"]
    N = moe.recv_rows(T, E, k, C, A)
    gout = W.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    y = W.f32_to_bf16_bits(rng.standard_normal((max(N, 1), H), dtype=np.float32))[:N]
    fill = np.full((N, H), 0x7FC1, np.uint16)
    ref_gy, ref_gw = oracle.combine_backward(gout, y, pos, rw, grad_y=fill.copy())
    gy, gw = moe.combine_backward(bf16_to_dev(gout), bf16_to_dev(y), torch.from_numpy(pos).to(DEV),
                                  torch.from_numpy(rw).to(DEV), grad_y=bf16_to_dev(fill.copy()))
    gx = moe.dispatch_backward(bf16_to_dev(y), torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_from_dev(gy), ref_gy), "grad_y"
    if T == 0:
        return
    gwh = gw.cpu().numpy().astype(np.float64)
    gf = W.bf16_bits_to_f32(gout).astype(np.float64)
    yf = W.bf16_bits_to_f32(y).astype(np.float64)
    mag = np.zeros(pos.shape)
    for j in range(k):
        ok = pos[:, j] >= 0
        mag[ok, j] = np.abs(gf[ok] * yf[pos[ok, j]]).sum(1)
    err = np.abs(gwh - ref_gw.astype(np.float64))
    assert np.all(err <= 1e-5 * mag + 1e-30), "grad_w"
    assert np.all(gwh[pos < 0] == 0), "grad_w of dropped pairs"
    ref_gx = oracle.dispatch_backward(y, pos)
    bad, rel, _ = bounds.combine_check(bf16_from_dev(gx), ref_gx, y, pos, np.ones((T, k), np.float32))
    assert bad == 0, f"{bad} grad_x outside the bound (max rel {rel:.3g})"
