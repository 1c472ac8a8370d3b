"""GPU parity: every kernel, through the C ABI, against the CPU oracle.

Bit-exact: top-k indices and weights, every layout output, FP8 codes and
scales, BF16 dispatch copies.  Combine: |gpu - oracle| <= 1e-2 |oracle| +
2 k 2^-24 sum_j |w_j y_j| per element (the kernel accumulates in fp32 with one
rounding per fma and rounds to bf16 once; the oracle sums in double and
rounds to bf16 once, so the two differ by at most the bf16 rounding of each
plus the fp32 accumulation error).  Full-size cases run in the launch
configuration the benchmark uses (the library's own choice).
"""
import ctypes
import os
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
from bounds import combine_check  # noqa: E402

DEV = torch.device("cuda:0")
HELPERS = os.path.join(os.path.dirname(__file__), "helpers")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_from_dev(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sf(wl):
    return oracle.SOFTMAX if wl.score == "softmax" else oracle.SIGMOID


# --------------------------------------------------------------------------
# per-workload reference data (oracle on the CPU), built once per module
# --------------------------------------------------------------------------
class Case:
    def __init__(self, wl, tie=False):
        self.wl = wl
        say(f"[oracle] {W.describe(wl)}{' tie-heavy' if tie else ''}")
        self.x = W.gen_x(wl)
        self.logits = W.gen_logits(wl)
        if tie:
            self.logits = W.tie_heavy(self.logits)
        self.y = W.gen_y(wl)
        self.idx, self.w = oracle.route(self.logits, wl.G, wl.g, wl.k, score_fn=sf(wl))
        self.lay = oracle.layout(self.idx, wl.E, wl.R, wl.capacity)
        fp8 = wl.dtype == "fp8"
        self.fill = 0xAB if fp8 else 0xABCD
        rx = np.full((wl.N, wl.H), self.fill, np.uint8 if fp8 else np.uint16)
        rs = np.full((wl.N, wl.S), -7.0, np.float32) if fp8 else None
        self.rx, self.rs = oracle.dispatch(self.x, self.lay["pos"], wl.N,
                                           oracle.FP8 if fp8 else oracle.BF16, rx, rs)
        self.out = oracle.combine(self.y, self.lay["pos"], self.w)


FULL = ["tiny", "dsv3_prefill", "ll_decode", "mixtral", "skewed_8k"]


@pytest.fixture(scope="module", params=FULL)
def case(request):
    return Case(W.get(request.param))


def test_route_parity(case):
    wl = case.wl
    say(f"[gpu] route {wl.name}")
    idx, w = moe.route_topk(torch.from_numpy(case.logits).to(DEV), wl.G, wl.g, wl.k, wl.score)
    assert np.array_equal(idx.cpu().numpy(), case.idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), case.w.view(np.uint32))


def test_layout_parity(case):
    wl = case.wl
    say(f"[gpu] layout {wl.name}")
    lay = moe.get_layout(torch.from_numpy(case.idx).to(DEV), wl.E, wl.R, wl.capacity)
    for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, name).cpu().numpy(), case.lay[name]), name
    assert int(lay.flags.item()) == case.lay["flags"]


def test_dispatch_parity(case):
    wl = case.wl
    say(f"[gpu] dispatch {wl.name}")
    fp8 = wl.dtype == "fp8"
    rx = torch.full((wl.N, wl.H), case.fill if fp8 else -21555, dtype=torch.uint8 if fp8 else torch.int16,
                    device=DEV)
    if not fp8:
        rx = rx.view(torch.bfloat16)
    rs = torch.full((wl.N, wl.S), -7.0, dtype=torch.float32, device=DEV) if fp8 else None
    moe.dispatch(bf16_to_dev(case.x), torch.from_numpy(case.lay["pos"]).to(DEV), wl.N, wl.dtype, rx, rs)
    got = rx.cpu().numpy() if fp8 else bf16_from_dev(rx)
    assert np.array_equal(got, case.rx)
    if fp8:
        assert np.array_equal(rs.cpu().numpy().view(np.uint32), case.rs.view(np.uint32))


def test_combine_parity(case):
    wl = case.wl
    say(f"[gpu] combine {wl.name}")
    out = moe.combine(bf16_to_dev(case.y), torch.from_numpy(case.lay["pos"]).to(DEV),
                      torch.from_numpy(case.w).to(DEV))
    nbad, maxrel, exact = combine_check(bf16_from_dev(out), case.out, case.y, case.lay["pos"], case.w)
    say(f"   combine {wl.name}: max rel err (|ref|>=1e-2) {maxrel:.3e}, exact fraction {exact:.6f}")
    assert nbad == 0
    assert maxrel <= 1e-2


def test_pipeline_end_to_end(case):
    """route -> layout -> dispatch -> combine entirely on the GPU, as the benchmark runs it."""
    wl = case.wl
    say(f"[gpu] pipeline {wl.name}")
    idx, w = moe.route_topk(torch.from_numpy(case.logits).to(DEV), wl.G, wl.g, wl.k, wl.score)
    lay = moe.get_layout(idx, wl.E, wl.R, wl.capacity)
    rx, rs = moe.dispatch(bf16_to_dev(case.x), lay.pos, lay.num_recv_rows, wl.dtype)
    out = moe.combine(bf16_to_dev(case.y), lay.pos, w)
    torch.cuda.synchronize()
    valid = case.lay["recv_src"] >= 0
    got_rx = rx.cpu().numpy() if wl.dtype == "fp8" else bf16_from_dev(rx)
    assert np.array_equal(got_rx[valid], case.rx[valid])
    if rs is not None:
        assert np.array_equal(rs.cpu().numpy()[valid], case.rs[valid])
    nbad, _, _ = combine_check(bf16_from_dev(out), case.out, case.y, case.lay["pos"], case.w)
    assert nbad == 0


# --------------------------------------------------------------------------
# FP8 conversion: every fp32 pattern of magnitude below 512, both signs
# --------------------------------------------------------------------------
def test_quantize_e4m3_exhaustive():
    import ctypes as C
    import subprocess
    src = os.path.join(HELPERS, "e4m3_check.c")
    so = os.path.join(HELPERS, "libe4m3check.so")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", so, src, "-lm"])
    chk = C.CDLL(so)
    chk.check_codes.restype = C.c_int64
    chk.check_codes.argtypes = [C.c_uint32, C.c_int64, C.c_void_p, C.POINTER(C.c_uint32)]
    chunk = 1 << 27
    first = C.c_uint32()
    total = 0
    for sign in (0, 0x80000000):
        for lo in range(0, 0x44000000, chunk):
            n = min(chunk, 0x44000000 - lo)
            bits = torch.arange(lo, lo + n, dtype=torch.int64, device=DEV) + sign
            bits = torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits).to(torch.int32)
            codes = moe.quantize_e4m3(bits.view(torch.float32)).cpu().numpy()
            bad = chk.check_codes(lo + sign, n, codes.ctypes.data, C.byref(first))
            assert bad == 0, f"first bad pattern {first.value:#x}"
            total += n
    say(f"   quantize sweep: {total} patterns checked")
    # and equal to the oracle's encoder on a random sample, odd length (tail path)
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(-460, 460, 999_999), rng.standard_normal(333) * 1e-3]).astype(np.float32)
    got = moe.quantize_e4m3(torch.from_numpy(y).to(DEV)).cpu().numpy()
    assert np.array_equal(got, oracle.e4m3_from_f32(y))


# --------------------------------------------------------------------------
# edge cases and ragged shapes
# --------------------------------------------------------------------------
RAGGED = [
    # T not a multiple of 4/64/256; H with a partial 512-channel unit; E not a
    # multiple of 64 (general group path); k = 1; one group; many groups
    W.custom("ragged_a", T=77, H=640, E=16, G=4, g=2, k=3, score="sigmoid", R=4, dtype="fp8"),
    W.custom("ragged_b", T=301, H=1152, E=96, G=4, g=2, k=6, score="sigmoid", R=8, dtype="fp8"),
    W.custom("ragged_c", T=513, H=128, E=32, G=1, g=1, k=1, score="sigmoid", R=32, dtype="fp8"),
    W.custom("ragged_d", T=1000, H=264, E=8, G=1, g=1, k=2, score="softmax", R=2, dtype="bf16"),
    W.custom("ragged_e", T=257, H=2048, E=64, G=64, g=8, k=8, score="sigmoid", R=16, dtype="fp8"),
    W.custom("ragged_f", T=65, H=7168, E=256, G=8, g=4, k=8, score="sigmoid", R=32, dtype="fp8",
             capacity=3),
    W.custom("ragged_g", T=200, H=512, E=512, G=16, g=3, k=12, score="sigmoid", R=64, dtype="fp8"),
    W.custom("ragged_h", T=130, H=1024, E=128, G=8, g=2, k=4, score="softmax", R=4, dtype="fp8",
             capacity=40),
]


@pytest.mark.parametrize("wl", RAGGED, ids=lambda w: w.name)
def test_ragged_shapes_all_stages(wl):
    say(f"[gpu] ragged {W.describe(wl)}")
    c = Case(wl)
    idx, w = moe.route_topk(torch.from_numpy(c.logits).to(DEV), wl.G, wl.g, wl.k, wl.score)
    assert np.array_equal(idx.cpu().numpy(), c.idx)
    assert np.array_equal(w.cpu().numpy(), c.w)
    lay = moe.get_layout(idx, wl.E, wl.R, wl.capacity)
    for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, name).cpu().numpy(), c.lay[name]), name
    assert int(lay.flags.item()) == c.lay["flags"]
    fp8 = wl.dtype == "fp8"
    rx = torch.full((wl.N, wl.H), 0xAB if fp8 else -21555, dtype=torch.uint8 if fp8 else torch.int16,
                    device=DEV)
    if not fp8:
        rx = rx.view(torch.bfloat16)
    rs = torch.full((wl.N, wl.S), -7.0, dtype=torch.float32, device=DEV) if fp8 else None
    moe.dispatch(bf16_to_dev(c.x), lay.pos, wl.N, wl.dtype, rx, rs)
    assert np.array_equal(rx.cpu().numpy() if fp8 else bf16_from_dev(rx), c.rx)
    if fp8:
        assert np.array_equal(rs.cpu().numpy(), c.rs)
    out = moe.combine(bf16_to_dev(c.y), lay.pos, w)
    nbad, _, _ = combine_check(bf16_from_dev(out), c.out, c.y, c.lay["pos"], c.w)
    assert nbad == 0


@pytest.mark.parametrize("name", ["tiny", "dsv3_prefill"])
def test_route_tie_heavy(name):
    wl = W.get(name)
    say(f"[gpu] tie-heavy route {name}")
    logits = W.tie_heavy(W.gen_logits(wl))
    logits[0, :] = 0.0
    logits[1, ::2] = -0.0
    logits[2, :] = -100.0          # every sigmoid score exactly 0
    logits[3, :] = 100.0           # every sigmoid score exactly 1
    for score in ("sigmoid", "softmax"):
        for renorm in (True, False):
            ref_i, ref_w = oracle.route(logits, wl.G, wl.g, wl.k, score_fn=oracle.SIGMOID if score == "sigmoid"
                                        else oracle.SOFTMAX, renormalize=renorm)
            idx, w = moe.route_topk(torch.from_numpy(logits).to(DEV), wl.G, wl.g, wl.k, score, renorm)
            assert np.array_equal(idx.cpu().numpy(), ref_i), (score, renorm)
            assert np.array_equal(w.cpu().numpy(), ref_w), (score, renorm)


def test_route_group_topn_override():
    wl = W.get("dsv3_prefill").replace(T=512)
    logits = W.gen_logits(wl)
    for n in (1, 2, 3, 32):
        ref_i, ref_w = oracle.route(logits, wl.G, wl.g, wl.k, group_topn=n)
        idx, w = moe.route_topk(torch.from_numpy(logits).to(DEV), wl.G, wl.g, wl.k, group_topn=n)
        assert np.array_equal(idx.cpu().numpy(), ref_i), n
        assert np.array_equal(w.cpu().numpy(), ref_w), n


# The row-routing kernel (four tokens per wave) serves batches of 2048 tokens
# or more with E in {16, 32, 64, 128, 256}, G dividing 16 and k <= 16; every
# such shape family, both score functions and both weightings, ragged token
# counts and tie-heavy logits, bit for bit against the oracle.
@pytest.mark.parametrize("T,E,G,g,k,n", [
    (2048, 16, 4, 2, 3, 0), (2053, 32, 2, 1, 5, 0), (2100, 64, 16, 4, 16, 0), (4099, 128, 8, 3, 7, 0),
    (2048, 256, 1, 1, 8, 0), (3001, 256, 16, 8, 12, 0), (2050, 256, 8, 4, 8, 3), (2047, 256, 8, 4, 8, 0),
])
@pytest.mark.parametrize("tie", [False, True])
def test_route_rows_shapes(T, E, G, g, k, n, tie):
    wl = W.custom("rows", T=T, H=128, E=E, G=G, g=g, k=k, score="sigmoid", R=1, dtype="fp8", seed=T + E)
    say(f"[gpu] route rows T={T} E={E} G={G} g={g} k={k} n={n} tie={tie}")
    logits = W.gen_logits(wl)
    if tie:
        logits = W.tie_heavy(logits)
        logits[0, :] = 0.0
        logits[1, ::2] = -0.0
        logits[2, :] = -100.0
        logits[3, :] = 100.0
    for score in ("sigmoid", "softmax"):
        for renorm in (True, False):
            ref_i, ref_w = oracle.route(logits, G, g, k, score_fn=oracle.SIGMOID if score == "sigmoid"
                                        else oracle.SOFTMAX, renormalize=renorm, group_topn=n)
            idx, w = moe.route_topk(torch.from_numpy(logits).to(DEV), G, g, k, score, renorm, group_topn=n)
            assert np.array_equal(idx.cpu().numpy(), ref_i), (score, renorm)
            assert np.array_equal(w.cpu().numpy().view(np.uint32), ref_w.view(np.uint32)), (score, renorm)


def test_dispatch_adversarial_rows():
    wl = W.custom("adv", T=64, H=1024, E=16, G=4, g=2, k=2, score="sigmoid", R=4, dtype="fp8")
    say("[gpu] adversarial dispatch rows")
    x = W.gen_x(wl)
    x[0] = 0                                   # all zeros
    x[1] = 0x8000                              # all -0
    x[2, 5] = W.f32_to_bf16_bits(np.float32([3.0e38]))[0]          # one huge value
    x[3] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(x[3]) * np.float32(1e-39))  # bf16 subnormals
    x[4, :128] = np.uint16(0x0001)             # smallest subnormal block
    x[5] = W.f32_to_bf16_bits(np.full(wl.H, 448.0, np.float32))
    x[6] = W.f32_to_bf16_bits(np.linspace(-1, 1, wl.H).astype(np.float32) * np.float32(1e-30))
    pos = np.arange(wl.T * wl.k, dtype=np.int32).reshape(wl.T, wl.k)
    ref_q, ref_s = oracle.dispatch(x, pos, wl.T * wl.k)
    q, s = moe.dispatch(bf16_to_dev(x), torch.from_numpy(pos).to(DEV), wl.T * wl.k)
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def test_out_of_range_positions_are_skipped():
    """pos outside [0, N) never causes an access: dispatch skips, combine adds nothing."""
    say("[gpu] out-of-range positions")
    T, H, k, N = 8, 256, 2, 10
    x = W.f32_to_bf16_bits(np.random.default_rng(1).standard_normal((T, H)).astype(np.float32))
    pos = np.array([[0, -1], [1, 10], [2, 999999], [3, -5], [4, 5], [6, 7], [8, 9], [-1, -1]], np.int32)
    ref_q, ref_s = oracle.dispatch(x, np.where((pos >= 0) & (pos < N), pos, -1), N,
                                   recv_x=np.zeros((N, H), np.uint8), recv_scales=np.zeros((N, 2), np.float32))
    q = torch.zeros((N, H), dtype=torch.uint8, device=DEV)
    s = torch.zeros((N, 2), dtype=torch.float32, device=DEV)
    moe.dispatch(bf16_to_dev(x), torch.from_numpy(pos).to(DEV), N, "fp8", q, s)
    assert np.array_equal(q.cpu().numpy(), ref_q)
    y = W.f32_to_bf16_bits(np.random.default_rng(2).standard_normal((N, H)).astype(np.float32))
    w = np.full((T, k), 0.5, np.float32)
    ref = oracle.combine(y, np.where((pos >= 0) & (pos < N), pos, -1), w)
    out = moe.combine(bf16_to_dev(y), torch.from_numpy(pos).to(DEV), torch.from_numpy(w).to(DEV))
    assert np.array_equal(bf16_from_dev(out), ref)


def test_layout_flags_bad_indices():
    say("[gpu] layout bad indices")
    idx = np.array([[0, 1], [2, 2], [3, 1]], np.int32)
    lay = moe.get_layout(torch.from_numpy(idx).to(DEV), 4, 2)
    assert int(lay.flags.item()) & moe.FLAG_BAD_INDEX
    idx = np.array([[0, 7], [2, -3], [3, 1]], np.int32)
    lay = moe.get_layout(torch.from_numpy(idx).to(DEV), 4, 2, capacity=2)
    assert int(lay.flags.item()) & moe.FLAG_BAD_INDEX
    # large T with one bad index in the last block (multi-block path)
    idx = np.tile(np.array([[0, 1]], np.int32), (2000, 1))
    idx[-1, 1] = 4
    lay = moe.get_layout(torch.from_numpy(idx).to(DEV), 4, 2)
    assert int(lay.flags.item()) == moe.FLAG_BAD_INDEX


@pytest.mark.parametrize("T,E,k,C,kind", [
    (100, 256, 8, 128, "dup"), (100, 256, 8, 128, "range"),  # 128-thread blocks, padded
    (200, 64, 4, 0, "dup"), (200, 64, 4, 0, "range"),        # 256-thread blocks
    (5000, 256, 8, 0, "dup"), (5000, 256, 8, 0, "range"),    # 1024-thread blocks, several iterations
    (5000, 256, 8, 40, "range"),                              # padded, overflowing and bad
    (20000, 16, 2, 0, "dup"),                                 # two-pass kernels
])
def test_layout_flags_bad_indices_every_kernel(T, E, k, C, kind):
    """One repeated or out-of-range index late in the batch raises the flag in
    every layout kernel; every pos the call writes stays in [-1, N)."""
    say(f"[gpu] layout bad index {kind} T={T} E={E} k={k} C={C}")
    idx = random_idx(T, E, k, T + k)
    t = T - 3
    if kind == "dup":
        idx[t, k - 1] = idx[t, 0]
    else:
        idx[t, k // 2] = E + 5
    lay = moe.get_layout(torch.from_numpy(idx).to(DEV), E, 4, C)
    flags = int(lay.flags.item())
    assert flags & moe.FLAG_BAD_INDEX
    N = E * C if C > 0 else T * k
    pos = lay.pos.cpu().numpy()
    assert pos.min() >= -1 and pos.max() < N
    # the clean pairs of the other tokens are placed exactly as the oracle places them
    ok = np.ones(T, bool)
    ok[t] = False
    ref = oracle.layout(np.delete(idx, t, axis=0), E, 4, C)
    if C == 0:
        return  # compact offsets count the bad token's pairs too; only padded rows are token-local
    assert np.array_equal(pos[ok][:t], ref["pos"][:t])


def random_idx(T, E, k, seed):
    """k distinct experts per token: the first k of a seeded random order."""
    return np.argsort(np.random.default_rng(seed).random((T, E)), axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,E,k,R,C", [
    (1, 256, 8, 32, 0),
    (127, 256, 8, 32, 128), (128, 256, 8, 32, 0),    # 128-thread blocks
    (129, 256, 8, 32, 128), (256, 256, 8, 32, 0),    # 256-thread blocks
    (257, 64, 4, 8, 64), (1023, 256, 8, 32, 0), (1025, 64, 4, 8, 0),
    (8192, 16, 2, 4, 0),           # the largest one-launch batch over few experts
    (8193, 64, 2, 8, 0),           # two-pass: above 8192 tokens over at most 64 experts
    (8193, 80, 2, 8, 0),           # one launch again above 64 experts
    (32768, 16, 2, 4, 0),          # two-pass
    (32769, 16, 2, 4, 0),          # above the one-launch limit: two-pass
    (32768, 512, 3, 8, 0),         # general k, the most tokens and experts of the one launch
    (5000, 256, 8, 32, 20),        # padded, overflowing experts
    (32768, 64, 1, 64, 600),       # padded, two-pass, k = 1
    (32768, 128, 1, 64, 300),      # padded at the one-launch limit, k = 1
])
def test_layout_token_limits(T, E, k, R, C):
    say(f"[gpu] layout T={T} E={E} k={k} R={R} C={C}")
    idx = random_idx(T, E, k, T + E)
    ref = oracle.layout(idx, E, R, C)
    lay = moe.get_layout(torch.from_numpy(idx).to(DEV), E, R, C)
    for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, name).cpu().numpy(), ref[name]), name
    assert int(lay.flags.item()) == ref["flags"]


def test_layout_capacity_overflow_multiblock():
    say("[gpu] layout capacity overflow")
    rng = np.random.default_rng(4)
    T, E, k, R, C = 3000, 32, 4, 4, 300
    p = (np.arange(E) + 1.0) ** -1.3
    p /= p.sum()
    idx = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    ref = oracle.layout(idx, E, R, C)
    assert ref["flags"] == 1
    lay = moe.get_layout(torch.from_numpy(idx).to(DEV), E, R, C)
    for name in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, name).cpu().numpy(), ref[name]), name
    assert int(lay.flags.item()) == 1


def test_zero_tokens():
    say("[gpu] zero tokens")
    e = torch.empty((0, 256), dtype=torch.float32, device=DEV)
    idx, w = moe.route_topk(e, 8, 4, 8)
    assert idx.shape == (0, 8)
    lay = moe.get_layout(idx, 256, 32)
    assert int(lay.cnt_e.sum().item()) == 0 and int(lay.off_e[-1].item()) == 0
    assert int(lay.flags.item()) == 0
    lay = moe.get_layout(idx, 256, 32, capacity=4)
    assert bool((lay.recv_src == -1).all().item())
    rx, rs = moe.dispatch(torch.empty((0, 7168), dtype=torch.bfloat16, device=DEV), lay.pos, 0)
    out = moe.combine(torch.empty((0, 7168), dtype=torch.bfloat16, device=DEV), lay.pos, w)
    torch.cuda.synchronize()
    assert out.shape == (0, 7168)


def test_launch_shapes_do_not_change_results():
    wl = W.get("dsv3_prefill").replace(T=300)
    say("[gpu] units_per_wave overrides")
    x = bf16_to_dev(W.gen_x(wl))
    rng = np.random.default_rng(9)
    pos = torch.from_numpy(rng.permutation(wl.T * wl.k).astype(np.int32).reshape(wl.T, wl.k)).to(DEV)
    ref_q, ref_s = moe.dispatch(x, pos, wl.N, units_per_wave=1)
    for u in (2, 7, 14):
        q, s = moe.dispatch(x, pos, wl.N, units_per_wave=u)
        assert torch.equal(q, ref_q) and torch.equal(s, ref_s), u
    y = bf16_to_dev(W.gen_y(wl))
    w = torch.from_numpy(rng.uniform(0, 1, (wl.T, wl.k)).astype(np.float32)).to(DEV)
    ref = moe.combine(y, pos, w, units_per_wave=1)
    for u in (2, 7):
        assert torch.equal(moe.combine(y, pos, w, units_per_wave=u), ref), u


def test_repeat_runs_are_identical():
    wl = W.get("skewed_8k").replace(T=2048)
    say("[gpu] determinism")
    logits = torch.from_numpy(W.gen_logits(wl)).to(DEV)
    x = bf16_to_dev(W.gen_x(wl))
    res = []
    for _ in range(2):
        idx, w = moe.route_topk(logits, wl.G, wl.g, wl.k)
        lay = moe.get_layout(idx, wl.E, wl.R)
        rx, rs = moe.dispatch(x, lay.pos, lay.num_recv_rows)
        res.append((idx.clone(), w.clone(), lay.pos.clone(), rx.clone(), rs.clone()))
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_stream_ordering_on_side_stream():
    """Calls honour the caller's stream: work on a side stream, then wait on it."""
    wl = W.get("tiny")
    say("[gpu] side stream")
    s = torch.cuda.Stream()
    logits = torch.from_numpy(W.gen_logits(wl)).to(DEV)
    ref_i, ref_w = oracle.route(W.gen_logits(wl), wl.G, wl.g, wl.k)
    with torch.cuda.stream(s):
        idx, w = moe.route_topk(logits, wl.G, wl.g, wl.k)
        lay = moe.get_layout(idx, wl.E, wl.R)
    torch.cuda.current_stream().wait_stream(s)
    assert np.array_equal(idx.cpu().numpy(), ref_i)
    assert np.array_equal(lay.cnt_e.cpu().numpy(), np.bincount(ref_i.ravel(), minlength=wl.E))


# --------------------------------------------------------------------------
# grouped-GEMM-friendly variants: aligned expert regions, power-of-two scales
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,T,A", [("dsv3_prefill", 4096, 128), ("dsv3_prefill", 4096, 64),
                                      ("dsv3_prefill", 200, 8), ("mixtral", 16384, 256), ("tiny", 64, 4)])
def test_layout_aligned_parity(name, T, A):
    wl = W.get(name).replace(T=T)
    say(f"[gpu] aligned layout {name} T={T} A={A}")
    idx, _ = oracle.route(W.gen_logits(wl), wl.G, wl.g, wl.k, score_fn=sf(wl))
    ref = oracle.layout(idx, wl.E, wl.R, align=A)
    lay = moe.get_layout(torch.from_numpy(idx).to(DEV), wl.E, wl.R, align_rows=A)
    for n in ("cnt_e", "cnt_r", "off_e", "off_r", "pos", "recv_src"):
        assert np.array_equal(getattr(lay, n).cpu().numpy(), ref[n]), n
    assert int(lay.flags.item()) == 0


@pytest.mark.parametrize("name", ["dsv3_prefill", "tiny", "skewed_8k"])
def test_dispatch_pow2_parity(name):
    wl = W.get(name)
    say(f"[gpu] pow2 dispatch {name}")
    x = W.gen_x(wl)
    x[0] = 0
    x[1, :128] = W.f32_to_bf16_bits(np.full(128, 448.0, np.float32))
    x[2, :128] = W.f32_to_bf16_bits(np.full(128, 450.0, np.float32))
    x[3] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(x[3]) * np.float32(3e38 / 5))
    x[4] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(x[4]) * np.float32(1e-38))
    idx, _ = oracle.route(W.gen_logits(wl), wl.G, wl.g, wl.k)
    lay = oracle.layout(idx, wl.E, wl.R, wl.capacity)
    ref_q, ref_s = oracle.dispatch(x, lay["pos"], wl.N, oracle.FP8_POW2)
    q, s = moe.dispatch(bf16_to_dev(x), torch.from_numpy(lay["pos"]).to(DEV), wl.N, "fp8_pow2",
                        torch.zeros((wl.N, wl.H), dtype=torch.uint8, device=DEV),
                        torch.zeros((wl.N, wl.S), dtype=torch.float32, device=DEV))
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


@pytest.mark.parametrize("name", ["dsv3_prefill", "tiny", "ll_decode", "skewed_8k"])
def test_dispatch_ue8m0_parity(name):
    """One-byte E8M0 scales: codes and scale bytes bit-exact, rows no pair
    addresses (padded layout) untouched, at the full shapes in the library's
    launch configuration."""
    wl = W.get(name)
    say(f"[gpu] ue8m0 dispatch {name}")
    x = W.gen_x(wl)
    x[0] = 0
    x[1, :128] = W.f32_to_bf16_bits(np.full(128, 448.0, np.float32))
    x[2, :128] = W.f32_to_bf16_bits(np.full(128, 450.0, np.float32))
    x[3] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(x[3]) * np.float32(3e38 / 5))
    x[4] = W.f32_to_bf16_bits(W.bf16_bits_to_f32(x[4]) * np.float32(1e-38))
    idx, _ = oracle.route(W.gen_logits(wl), wl.G, wl.g, wl.k)
    lay = oracle.layout(idx, wl.E, wl.R, wl.capacity)
    ref_q, ref_s = oracle.dispatch(x, lay["pos"], wl.N, oracle.FP8_UE8M0,
                                   np.full((wl.N, wl.H), 0xCD, np.uint8), np.full((wl.N, wl.S), 0xEE, np.uint8))
    q, s = moe.dispatch(bf16_to_dev(x), torch.from_numpy(lay["pos"]).to(DEV), wl.N, "fp8_ue8m0",
                        torch.full((wl.N, wl.H), 0xCD, dtype=torch.uint8, device=DEV),
                        torch.full((wl.N, wl.S), 0xEE, dtype=torch.uint8, device=DEV))
    assert s.dtype == torch.uint8
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy(), ref_s)
