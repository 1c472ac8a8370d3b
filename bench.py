"""Benchmark of the MoE dispatch/combine hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
route (group-limited top-k) -> layout -> FP8 dispatch -> BF16 combine, on the
DeepSeek-V3-shaped prefill workload (4096 tokens x hidden 7168, 256 experts in
8 groups, top-4 groups then top-8 experts, 32 virtual ranks).  The expert MLP
is not on this path: the combine reads synthetic expert outputs y [T*k, H].

Inputs sit in HBM before the timed region; two input sets alternate between
steps so no input is re-read from the 256 MB last-level cache.  Before the
timed region the GPU is held by a short spin kernel while all K steps are
enqueued, so the timeline holds only GPU work.  A third pass of K steps, each
preceded by a 1 GiB scratch read, reports the same stages with cold caches.
For batches of at most 1024 tokens a fourth pass times the step with route,
layout and dispatch in one launch (moe_route_dispatch), and both decode steps
are also timed captured in a HIP graph and submitted one by one from the
host with the GPU not held (where the per-call host cost sets the pace).  HIP
events on the launch stream (created without the system-scope fence) bracket
every stage of every timed step; a second pass of K steps without them gives
the step time free of their cost.

Prints one JSON line.  ``value`` is the effective HBM bandwidth of dispatch +
combine: their algorithmic bytes over their measured time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
METRIC = "dispatch+combine µs and effective HBM GB/s (% of peak), 4096 tok×7168 top-8"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=0, help="oracle repetitions (0: about 10 s)")
    ap.add_argument("--direction", choices=["forward", "backward"], default="forward",
                    help="backward: time combine_backward -> dispatch_backward instead")
    ap.add_argument("--layer-tokens", type=int, default=16384,
                    help="tokens of the --stage layer workload (512 gives a decode-sized batch)")
    ap.add_argument("--stage", choices=["dispatch_combine", "mlp", "layer"], default="dispatch_combine",
                    help="mlp: time the expert MLP (up + SwiGLU + FP8 requantisation, down) instead")
    ap.add_argument("--mlp-workload", default="mlp_rank", choices=sorted(W.MLP_WORKLOADS))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also time a plain 1 GiB device copy (reference for counters and peak)")
    args = ap.parse_args()
    # 2 receive rows per token x 7168 bytes must stay within the expert MLP's 32-bit row offsets
    if not 1 <= args.layer_tokens <= 262144:
        ap.error(f"--layer-tokens must be in [1, 262144], got {args.layer_tokens}")
    return args


class HipEvents:
    """HIP events created with hipEventDisableSystemFence, from the HIP runtime
    already loaded in this process (the one torch and the library share).
    Recording one costs about 1.5 us of GPU time between kernels, against about
    5.5 us for a default event, whose system-scope release fence flushes."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        L = ctypes.CDLL(path)
        L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L = L

    def create(self, n):
        evs = []
        for _ in range(n):
            e = self.ct.c_void_p()
            if self.L.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            evs.append(e)
        return evs

    def record(self, ev, stream):
        if self.L.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        f = self.ct.c_float()
        if self.L.hipEventElapsedTime(self.ct.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "combine_group_limited_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, digest: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json),
    only for the workload they were taken on and while the kernel's sources are
    unchanged since the measurement."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        data = json.load(f)
    ent = data.get(kernel)
    if not ent or ent.get("source_digest") != digest or ent.get("workload") != workload:
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(wl, reps: int):
    """The oracle (plain single-threaded C) on the same workload, timed on the host."""
    import oracle
    x, logits, y = W.gen_x(wl), W.gen_logits(wl), W.gen_y(wl)
    t_dc = 0.0
    n = 0
    t_start = time.perf_counter()
    while True:
        idx, w = oracle.route(logits, wl.G, wl.g, wl.k,
                              score_fn=oracle.SOFTMAX if wl.score == "softmax" else oracle.SIGMOID)
        lay = oracle.layout(idx, wl.E, wl.R, wl.capacity)
        t0 = time.perf_counter()
        oracle.dispatch(x, lay["pos"], wl.N, oracle.FP8 if wl.dtype == "fp8" else oracle.BF16)
        oracle.combine(y, lay["pos"], w)
        t_dc += time.perf_counter() - t0
        n += 1
        if (reps and n >= reps) or (not reps and time.perf_counter() - t_start >= 10.0):
            break
    b = W.algorithmic_bytes(wl)
    gbps = (b["dispatch"] + b["combine"]) * n / t_dc / 1e9
    res = {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{n} full passes of the {wl.name} workload ({wl.T} tokens) through the oracle; "
                     f"dispatch+combine {t_dc / n * 1e3:.1f} ms per pass, single thread",
           "dispatch_plus_combine_ms": round(t_dc / n * 1e3, 3)}
    res["all_cores"] = cpu_baseline_all_cores(wl, x, y, idx, w, lay, b)
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_all_cores(wl, x, y, idx, w, lay, b, passes: int = 3):
    """The same oracle calls split over contiguous token ranges on a thread pool
    (the C oracle releases the GIL): every range writes its own receive rows and
    output tokens, so the result is the single-threaded one bit for bit."""
    import concurrent.futures
    import oracle
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    nt = max(1, min(16, cores))
    dt = oracle.FP8 if wl.dtype == "fp8" else oracle.BF16
    pos = lay["pos"]
    cuts = np.linspace(0, wl.T, nt + 1).astype(int)
    ranges = [(int(a), int(c)) for a, c in zip(cuts[:-1], cuts[1:]) if c > a]
    ref_rx, ref_rs = oracle.dispatch(x, pos, wl.N, dt)
    ref_out = oracle.combine(y, pos, w)
    best = None
    with concurrent.futures.ThreadPoolExecutor(nt) as ex:
        for _ in range(passes):
            rx = np.zeros_like(ref_rx)
            rs = np.zeros_like(ref_rs) if ref_rs is not None else None
            t0 = time.perf_counter()
            list(ex.map(lambda r: oracle.dispatch(x[r[0]:r[1]], pos[r[0]:r[1]], wl.N, dt, rx, rs), ranges))
            outs = list(ex.map(lambda r: oracle.combine(y, pos[r[0]:r[1]], w[r[0]:r[1]]), ranges))
            t = time.perf_counter() - t0
            best = t if best is None else min(best, t)
    same = (np.array_equal(rx, ref_rx) and (rs is None or np.array_equal(rs.view(np.uint32), ref_rs.view(np.uint32)))
            and np.array_equal(np.concatenate(outs), ref_out))
    return {"value": round((b["dispatch"] + b["combine"]) / best / 1e9, 4), "unit": "GB/s", "cores": nt,
            "host_cores": cores, "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"best of {passes} full passes, dispatch+combine over {len(ranges)} token ranges on "
                      f"{nt} threads: {best * 1e3:.1f} ms per pass",
            "bit_identical_to_single_thread": bool(same)}


def backward_main(args, wl, moe, torch, dev, sets, hev, stream):
    """The backward pair on the routing of the first input set: combine's
    backward (grad_out -> grad_y, grad_w) then dispatch's backward
    (grad_recv = grad_y, identity experts -> grad_x)."""
    idx, w = moe.route_topk(sets[0][1], wl.G, wl.g, wl.k, wl.score)
    lay = moe.get_layout(idx, wl.E, wl.R, wl.capacity)
    N = lay.num_recv_rows
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 2000)
    gouts = [torch.randn((wl.T, wl.H), generator=g, device=dev).to(torch.bfloat16) for _ in range(2)]
    grad_y = torch.empty((N, wl.H), dtype=torch.bfloat16, device=dev)
    grad_w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
    grad_x = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    def step(i, ev=None):
        y = sets[i % 2][2]
        if ev: hev.record(ev[0], stream)
        moe.combine_backward(gouts[i % 2], y, lay.pos, w, grad_y, grad_w)
        if ev: hev.record(ev[1], stream)
        moe.dispatch_backward(grad_y, lay.pos, grad_x)
        if ev: hev.record(ev[2], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    evs = [hev.create(3) for _ in range(K)]
    start, end = hev.create(2)
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(2e7))
    hev.record(start, stream)
    for i in range(K):
        step(i, evs[i])
    hev.record(end, stream)
    torch.cuda.synchronize()
    st = np.array([[hev.ms(e[q], e[q + 1]) for q in range(2)] for e in evs]) * 1e3
    cb_us, db_us = (float(v) for v in st.mean(0))
    b = W.algorithmic_bytes(wl)
    tot = b["combine_backward"] + b["dispatch_backward"]
    res = {
        "metric": "combine_backward+dispatch_backward effective HBM GB/s, " + wl.name,
        "value": round(tot / ((cb_us + db_us) * 1e-6) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(hev.ms(start, end) / K, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 gradients (fp32 arithmetic)",
        "data": "synthetic (seeded N(0,1) bf16 gradients and expert outputs)",
        "config": {"workload": W.describe(wl), "direction": "backward"},
        "combine_backward_us": round(cb_us, 2), "dispatch_backward_us": round(db_us, 2),
        "combine_backward_gbps": round(b["combine_backward"] / (cb_us * 1e-6) / 1e9, 1),
        "dispatch_backward_gbps": round(b["dispatch_backward"] / (db_us * 1e-6) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * tot / ((cb_us + db_us) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
    }
    # the dominant kernel is combine's backward (gather y, write grad_y)
    achieved = b["combine_backward"] / (cb_us * 1e-6) / 1e9
    digest = source_digest("backward.hip", "moe_device.hpp")
    res["roofline"] = {"kernel": "combine_backward", "bound": "hbm", "achieved": round(achieved, 1),
                       "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                       "traffic": load_traffic("combine_backward", digest, wl.name),
                       "algorithmic_bytes": b["combine_backward"], "avg_launch_us": round(cb_us, 2),
                       "source_digest": digest}
    print(json.dumps(res), flush=True)


FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix peak, published


def mlp_cpu_baseline(wl, x, xs, w1, w1s, w2, w2s, start, count, rows: int = 4):
    """The oracle's expert MLP on a sample of rows (plain single-threaded C)."""
    import oracle
    sel = np.array([start[e] + count[e] // 2 for e in range(min(rows, wl.E)) if count[e] > 0], np.int32)
    t0 = time.perf_counter()
    act, act_s, _ = oracle.mlp_up(x, xs, w1, w1s, start, count, rows=sel)
    oracle.mlp_down(act, act_s, w2, w2s, start, count, rows=sel)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(sel) * (2 * wl.I * wl.H + wl.H * wl.I)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(sel)} receive rows (one per expert) through the oracle's up and down "
                      f"projections, {dt:.1f} s, single thread"}


def layer_main(args, torch, moe, hev, dev):
    """The MoE layer after routing on one rank's shape (--layer-tokens tokens,
    16384 by default, x 7168, top-2 of 8 experts, I 2048; 2 receive rows per
    token): moe_layer_forward (one launch) against the four calls
    moe_dispatch -> moe_expert_up -> moe_expert_down -> moe_combine on the
    same inputs."""
    T, H, I, E, k = args.layer_tokens, 7168, 2048, 8, 2
    wl = W.custom("layer_rank", T=T, H=H, E=E, G=1, g=1, k=k, score="sigmoid", R=E, dtype="fp8")
    mw = W.MlpWorkload("layer_rank_mlp", N=1, H=H, I=I, E=E, seed=7)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x = torch.from_numpy(W.gen_x(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    idx, w = moe.route_topk(d(W.gen_logits(wl)), 1, 1, k)
    lay = moe.get_layout(idx, E, E)
    N = lay.num_recv_rows
    w1h, w1sh = W.gen_mlp_weights(mw, "w1")
    w2h, w2sh = W.gen_mlp_weights(mw, "w2")
    w1, w1s, w2, w2s = map(d, (w1h, w1sh, w2h, w2sh))
    rx = torch.empty((N, H), dtype=torch.uint8, device=dev)
    rs = torch.empty((N, H // 128), dtype=torch.float32, device=dev)
    act = torch.empty((N, I), dtype=torch.uint8, device=dev)
    act_s = torch.empty((N, I // 128), dtype=torch.float32, device=dev)
    y = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    bufs = (rx, rs, act, act_s, y)
    ws = moe.layer_workspace(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def four(ev=None):
        if ev: hev.record(ev[0], stream)
        moe.dispatch(x, lay.pos, N, "fp8_pow2", rx, rs)
        if ev: hev.record(ev[1], stream)
        moe.expert_up(rx, rs, w1, w1s, lay.cnt_e, lay.off_e, 0, act, act_s)
        if ev: hev.record(ev[2], stream)
        moe.expert_down(act, act_s, w2, w2s, lay.cnt_e, lay.off_e, 0, y)
        if ev: hev.record(ev[3], stream)
        moe.combine(y, lay.pos, w, out)
        if ev: hev.record(ev[4], stream)

    def one():
        moe.layer_forward(x, lay.pos, w, lay.cnt_e, lay.off_e, w1, w1s, w2, w2s, N, 0, workspace=ws, out=out,
                          buffers=bufs)

    def timed(f, K, nev):
        evs = [hev.create(nev) for _ in range(K)] if nev else None
        s0, s1 = hev.create(2)
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(2e7))
        hev.record(s0, stream)
        for i in range(K):
            f(evs[i]) if nev else f()
        hev.record(s1, stream)
        torch.cuda.synchronize()
        return hev.ms(s0, s1) / K * 1e3, evs

    for _ in range(args.warmup):
        four()
        one()
    torch.cuda.synchronize()
    K = args.steps
    four_us, evs = timed(four, K, 5)
    st = np.array([[hev.ms(e[q], e[q + 1]) for q in range(4)] for e in evs]) * 1e3
    four_nev_us, _ = timed(lambda: four(), K, 0)
    one_us, _ = timed(one, K, 0)
    flops = 2.0 * N * 3 * I * H
    words = ws.view(torch.int32).cpu().numpy()
    ticks = ws.view(torch.int64).cpu().numpy()[384:388].astype(np.float64)  # last call, 100 MHz
    phase_us = np.diff(ticks) / 100.0
    res = {
        "metric": "MoE layer after routing (dispatch + expert up + expert down + combine), us per layer",
        "value": round(one_us, 1), "unit": "us", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(one_us / 1e3, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 e4m3 GEMMs (fp32 accumulate), bf16 combine",
        "data": "synthetic bf16 tokens, N(0,1) router logits, FP8 weights with power-of-two block scales",
        "config": {"workload": f"one rank's layer: T={T} H={H} I={I} E={E} top-{k}", "rows": N,
                   "parallelism": "single GPU"},
        "one_launch_us": round(one_us, 1),
        "four_launches_us": round(four_nev_us, 1),
        "four_launches_stage_us": {n: round(float(v), 1) for n, v in
                                   zip(("dispatch", "up", "down", "combine"), st.mean(0))},
        "layer_tflops_one_launch": round(flops / (one_us * 1e-6) / 1e12, 1),
        "one_launch_phase_us_block0": {n: round(float(v), 1) for n, v in
                                       zip(("dispatch", "up", "down"), phase_us)},
        "barrier_workspace_at_rest": bool(words[0] == 0 and words[2] == 0),
    }
    print(json.dumps(res), flush=True)


def mlp_main(args, torch, moe, hev, dev):
    """The expert MLP between dispatch and combine on one rank's receive
    buffer: moe_expert_up (first layer, SwiGLU, FP8 requantisation) then
    moe_expert_down (second layer to bf16)."""
    wl = W.MLP_WORKLOADS[args.mlp_workload]
    start, count, _ = W.mlp_ranges(wl)
    xh, xsh = W.gen_mlp_x(wl)
    w1h, w1sh = W.gen_mlp_weights(wl, "w1")
    w2h, w2sh = W.gen_mlp_weights(wl, "w2")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, xs, w1, w1s, w2, w2s = map(d, (xh, xsh, w1h, w1sh, w2h, w2sh))
    off = np.zeros(wl.E + 1, np.int32)
    off[:wl.E] = start
    off[wl.E] = start[-1] + count[-1]
    cnt, off_d = d(count.astype(np.int32)), d(off)
    act = torch.empty((wl.N, wl.I), dtype=torch.uint8, device=dev)
    act_s = torch.empty((wl.N, wl.I // 128), dtype=torch.float32, device=dev)
    y = torch.empty((wl.N, wl.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(ev=None):
        if ev: hev.record(ev[0], stream)
        moe.expert_up(x, xs, w1, w1s, cnt, off_d, 0, act, act_s)
        if ev: hev.record(ev[1], stream)
        moe.expert_down(act, act_s, w2, w2s, cnt, off_d, 0, y)
        if ev: hev.record(ev[2], stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [hev.create(3) for _ in range(K)]
    start_ev, end_ev = hev.create(2)
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(2e7))
    hev.record(start_ev, stream)
    for i in range(K):
        step(evs[i])
    hev.record(end_ev, stream)
    torch.cuda.synchronize()
    st = np.array([[hev.ms(e[q], e[q + 1]) for q in range(2)] for e in evs]) * 1e3
    up_us, down_us = (float(v) for v in st.mean(0))
    rows = int(count.sum())
    f_up = 2.0 * rows * 2 * wl.I * wl.H
    f_down = 2.0 * rows * wl.H * wl.I
    tf_up = f_up / (up_us * 1e-6) / 1e12
    tf_down = f_down / (down_us * 1e-6) / 1e12
    value = (f_up + f_down) / ((up_us + down_us) * 1e-6) / 1e12
    dom = "up" if up_us >= down_us else "down"
    ach = tf_up if dom == "up" else tf_down
    digest = source_digest("mlp.hip", "mlp_impl.hpp", "moe_device.hpp")
    res = {
        "metric": "expert MLP TFLOP/s (FP8 up + SwiGLU + FP8 requantisation, FP8 down to bf16)",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(hev.ms(start_ev, end_ev) / K, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 e4m3 (fp32 accumulate)",
        "data": "synthetic FP8 codes with power-of-two block scales, multinomial rows per expert",
        "config": {"workload": f"{wl.name}: N={wl.N} H={wl.H} I={wl.I} E={wl.E}", "rows": rows,
                   "parallelism": "single GPU"},
        "up_us": round(up_us, 1), "down_us": round(down_us, 1),
        "up_tflops": round(tf_up, 1), "down_tflops": round(tf_down, 1),
        "roofline": {"kernel": f"mlp_kernel<{'true' if dom == 'up' else 'false'}> ({dom})", "bound": "mfma",
                     "achieved": round(ach, 1), "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / FP8_MFMA_PEAK_TFLOPS, 4),
                     "traffic": load_traffic("mlp_" + dom, digest, wl.name),
                     "algorithmic_flops": f_up if dom == "up" else f_down,
                     "avg_launch_us": round(up_us if dom == "up" else down_us, 1), "source_digest": digest},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = mlp_cpu_baseline(wl, xh, xsh, w1h, w1sh, w2h, w2sh, start, count)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "inter-GPU transport; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_group_limited_amd as moe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.stage == "layer":
        return layer_main(args, torch, moe, HipEvents(), dev)
    if args.stage == "mlp":
        return mlp_main(args, torch, moe, HipEvents(), dev)
    wl = W.get(args.workload)
    fp8 = wl.dtype == "fp8"

    # ---- inputs (two sets), outputs and workspace, all resident in HBM ----
    sets = []
    x0 = torch.from_numpy(W.gen_x(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    l0 = torch.from_numpy(W.gen_logits(wl)).to(dev)
    y0 = torch.from_numpy(W.gen_y(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    sets.append((x0, l0, y0))
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 1000)
    x1 = torch.randn(x0.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    l1 = torch.randn(l0.shape, generator=g, device=dev, dtype=torch.float32)
    if wl.skew:
        l1 += torch.from_numpy(W.zipf_bias(wl)).to(dev)[None, :]
    y1 = torch.randn(y0.shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    sets.append((x1, l1, y1))

    idx = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
    wts = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev)
    lay_out = moe.alloc_layout(wl.T, wl.E, wl.k, wl.R, wl.capacity, dev)
    N = lay_out[0].num_recv_rows
    recv_x = torch.empty((N, wl.H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    recv_s = torch.empty((N, wl.S), dtype=torch.float32, device=dev) if fp8 else None
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)

    hev = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(i, ev=None):
        x, logits, y = sets[i % 2]
        if ev: hev.record(ev[0], stream)
        moe.route_topk(logits, wl.G, wl.g, wl.k, wl.score, out=(idx, wts))
        if ev: hev.record(ev[1], stream)
        lay = moe.get_layout(idx, wl.E, wl.R, wl.capacity, out=lay_out)
        if ev: hev.record(ev[2], stream)
        moe.dispatch(x, lay.pos, N, wl.dtype, recv_x, recv_s)
        if ev: hev.record(ev[3], stream)
        moe.combine(y, lay.pos, wts, out)
        if ev: hev.record(ev[4], stream)

    if args.direction == "backward":
        return backward_main(args, wl, moe, torch, dev, sets, hev, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    evs = [hev.create(5) for _ in range(K)]
    start, end = hev.create(2)
    # timed region: K steps, every stage bracketed by events on the launch stream
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(2e7))    # hold the GPU while the host enqueues the K steps
    t_wall = time.perf_counter()
    hev.record(start, stream)
    for i in range(K):
        step(i, evs[i])
    hev.record(end, stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall

    # the same K steps without stage events (the events' own cost excluded)
    start2, end2 = hev.create(2)
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(2e7))
    hev.record(start2, stream)
    for i in range(K):
        step(i)
    hev.record(end2, stream)
    torch.cuda.synchronize()
    ms_step_plain = hev.ms(start2, end2) / K

    # dispatch -> combine back to back: one event pair around the two kernels,
    # none between them (route and layout run first, outside the pair)
    evs_b2b = [hev.create(2) for _ in range(K)]

    def step_b2b(i, ev):
        x, logits, y = sets[i % 2]
        moe.route_topk(logits, wl.G, wl.g, wl.k, wl.score, out=(idx, wts))
        lay = moe.get_layout(idx, wl.E, wl.R, wl.capacity, out=lay_out)
        hev.record(ev[0], stream)
        moe.dispatch(x, lay.pos, N, wl.dtype, recv_x, recv_s)
        moe.combine(y, lay.pos, wts, out)
        hev.record(ev[1], stream)

    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(2e7))
    for i in range(K):
        step_b2b(i, evs_b2b[i])
    torch.cuda.synchronize()
    b2b_us = np.array([hev.ms(e[0], e[1]) for e in evs_b2b]) * 1e3

    # cold-cache pass: before every step, outside its stage events, a 1 GiB
    # scratch read evicts everything from the L2s and the 256 MB last-level
    # cache (a read, not a write, so no dirty flush lines are left behind for
    # the step's own stores to write back)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sum = torch.empty((), dtype=torch.float32, device=dev)
    evs_cold = [hev.create(5) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        torch.sum(flush, dim=0, out=flush_sum)
        step(i, evs_cold[i])
    torch.cuda.synchronize()
    cold = np.array([[hev.ms(e[q], e[q + 1]) for q in range(4)] for e in evs_cold]) * 1e3  # us

    # write-back included: dispatch -> combine followed, inside the same event
    # pair, by the 1 GiB read, which evicts the dirty receive rows and output
    # from the last-level cache (so their write-back to HBM lands inside the
    # pair); minus the same read timed after a clean read
    evs_wb = [hev.create(2) for _ in range(K)]
    evs_rd = [hev.create(2) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        x, logits, y = sets[i % 2]
        torch.sum(flush, dim=0, out=flush_sum)
        moe.route_topk(logits, wl.G, wl.g, wl.k, wl.score, out=(idx, wts))
        lay = moe.get_layout(idx, wl.E, wl.R, wl.capacity, out=lay_out)
        hev.record(evs_wb[i][0], stream)
        moe.dispatch(x, lay.pos, N, wl.dtype, recv_x, recv_s)
        moe.combine(y, lay.pos, wts, out)
        torch.sum(flush, dim=0, out=flush_sum)
        hev.record(evs_wb[i][1], stream)
        torch.sum(flush, dim=0, out=flush_sum)
        hev.record(evs_rd[i][0], stream)
        torch.sum(flush, dim=0, out=flush_sum)
        hev.record(evs_rd[i][1], stream)
    torch.cuda.synchronize()
    del flush
    wb_us = np.array([hev.ms(e[0], e[1]) for e in evs_wb]) * 1e3
    rd_us = np.array([hev.ms(e[0], e[1]) for e in evs_rd]) * 1e3

    ms_step = hev.ms(start, end) / K
    stage = np.array([[hev.ms(e[q], e[q + 1]) for q in range(4)] for e in evs])  # ms
    st_mean = stage.mean(0) * 1e3   # us
    route_us, layout_us, disp_us, comb_us = (float(v) for v in st_mean)

    b = W.algorithmic_bytes(wl)
    dc_bytes = b["dispatch"] + b["combine"]
    dc_us = disp_us + comb_us
    value = dc_bytes / (dc_us * 1e-6) / 1e9

    kernels = {"dispatch": (disp_us, b["dispatch"], ("dispatch.hip", "dispatch_impl.hpp", "moe_device.hpp")),
               "combine": (comb_us, b["combine"], ("combine.hip", "combine_impl.hpp", "moe_device.hpp"))}
    dom = max(kernels, key=lambda k: kernels[k][0])
    dom_us, dom_bytes, dom_src = kernels[dom]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    digest = source_digest(*dom_src)
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(dom, digest, wl.name), "algorithmic_bytes": dom_bytes,
            "avg_launch_us": round(dom_us, 2), "source_digest": digest}

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8-e4m3 dispatch" if fp8 else "bf16 dispatch") + ", bf16 combine (fp32 arithmetic)",
        "data": "synthetic (seeded N(0,1) bf16 tokens and expert outputs, N(0,1) fp32 router logits)",
        "config": {"workload": W.describe(wl), "tokens": wl.T, "hidden": wl.H, "experts": wl.E,
                   "groups": wl.G, "topk_group": wl.g, "topk": wl.k, "virtual_ranks": wl.R,
                   "dispatch": "fp8 e4m3 1x128" if fp8 else "bf16",
                   "combine": "bf16 (fp32 accumulate)", "parallelism": "single GPU"},
        "dispatch_us": round(disp_us, 2),
        "combine_us": round(comb_us, 2),
        "dispatch_plus_combine_us": round(dc_us, 2),
        "route_us": round(route_us, 2),
        "layout_us": round(layout_us, 2),
        "dispatch_gbps": round(b["dispatch"] / (disp_us * 1e-6) / 1e9, 1),
        "combine_gbps": round(b["combine"] / (comb_us * 1e-6) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "step_effective_gbps": round(b["total"] / (ms_step * 1e-3) / 1e9, 1),
        "ms_per_step_without_stage_events": round(ms_step_plain, 4),
        "p10_p90_dispatch_plus_combine_us": [round(float(v), 2) for v in np.percentile(
            (stage[:, 2] + stage[:, 3]) * 1e3, [10, 90])],
        "median_dispatch_plus_combine_us": round(float(np.median(stage[:, 2] + stage[:, 3])) * 1e3, 2),
        "wall_s_timed_region": round(t_wall, 4),
        "roofline": roof,
        "back_to_back": {
            "dispatch_plus_combine_us": round(float(b2b_us.mean()), 2),
            "median_us": round(float(np.median(b2b_us)), 2),
            "gbps": round(dc_bytes / (float(b2b_us.mean()) * 1e-6) / 1e9, 1),
            "note": "one event pair around dispatch and combine, no event between them",
        },
        "with_write_back": {
            "dispatch_plus_combine_us": round(float((wb_us - rd_us).mean()), 2),
            "gbps": round(dc_bytes / (float((wb_us - rd_us).mean()) * 1e-6) / 1e9, 1),
            "pair_plus_read_us": round(float(wb_us.mean()), 2),
            "clean_read_us": round(float(rd_us.mean()), 2),
            "note": "dispatch, combine and a 1 GiB read inside one event pair (the read evicts the dirty "
                    "receive rows and outputs, so their write-back is inside), minus the same read after "
                    "a clean read",
        },
        "cold_cache": {
            "dispatch_us": round(float(cold[:, 2].mean()), 2),
            "combine_us": round(float(cold[:, 3].mean()), 2),
            "dispatch_plus_combine_us": round(float((cold[:, 2] + cold[:, 3]).mean()), 2),
            "median_dispatch_plus_combine_us": round(float(np.median(cold[:, 2] + cold[:, 3])), 2),
            "p10_p90_dispatch_plus_combine_us": [round(float(v), 2) for v in np.percentile(
                cold[:, 2] + cold[:, 3], [10, 90])],
            "gbps": round(dc_bytes / (float((cold[:, 2] + cold[:, 3]).mean()) * 1e-6) / 1e9, 1),
            "route_us": round(float(cold[:, 0].mean()), 2),
            "layout_us": round(float(cold[:, 1].mean()), 2),
            "note": "each step preceded by a 1 GiB scratch read outside its events",
        },
    }

    # decode-sized batches: the same step with route + layout + dispatch in one
    # launch (moe_route_dispatch), then the combine
    if wl.T <= 1024:
        try:
            f_out = (idx, wts, lay_out[0], recv_x, recv_s)

            def fstep(i, ev=None):
                x, logits, y = sets[i % 2]
                if ev: hev.record(ev[0], stream)
                moe.route_dispatch(logits, x, wl.G, wl.g, wl.k, wl.R, wl.capacity, wl.dtype, wl.score,
                                   out=f_out)
                if ev: hev.record(ev[1], stream)
                moe.combine(y, lay_out[0].pos, wts, out)
                if ev: hev.record(ev[2], stream)

            for i in range(args.warmup):
                fstep(i)
            fevs = [hev.create(3) for _ in range(K)]
            torch.cuda.synchronize()
            if hasattr(torch.cuda, "_sleep"):
                torch.cuda._sleep(int(2e7))
            for i in range(K):
                fstep(i, fevs[i])
            fs, fe = hev.create(2)
            if hasattr(torch.cuda, "_sleep"):
                torch.cuda._sleep(int(2e7))
            hev.record(fs, stream)
            for i in range(K):
                fstep(i)
            hev.record(fe, stream)
            torch.cuda.synchronize()
            fst = np.array([[hev.ms(e[q], e[q + 1]) for q in range(2)] for e in fevs]) * 1e3
            res["one_launch_decode"] = {
                "route_layout_dispatch_us": round(float(fst[:, 0].mean()), 2),
                "combine_us": round(float(fst[:, 1].mean()), 2),
                "ms_per_step_without_stage_events": round(hev.ms(fs, fe) / K, 4),
                "separate_route_layout_dispatch_us": round(route_us + layout_us + disp_us, 2),
            }
            # both decode steps captured in a HIP graph and replayed K times
            # (inputs of set 0; the graph holds only this library's kernels)
            for name, fn in (("graph_step_us_separate", lambda: step(0)), ("graph_step_us_one_launch",
                                                                           lambda: fstep(0))):
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    fn()
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    fn()
                graph.replay()
                torch.cuda.synchronize()
                gs, ge = hev.create(2)
                hev.record(gs, stream)
                for _ in range(K):
                    graph.replay()
                hev.record(ge, stream)
                torch.cuda.synchronize()
                res["one_launch_decode"][name] = round(hev.ms(gs, ge) / K * 1e3, 2)
                del graph
            # host-driven loop: K steps submitted one after another from Python
            # with the GPU not held, wall clock to the final synchronise; the
            # per-call host cost of the binding then sets the pace
            for name, fn in (("host_loop_step_us_separate", step), ("host_loop_step_us_one_launch", fstep)):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for i in range(K):
                    fn(i)
                torch.cuda.synchronize()
                res["one_launch_decode"][name] = round((time.perf_counter() - t0) / K * 1e6, 2)
        except moe.MoeError as e:
            res["one_launch_decode"] = {"unsupported": str(e)}

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        res["device_copy_gbps"] = round(2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_reps)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
