"""Benchmark: causal attention forward + backward on one MI355X.

One step = the whole hot path on one batch: gptattn_fwd (attn_fwd kernel),
then the backward as its two launches gptattn_bwd_dq (attn_bwd_dq) and
gptattn_bwd_dkdv (attn_bwd_dkdv), on the GPT-2 124M attention shape
(B=12, H=12, T=1024, D=64, bf16) with inputs resident in HBM.

Throughput counts algorithmic work only: 6 * D * T * (T + 1) flops per
head-problem (QK^T and PV forward; dV, dP, dQ, dK backward over the causal
triangle including the diagonal).  Score recomputation in the backward is
implementation work and is not counted.

Prints one JSON line.  Per-kernel durations come from HIP events recorded on
the launch stream around every launch of a separate pass of steps.  Each
event record costs the stream a few microseconds, so the timed steps carry
only two per step, around the dominant kernel: its duration for the roofline
is measured live over the timed steps, and the step-to-step intervals of the
second event give the per-step spread.

The line also carries "variants": the strided entry points timed the same
way (HIP events around each step) on the same head shape -- q, k, v read in
place from a packed [B, T, 3C] buffer with gradients written into one packed
buffer; a locally banded causal mask of 256 positions; attention dropout with
p = 0.1; and one decoding step (one query against a 1024-token context,
forward only, reported in GB/s).
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s at GPT-2 124M shape; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# Transcendental roof: v_exp_f32 issues at half the fp32 rate (measured: one
# wave64 instruction per 8 cycles per SIMD), i.e. 256 CU x 4 SIMD x 64 lanes
# / 8 cycles x 2.4 GHz exponentials per second.
PEAK_EXP_PER_S = 256 * 4 * 64 / 8 * 2.4e9
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gpt2_124m.json")
KERNEL_SOURCES = ["attn_bf16.hip", "attn_common.h"]


def unit_flops(N, T, D):
    """Flops of one causal product (T(T+1)/2 pairs x D multiply-adds x 2)."""
    return N * D * T * (T + 1)


def kernel_table(N, T, D):
    """Algorithmic flops, bytes and exponentials per launch of each kernel
    (bf16).  Each kernel takes one exponential per visible score element."""
    u = unit_flops(N, T, D)
    t = N * T * D * 2      # one bf16 [B,H,T,D] tensor
    r = N * T * 4          # one float32 [B,H,T] vector
    x = N * T * (T + 1) // 2
    return {
        # QK^T and PV; reads Q, K, V, writes O and lse
        "attn_fwd": {"flops": 2 * u, "bytes": 4 * t + r, "exps": x},
        # the dQ product; reads Q, K, V, O, dO, lse, writes dQ and the row term
        "attn_bwd_dq": {"flops": 1 * u, "bytes": 6 * t + 2 * r, "exps": x},
        # dP, dV and dK products; reads Q, K, V, dO, lse, row term, writes dK, dV
        "attn_bwd_dkdv": {"flops": 3 * u, "bytes": 6 * t + 2 * r, "exps": x},
    }


def source_sha():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "causal_self_attention_gptattn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter profile, or None if
    there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != source_sha():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    return int(k["fetch_bytes"] + k["write_bytes"])


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def clocks_under_load(run_some_steps, limit_s):
    """sclk and power as rocm-smi reports them while steps keep the GPU busy
    (best effort: None when the tool is missing or fails)."""
    import subprocess

    try:
        proc = subprocess.Popen(["rocm-smi", "--showclocks", "--showpower", "--json"],
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.time()
    while proc.poll() is None and time.time() - t0 < limit_s:
        run_some_steps()
    try:
        out, _ = proc.communicate(timeout=5)
        rec = json.loads(out)
    except Exception:  # noqa: BLE001 -- a diagnostic, never fatal
        proc.kill()
        return None
    card = next(iter(rec.values()), {}) if isinstance(rec, dict) else {}
    keep = {k_: v_ for k_, v_ in card.items()
            if "sclk" in k_.lower() or "mclk" in k_.lower() or "power" in k_.lower()}
    return keep or None


def cpu_baseline(inp, budget_s):
    """Time the float64 oracle on a bounded sample of whole heads."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import attention as A

    q, k, v, do = (inp[n].float().numpy() for n in ("q", "k", "v", "do"))
    B, H, T, D = q.shape
    cores = min(len(os.sched_getaffinity(0)), 16)
    heads = [(b, h) for b in range(B) for h in range(H)]
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        while True:
            b, h = heads[done % len(heads)]
            A.forward_head(q[b, h], k[b, h], v[b, h], inp["scale"])
            A.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], inp["scale"])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    flops = 6 * done * D * T * (T + 1)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(used),
        "kind": "oracle",
        "sample": "%d head-problems (cycling over the %d heads of B=%d, H=%d, T=%d, D=%d), "
                  "float64 numpy oracle forward + backward, %.1f s, %s"
                  % (done, B * H, B, H, T, D, dt, cpu_model()),
    }


def visible_pairs(Tq, Tk, off, win):
    """Number of (query, key) pairs the mask lets through."""
    n = 0
    for i in range(Tq):
        hi = min(Tk - 1, i + off)
        lo = max(0, i + off - win + 1) if win > 0 else 0
        n += max(0, hi - lo + 1)
    return n


def time_steps(step, steps, warmup, stream):
    """Average GPU time (ms) of `step` between HIP events on `stream`."""
    import torch

    for _ in range(warmup):
        step()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        step()
    ev[1].record(stream)
    ev[1].synchronize()
    return ev[0].elapsed_time(ev[1]) / steps


def variants(G, inp, dev, stream, steps):
    """Time the strided entry points on the workload's head shape."""
    import ctypes

    import torch

    lib = G.library()
    sp = stream.cuda_stream
    q0, k0, v0, do0 = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    B, H, T, D = q0.shape
    sc = inp["scale"]
    out = {}

    def ex_step(pb, q, k, v, o, lse, do, dq, dk, dv, ws, fwd_only=False):
        P = ctypes.byref
        tq, tk, tv, to = (G._tensor(t) for t in (q, k, v, o))
        if fwd_only:
            def step():
                rc = lib.gptattn_fwd_ex(P(pb), P(tq), P(tk), P(tv), P(to), lse.data_ptr(), sp)
                if rc:
                    raise RuntimeError(G.status_string(rc))
            return step
        tdo, tdq, tdk, tdv = (G._tensor(t) for t in (do, dq, dk, dv))
        nbytes = ws.numel()

        def step():
            rc = lib.gptattn_fwd_ex(P(pb), P(tq), P(tk), P(tv), P(to), lse.data_ptr(), sp)
            rc = rc or lib.gptattn_bwd_ex(P(pb), P(tq), P(tk), P(tv), P(to), P(tdo),
                                          lse.data_ptr(), P(tdq), P(tdk), P(tdv),
                                          ws.data_ptr(), nbytes, sp)
            if rc:
                raise RuntimeError(G.status_string(rc))
        return step

    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ws = torch.empty(B * H * T * 4, dtype=torch.uint8, device=dev)

    # packed [B, T, 3C] projection output and packed gradient buffer
    x = torch.cat([t.transpose(1, 2).reshape(B, T, H * D) for t in (q0, k0, v0)], dim=-1)
    q, k, v = G.split_qkv(x.contiguous(), H)
    y = torch.empty(B, T, H * D, dtype=q0.dtype, device=dev)
    o = y.view(B, T, H, D).transpose(1, 2)
    gx = torch.empty(B, T, 3 * H * D, dtype=q0.dtype, device=dev)
    dq, dk, dv = G.split_qkv(gx, H)
    pb = G._problem(q, k, sc, 0, 0)
    ms = time_steps(ex_step(pb, q, k, v, o, lse, do0, dq, dk, dv, ws), steps, 3, stream)
    fl = 12 * D * visible_pairs(T, T, 0, 0) * B * H
    out["packed_qkv"] = {"B": B, "H": H, "T": T, "D": D, "ms": round(ms, 5),
                         "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}

    # locally banded causal mask, 256 positions
    o2 = torch.empty_like(q0)
    dq2, dk2, dv2 = (torch.empty_like(q0) for _ in range(3))
    win = 256
    pb = G._problem(q0, k0, sc, 0, win)
    ms = time_steps(ex_step(pb, q0, k0, v0, o2, lse, do0, dq2, dk2, dv2, ws), steps, 3, stream)
    fl = 12 * D * visible_pairs(T, T, 0, win) * B * H
    out["banded_w256"] = {"B": B, "H": H, "T": T, "D": D, "window": win, "ms": round(ms, 5),
                          "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}

    # attention dropout, p = 0.1 (the keep mask is redrawn in every kernel)
    pb = G._problem(q0, k0, sc, 0, 0, 0.1, 1234, 0)
    ms = time_steps(ex_step(pb, q0, k0, v0, o2, lse, do0, dq2, dk2, dv2, ws), steps, 3, stream)
    fl = 12 * D * visible_pairs(T, T, 0, 0) * B * H
    out["dropout_p0.1"] = {"B": B, "H": H, "T": T, "D": D, "dropout": 0.1, "ms": round(ms, 5),
                           "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}

    # one decoding step: one query against the T-token context (forward only)
    qd = q0[:, :, T - 1:].contiguous()
    od = torch.empty_like(qd)
    lsed = torch.empty((B, H, 1), dtype=torch.float32, device=dev)
    pb = G._problem(qd, k0, sc, T - 1, 0)
    ms = time_steps(ex_step(pb, qd, k0, v0, od, lsed, None, None, None, None, None,
                            fwd_only=True), steps, 3, stream)
    nbytes = B * H * (2 * T * D * 2 + 2 * D * 2 + 4)
    out["decode_1x%d" % T] = {"B": B, "H": H, "Tq": 1, "Tk": T, "D": D, "ms": round(ms, 5),
                              "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps timed with the caches flushed before each one")
    ap.add_argument("--variant-steps", type=int, default=20,
                    help="timed steps per strided-entry-point variant (0 = skip them)")
    ap.add_argument("--smi-seconds", type=float, default=15.0,
                    help="at most this long, run steps while rocm-smi reads sclk and power "
                         "(0 = skip)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (calibrates the "
                         "HBM byte counters against a copy of known size) and exit")
    args = ap.parse_args()

    if args.copy_probe:
        import torch

        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_per_launch": {"read": n, "write": n}, "launches": 5}))
        return

    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import causal_self_attention_gptattn_amd as G
    from causal_self_attention_gptattn_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path")
    print("bench: generating %s inputs" % w.name, file=sys.stderr, flush=True)
    inp = W.workload_inputs(w.name, seed=0)
    B, H, T, D, N = w.B, w.H, w.T, w.D, w.N
    sc = inp["scale"]
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws_bytes = G.workspace_bytes(B, H, T, D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    lib = G.library()
    P = lambda t: t.data_ptr()  # noqa: E731
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def fwd():
        return lib.gptattn_fwd(P(q), P(k), P(v), P(o), P(lse), B, H, T, D, sc, sp)

    def bdq():
        return lib.gptattn_bwd_dq(P(q), P(k), P(v), P(o), P(do), P(lse), P(dq), B, H, T, D, sc,
                                  P(ws), ws_bytes, sp)

    def bdkdv():
        return lib.gptattn_bwd_dkdv(P(q), P(k), P(v), P(do), P(lse), P(dk), P(dv), B, H, T, D,
                                    sc, P(ws), ws_bytes, sp)

    launches = [("attn_fwd", fwd), ("attn_bwd_dq", bdq), ("attn_bwd_dkdv", bdkdv)]

    def step(events=None, around=None):
        """One step.  events: one event per launch boundary (len(launches) + 1),
        or with `around` = i a pair recorded just before and after launch i."""
        for i, (name, fn) in enumerate(launches):
            if events is not None and (around is None or around == i):
                events[0 if around is not None else i].record(stream)
            rc = fn()
            if rc != 0:
                raise RuntimeError("%s: %s" % (name, G.status_string(rc)))
            if events is not None and around == i:
                events[1].record(stream)
        if events is not None and around is None:
            events[len(launches)].record(stream)

    print("bench: warmup %d steps" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    # per-kernel durations: a pass with an event at every launch boundary
    print("bench: per-kernel pass %d steps" % args.steps, file=sys.stderr, flush=True)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(pev[i])
    torch.cuda.synchronize(dev)
    per_kernel_ms = {name: 0.0 for name, _ in launches}
    for e in pev:
        for i, (name, _) in enumerate(launches):
            per_kernel_ms[name] += e[i].elapsed_time(e[i + 1])
    per_kernel_ms = {k_: t / args.steps for k_, t in per_kernel_ms.items()}
    dom = max(per_kernel_ms, key=per_kernel_ms.get)
    dom_i = [name for name, _ in launches].index(dom)

    # timed steps: two events per step, around the dominant kernel
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i], around=dom_i)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0

    dom_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    step_ms = [evs[i - 1][1].elapsed_time(evs[i][1]) for i in range(1, args.steps)]
    q1, med, q3 = (float(x) for x in np.percentile(step_ms, [25, 50, 75]))

    # Cold-cache steps: overwrite a 1 GiB buffer before each (outside events).
    cold_ms = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(args.cold_steps)]
        for e in cev:
            flush.fill_(1)
            e[0].record(stream)
            step()
            e[1].record(stream)
        torch.cuda.synchronize(dev)
        cold_ms = sum(a.elapsed_time(b) for a, b in cev) / args.cold_steps
        del flush

    flops = 6 * N * D * T * (T + 1)
    ms = wall * 1e3 / args.steps
    value = flops / (wall / args.steps) / 1e12
    table = kernel_table(N, T, D)
    achieved = table[dom]["flops"] / (dom_ms * 1e-3) / 1e12
    kernels = {}
    for name, t_ms in per_kernel_ms.items():
        tf = table[name]["flops"] / (t_ms * 1e-3) / 1e12
        gbs = table[name]["bytes"] / (t_ms * 1e-3) / 1e9
        eps = table[name]["exps"] / (t_ms * 1e-3)
        kernels[name] = {
            "ms": round(t_ms, 5),
            "alg_tflops": round(tf, 2),
            "alg_gbs": round(gbs, 1),
            # fraction of each roof: bf16 MFMA, HBM, transcendental (exp)
            "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "exp_frac": round(eps / PEAK_EXP_PER_S, 4),
        }
    traffic = measured_traffic(dom)

    # clocks and power while the step runs (outside every timed region)
    def some_steps():
        for _ in range(20):
            step()
        torch.cuda.synchronize(dev)

    gpu_state = clocks_under_load(some_steps, args.smi_seconds) if args.smi_seconds > 0 else None

    var = None
    if args.variant_steps > 0:
        print("bench: strided entry points", file=sys.stderr, flush=True)
        var = variants(G, inp, dev, stream, args.variant_steps)

    base = None
    if args.cpu_budget > 0:
        print("bench: oracle CPU baseline (%.0f s budget)" % args.cpu_budget,
              file=sys.stderr, flush=True)
        base = cpu_baseline(inp, args.cpu_budget)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "D": D, "causal": True,
                   "scale": sc, "alg_gflop_per_step": round(flops / 1e9, 3)},
        "pct_of_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        # the FlashAttention-paper convention (7 D T^2 per head-problem, counts
        # the backward's recomputation); labelled, never mixed with `value`
        "fa_convention_tflops": round(7 * N * D * T * T / (wall / args.steps) / 1e12, 2),
        "step_ms_events": {"median": round(med, 5), "min": round(float(min(step_ms)), 5),
                           "iqr": round(q3 - q1, 5)},
        "kernels": kernels,
        "cold_cache_ms_per_step": None if cold_ms is None else round(cold_ms, 5),
        "roofline": {
            "kernel": dom,
            "kernel_ms": round(dom_ms, 5),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": base,
        "gpu_under_load": gpu_state,
        "variants": var,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
