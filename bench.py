"""Benchmark: causal attention forward + backward on one MI355X.

One step = the whole hot path on one batch: gptattn_fwd (attn_fwd kernel),
then the backward as its two launches gptattn_bwd_dq (the dQ kernel) and
gptattn_bwd_dkdv (the dK/dV kernel), on the GPT-2 124M attention shape
(B=12, H=12, T=1024, D=64, bf16) with inputs resident in HBM.

Throughput counts algorithmic work only: 6 * D * T * (T + 1) flops per
head-problem (QK^T and PV forward; dV, dP, dQ, dK backward over the causal
triangle including the diagonal).  Score recomputation in the backward is
implementation work and is not counted.

Timing.  `value` is the cold-cache figure: before every timed step a 1 GiB
buffer is overwritten (outside the HIP events), which evicts the step's
152.8 MB working set (Q, K, V, O, dO, dQ, dK, dV, lse and the two
workspace vectors) from the 256 MB last-level cache, so every step reads
its inputs from HBM.  Each timed step carries three events on the launch
stream (before the forward, before the dominant kernel, after the step):
the step time, and the dominant kernel's time for the roofline, both
measured live over the timed steps.  The events are HIP events created
with hipEventDisableSystemFence: a default event fences at system scope
when recorded (a cache writeback and invalidation), which would slow the
kernel after it.  The warm figure (steps back to back,
no flush, wall clock) is reported beside it.  A separate pass with an event
at every launch boundary gives the per-kernel table.  The clock (sclk) is
sampled with rocm-smi while the same flushed steps keep running right after
the timed region.

Prints one JSON line with, besides the contract's keys: the roofline of the
dominant kernel against whichever of its two roofs (bf16 MFMA, HBM) is the
tighter one, the measured dense bf16 GEMM rate of the box (the attainable
matrix-core peak), sclk samples taken under the same load, the CPU
oracle baseline, the other workloads of the pages (`configs`), and the
strided entry points (`variants`).
"""

import argparse
import hashlib
import json
import os
import platform
import re
import subprocess
import sys
import threading
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
TRAFFIC_DIR = os.path.join(ROOT, "profiles")  # traffic_<workload>.json
KERNEL_SOURCES = ["attn_bf16.hip", "attn_d64.hip", "attn_d128.hip", "attn_common.h"]
FLUSH_BYTES = 1 << 30
# hipEventDisableSystemFence (hip_runtime_api.h): record the event without
# the system-scope fence a default event performs, a cache writeback and
# invalidation that slows whatever kernel follows it
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence,
    with torch.cuda.Event's record / elapsed_time interface.  A default
    event (torch's) fences at system scope when recorded: one recorded
    between two kernels writes back and invalidates the caches, which costs
    the step about 4 us at the GPT-2 shape and slows the kernel after it."""

    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes

            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                    ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes

        self.ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev),
                                                 HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)

    def record(self, stream):
        import ctypes

        rc = self._lib().hipEventRecord(self.ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def synchronize(self):
        """Wait on the host until the event has been reached."""
        rc = self._lib().hipEventSynchronize(self.ev)
        if rc != 0:
            raise RuntimeError("hipEventSynchronize failed (%d)" % rc)

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and done)."""
        import ctypes

        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def unit_flops(N, T, D):
    """Flops of one causal product (T(T+1)/2 pairs x D multiply-adds x 2)."""
    return N * D * T * (T + 1)


def kernel_table(N, T, D, elem=2):
    """Algorithmic flops, bytes and exponentials per launch of each kernel.
    Each kernel takes one exponential per visible score element."""
    u = unit_flops(N, T, D)
    t = N * T * D * elem   # one [B,H,T,D] tensor
    r = N * T * 4          # one float32 [B,H,T] vector
    x = N * T * (T + 1) // 2
    return {
        # QK^T and PV; reads Q, K, V, writes O and lse
        "attn_fwd": {"flops": 2 * u, "bytes": 4 * t + r, "exps": x},
        # the dQ product; reads Q, K, V, O, dO, lse, writes dQ and two row
        # vectors (the softmax row term, lse / scale) for the dK/dV kernel
        "attn_bwd_dq": {"flops": 1 * u, "bytes": 6 * t + 3 * r, "exps": x},
        # dP, dV and dK products; reads Q, K, V, dO and the two row vectors,
        # writes dK, dV
        "attn_bwd_dkdv": {"flops": 3 * u, "bytes": 6 * t + 2 * r, "exps": x},
    }


def roofline(flops, nbytes, seconds):
    """The tighter of the two roofs for work (flops, bytes) done in `seconds`:
    frac = max(F / peak_flops, B / peak_bw) / t.  Reported in the unit of the
    binding roof."""
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        ach = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS}
    ach = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS}


def code_of(text):
    """A kernel source with its comments and blank space taken out: what the
    compiler sees (the sources hold no string literal with // or /*)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha():
    """Hash of the kernel code (comments excluded) that counter profiles
    are tied to."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "causal_self_attention_gptattn_amd", "csrc", name)) as f:
            h.update(code_of(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter profile of this
    workload, or None if there is none or the kernel sources changed since it
    was taken."""
    try:
        with open(os.path.join(TRAFFIC_DIR, "traffic_%s.json" % workload)) as f:
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


def parse_smi(rec):
    """sclk readings (MHz) and power readings (W) of the first card in a
    `rocm-smi --showclocks --showpower --json` record."""
    card = next(iter(rec.values()), {}) if isinstance(rec, dict) else {}
    sclk, power = [], []
    for k_, v_ in card.items():
        key = k_.lower()
        if "sclk" in key and "speed" in key:
            digits = "".join(ch for ch in str(v_) if ch.isdigit())
            if digits:
                sclk.append(int(digits))
        elif "power" in key and "(w)" in key:
            try:
                power.append(float(v_))
            except (TypeError, ValueError):
                pass
    return sclk, power


def parse_amdsmi_power(rec):
    """Socket power (W) of the first GPU in an `amd-smi metric --power --json`
    record."""
    try:
        gpus = rec["gpu_data"] if isinstance(rec, dict) else rec
        sp = gpus[0]["power"]["socket_power"]
        return [float(sp["value"] if isinstance(sp, dict) else sp)]
    except (KeyError, IndexError, TypeError, ValueError):
        return []


class ClockSampler:
    """Polls rocm-smi for sclk and power in a background thread while the
    GPU works; best effort (no samples when the tool is missing)."""

    def __init__(self, enabled=True):
        self.samples = []
        self.power = []
        self.enabled = enabled
        self._stop = threading.Event()
        self._t = None

    def _poll(self):
        while not self._stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"],
                                     capture_output=True, text=True, timeout=10).stdout
                rec = json.loads(out)
            except Exception:  # noqa: BLE001 -- a diagnostic, never fatal
                return
            sclk, power = parse_smi(rec)
            self.samples += sclk
            if not power:
                try:
                    out = subprocess.run(["amd-smi", "metric", "--power", "--json"],
                                         capture_output=True, text=True, timeout=10).stdout
                    power = parse_amdsmi_power(json.loads(out))
                except Exception:  # noqa: BLE001 -- a diagnostic, never fatal
                    power = []
            self.power += power[:1]

    def __enter__(self):
        if self.enabled:
            self._t = threading.Thread(target=self._poll, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._t is not None:
            self._t.join(timeout=15)


def cpu_baseline(inp, budget_s):
    """Time the float64 oracle (forward and backward separately) on whole
    heads of the workload, with every core of this process's affinity set
    as BLAS threads, for about budget_s seconds."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import attention as A

    q, k, v, do = (inp[n].float().numpy() for n in ("q", "k", "v", "do"))
    B, H, T, D = q.shape
    cores = len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(B) for h in range(H)]
    done, t_fwd, t_bwd = 0, 0.0, 0.0
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        while t_fwd + t_bwd < budget_s:
            b, h = heads[done % len(heads)]
            t0 = time.perf_counter()
            A.forward_head(q[b, h], k[b, h], v[b, h], inp["scale"])
            t1 = time.perf_counter()
            A.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], inp["scale"])
            t2 = time.perf_counter()
            t_fwd += t1 - t0
            t_bwd += t2 - t1
            done += 1
    alg = 6 * done * D * T * (T + 1)
    # dense products of the explicit T x T formulation: forward QK^T and PV,
    # backward dV, dP, dQ, dK (12 T^2 D per head-problem)
    return {
        "value": alg / (t_fwd + t_bwd) / 1e12,
        "unit": "TFLOP/s",
        "cores": int(used),
        "kind": "oracle",
        "sample": "%d head-problems (cycling over the %d heads of B=%d, H=%d, T=%d, D=%d), "
                  "float64 numpy oracle, forward %.1f s + backward %.1f s, %d cores of %s"
                  % (done, B * H, B, H, T, D, t_fwd, t_bwd, cores, cpu_model()),
        "fwd_s_per_head": t_fwd / done,
        "bwd_s_per_head": t_bwd / done,
        "dense_fp64_gflops_fwd": 4 * T * T * D * done / t_fwd / 1e9,
        "dense_fp64_gflops_bwd": 8 * T * T * D * done / t_bwd / 1e9,
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
    ev = [TimingEvent() for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / steps


def gemm_rate(dev, n=8192, reps=20):
    """Measured dense bf16 matrix-core rate of this machine (TFLOP/s): a large
    square bf16 product through the vendor GEMM library, the attainable
    counterpart of the spec peak."""
    import torch

    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    e1.synchronize()
    return 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def gpu_inputs(B, H, T, D, dtype, dev, seed=0):
    """Inputs of the workloads' recipe (projection of Gaussian activations,
    or iid for float32), drawn with torch's generator on the GPU: the
    `configs` timings need the shapes and value distribution, not the exact
    numbers of the CPU generator the parity tests use."""
    import torch

    g = torch.Generator(device=dev).manual_seed(seed)
    if dtype == "f32":
        return [torch.randn(B, H, T, D, device=dev, generator=g) for _ in range(4)]
    C = H * D
    x = torch.randn(B * T, C, device=dev, generator=g)
    out = []
    for _ in range(3):
        w = torch.randn(C, C, device=dev, generator=g) * 0.02
        out.append((x @ w).view(B, T, H, D).transpose(1, 2).contiguous().bfloat16())
    out.append((torch.randn(B, H, T, D, device=dev, generator=g) * 0.01).bfloat16())
    return out


class Step:
    """One forward + backward of a dense [B,H,T,D] problem through the C ABI,
    launch by launch (bf16 or float32 entry points)."""

    def __init__(self, G, q, k, v, do, scale, stream):
        import torch

        self.lib = G.library()
        self.G = G
        B, H, T, D = q.shape
        self.shape = (B, H, T, D)
        f32 = q.dtype == torch.float32
        self.q, self.k, self.v, self.do = q, k, v, do
        self.o = torch.empty_like(q)
        self.lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
        self.dq, self.dk, self.dv = (torch.empty_like(q) for _ in range(3))
        self.wsb = G.workspace_bytes(B, H, T, D, f32)
        self.ws = torch.empty(self.wsb, dtype=torch.uint8, device=q.device)
        self.sc = scale
        self.sp = stream.cuda_stream
        sfx = "_f32" if f32 else ""
        self.fn = [getattr(self.lib, "gptattn_fwd" + sfx),
                   getattr(self.lib, "gptattn_bwd_dq" + sfx),
                   getattr(self.lib, "gptattn_bwd_dkdv" + sfx)]

    def launch(self, i):
        B, H, T, D = self.shape
        P = lambda t: t.data_ptr()  # noqa: E731
        if i == 0:
            rc = self.fn[0](P(self.q), P(self.k), P(self.v), P(self.o), P(self.lse), B, H, T, D,
                            self.sc, self.sp)
        elif i == 1:
            rc = self.fn[1](P(self.q), P(self.k), P(self.v), P(self.o), P(self.do), P(self.lse),
                            P(self.dq), B, H, T, D, self.sc, P(self.ws), self.wsb, self.sp)
        else:
            rc = self.fn[2](P(self.q), P(self.k), P(self.v), P(self.do), P(self.lse), P(self.dk),
                            P(self.dv), B, H, T, D, self.sc, P(self.ws), self.wsb, self.sp)
        if rc != 0:
            raise RuntimeError("%s: %s" % (LAUNCHES[i], self.G.status_string(rc)))

    def __call__(self):
        for i in range(3):
            self.launch(i)


LAUNCHES = ("attn_fwd", "attn_bwd_dq", "attn_bwd_dkdv")


def per_kernel_pass(step, steps, stream, flush, keep_busy=0, events=None, step_times=None):
    """Each kernel's average duration (ms) with an event at every launch
    boundary, the caches flushed before each step (outside the events).
    With keep_busy > 0, that many more (untimed) steps are queued behind the
    pass, and the results are read while the GPU runs them.  `events`:
    steps x 4 TimingEvents created beforehand (else created here).  A list
    passed as `step_times` receives each step's duration (ms)."""
    ev = events if events is not None else [[TimingEvent() for _ in range(4)]
                                            for _ in range(steps)]
    for e in ev:
        if flush is not None:
            flush.fill_(1)
        for i in range(3):
            e[i].record(stream)
            step.launch(i)
        e[3].record(stream)
    for _ in range(keep_busy):
        if flush is not None:
            flush.fill_(1)
        step()
    ev[-1][3].synchronize()
    if step_times is not None:
        step_times.extend(e[0].elapsed_time(e[3]) for e in ev)
    return [sum(e[i].elapsed_time(e[i + 1]) for e in ev) / steps for i in range(3)]


def workload_configs(G, dev, stream, steps, flush):
    """The pages' other workloads, timed like the main one (cold caches,
    events at every launch boundary)."""
    import numpy as np

    from causal_self_attention_gptattn_amd import workloads as W

    out = {}
    for name, w in W.WORKLOADS.items():
        q, k, v, do = gpu_inputs(w.B, w.H, w.T, w.D, w.dtype, dev)
        st = Step(G, q, k, v, do, W.default_scale(w.D), stream)
        evs = [[TimingEvent() for _ in range(4)] for _ in range(steps)]
        # flushed warm-up running on into the pass (no idle gap, see main)
        for _ in range(20):
            flush.fill_(1)
            st()
        totals = []
        ks = per_kernel_pass(st, steps, stream, flush, events=evs, step_times=totals)
        ms = sum(ks)
        q1, med, q3 = (float(x) for x in np.percentile(totals, [25, 50, 75]))
        flops = 6 * unit_flops(w.N, w.T, w.D)
        table = kernel_table(w.N, w.T, w.D, 4 if w.dtype == "f32" else 2)
        rec = {"B": w.B, "H": w.H, "T": w.T, "D": w.D, "dtype": w.dtype,
               "ms_per_step": round(ms, 5), "alg_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
               "pct_of_bf16_mfma_peak": round(100.0 * flops / (ms * 1e-3) / 1e12
                                              / PEAK_BF16_TFLOPS, 2),
               "step_ms_events": {"median": round(med, 5), "min": round(min(totals), 5),
                                  "iqr": round(q3 - q1, 5)},
               "kernels_ms": {n: round(t, 5) for n, t in zip(LAUNCHES, ks)}}
        dom = max(range(3), key=lambda i: ks[i])
        rl = roofline(table[LAUNCHES[dom]]["flops"], table[LAUNCHES[dom]]["bytes"],
                      ks[dom] * 1e-3)
        rec["roofline"] = {"kernel": LAUNCHES[dom], "bound": rl["bound"],
                           "frac": round(rl["frac"], 4)}
        out[name] = rec
        del st, q, k, v, do
    return out


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
    ws = torch.empty(2 * B * H * T * 4, dtype=torch.uint8, device=dev)

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
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first, each after a cache flush like the timed ones "
                         "(about 0.1 s at the default: the clock settles under the load)")
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--config-steps", type=int, default=10,
                    help="timed steps per workload in the configs block (0 = skip it)")
    ap.add_argument("--variant-steps", type=int, default=20,
                    help="timed steps per strided-entry-point variant (0 = skip them)")
    ap.add_argument("--no-smi", action="store_true",
                    help="do not poll rocm-smi for clocks while the timed steps run")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps and the per-kernel pass (for profiling)")
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
    stream = torch.cuda.current_stream(dev)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    step = Step(G, q, k, v, do, sc, stream)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    table = kernel_table(N, T, D)
    flops = 6 * unit_flops(N, T, D)

    # Every timing event is created up front: creating them later would
    # leave the GPU idle in between, and its clock would drop.
    pk_evs = [[TimingEvent() for _ in range(4)] for _ in range(args.steps)]
    evs = [[TimingEvent() for _ in range(3)] for _ in range(args.steps)]

    # warm-up in the pattern of the timed steps (flush, step), running on into
    # the per-kernel pass without a pause
    print("bench: warmup %d steps" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        flush.fill_(1)
        step()

    # per-kernel table: events at every launch boundary, caches flushed
    print("bench: per-kernel pass %d steps" % args.steps, file=sys.stderr, flush=True)
    pk = per_kernel_pass(step, args.steps, stream, flush, keep_busy=10, events=pk_evs)
    dom_i = max(range(3), key=lambda i: pk[i])
    dom = LAUNCHES[dom_i]

    # timed steps: caches flushed before each (outside the events); events
    # before the forward, before the dominant kernel and after the step.  The
    # events were created beforehand and the per-kernel pass left the GPU
    # busy while its results were read, so the GPU does not idle (and its
    # clock does not drop) between that pass and the timed steps.
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for e in evs:
        flush.fill_(1)
        e[0].record(stream)
        for i in range(3):
            if i == dom_i:
                e[1].record(stream)
            step.launch(i)
        e[2].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0

    # warm steps: back to back, no flush, wall clock; right after the timed
    # steps (after the clock sampling below, whose rocm-smi / amd-smi calls
    # leave the next steps measurably slower, they read 0.1435 against
    # 0.1338 ms for the flushed steps on one box)
    tw = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    warm_ms = (time.perf_counter() - tw) * 1e3 / args.steps

    # The clock under this load: rocm-smi polled while the same flushed steps
    # keep running right after the timed region (a rocm-smi call during the
    # timed steps stalls the step it lands on by half a millisecond, so it
    # stays out of them).
    with ClockSampler(not args.no_smi) as clocks:
        t1 = time.perf_counter()
        while clocks.enabled and len(clocks.samples) < 3 and time.perf_counter() - t1 < 5.0:
            for _ in range(10):
                flush.fill_(1)
                step()
            torch.cuda.synchronize(dev)
    step_ms = np.array([a.elapsed_time(c) for a, _, c in evs])
    dom_ms = float(np.mean([b.elapsed_time(c) if dom_i == 2 else 0.0 for _, b, c in evs]))
    if dom_i != 2:  # the dominant kernel is followed by others: use the per-kernel pass
        dom_ms = pk[dom_i]
    ms = float(step_ms.mean())
    value = flops / (ms * 1e-3) / 1e12
    q1, med, q3 = (float(x) for x in np.percentile(step_ms, [25, 50, 75]))

    rl = roofline(table[dom]["flops"], table[dom]["bytes"], dom_ms * 1e-3)
    kernels = {}
    for name, t_ms in zip(LAUNCHES, pk):
        tf = table[name]["flops"] / (t_ms * 1e-3) / 1e12
        gbs = table[name]["bytes"] / (t_ms * 1e-3) / 1e9
        eps = table[name]["exps"] / (t_ms * 1e-3)
        r = roofline(table[name]["flops"], table[name]["bytes"], t_ms * 1e-3)
        kernels[name] = {
            "ms": round(t_ms, 5),
            "alg_tflops": round(tf, 2),
            "alg_gbs": round(gbs, 1),
            # fraction of each roof: bf16 MFMA, HBM, transcendental (exp)
            "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "exp_frac": round(eps / PEAK_EXP_PER_S, 4),
            "bound": r["bound"],
            "frac": round(r["frac"], 4),
        }

    extras = not args.no_extras
    gemm = None
    if extras:
        print("bench: dense bf16 GEMM rate", file=sys.stderr, flush=True)
        gemm = gemm_rate(dev)
    cfgs = None
    if extras and args.config_steps > 0:
        print("bench: the other workloads", file=sys.stderr, flush=True)
        cfgs = workload_configs(G, dev, stream, args.config_steps, flush)
    var = None
    if extras and args.variant_steps > 0:
        print("bench: strided entry points", file=sys.stderr, flush=True)
        var = variants(G, inp, dev, stream, args.variant_steps)
    base = None
    if extras and args.cpu_budget > 0:
        print("bench: oracle CPU baseline (%.0f s budget)" % args.cpu_budget,
              file=sys.stderr, flush=True)
        base = cpu_baseline(inp, args.cpu_budget)
        # GPU speed-up over the oracle on the same workload (algorithmic rates)
        base["gpu_speedup"] = round(value / base["value"], 1)

    sclk = clocks.samples
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
                   "scale": sc, "alg_gflop_per_step": round(flops / 1e9, 3),
                   "caches": "flushed before every timed step"},
        "pct_of_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "measured_bf16_gemm_tflops": None if gemm is None else round(gemm, 1),
        "pct_of_measured_gemm_rate": None if gemm is None else round(100.0 * value / gemm, 2),
        "warm": {"ms_per_step": round(warm_ms, 5),
                 "tflops": round(flops / (warm_ms * 1e-3) / 1e12, 2)},
        # the FlashAttention-paper convention (7 D T^2 per head-problem, counts
        # the backward's recomputation); labelled, never mixed with `value`
        "fa_convention_tflops": round(7 * N * D * T * T / (ms * 1e-3) / 1e12, 2),
        "step_ms_events": {"median": round(med, 5), "min": round(float(step_ms.min()), 5),
                           "max": round(float(step_ms.max()), 5), "iqr": round(q3 - q1, 5),
                           "all": [round(float(x), 4) for x in step_ms]},
        "timed_region_wall_s": round(wall, 4),
        "kernels": kernels,
        "roofline": {
            "kernel": dom,
            "kernel_ms": round(dom_ms, 5),
            "bound": rl["bound"],
            "achieved": round(rl["achieved"], 2),
            "peak": rl["peak"],
            "unit": rl["unit"],
            "frac": round(rl["frac"], 4),
            "traffic": measured_traffic(dom, w.name),
            # the algorithmic work of one launch, against which traffic compares
            "alg_bytes": table[dom]["bytes"],
            "alg_flops": table[dom]["flops"],
        },
        # forward and backward separately (the per-kernel pass; backward =
        # dQ + dK/dV launches)
        "fwd_ms": round(pk[0], 5),
        "bwd_ms": round(pk[1] + pk[2], 5),
        "cpu_baseline": base,
        "sclk_mhz_under_load": {"samples": len(sclk),
                                "median": int(np.median(sclk)) if sclk else None,
                                "min": min(sclk) if sclk else None},
        "power_w_under_load": {"samples": len(clocks.power),
                               "median": round(float(np.median(clocks.power)), 1)
                               if clocks.power else None},
        "configs": cfgs,
        "variants": var,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
