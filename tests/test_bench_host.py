"""Host-side logic of bench.py (CPU): the algorithmic work counts, the pair
count of the masked variants, the traffic profile's staleness check and the
one-GPU guard."""

import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import attention as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_work_counts_at_the_gpt2_shape(bench):
    N, T, D = 144, 1024, 64
    tab = bench.kernel_table(N, T, D)
    flops = sum(k["flops"] for k in tab.values())
    assert flops == 6 * N * D * T * (T + 1)
    assert abs(flops / 1e9 - 58.039) < 1e-3
    # one bf16 tensor 18.87 MB, one float32 row vector N*T*4 bytes
    t, r = N * T * D * 2, N * T * 4
    assert tab["attn_fwd"]["bytes"] == 4 * t + r
    assert tab["attn_bwd_dq"]["bytes"] == 6 * t + 3 * r
    assert tab["attn_bwd_dkdv"]["bytes"] == 6 * t + 2 * r
    assert all(k["exps"] == N * T * (T + 1) // 2 for k in tab.values())


@pytest.mark.parametrize("Tq,Tk,off,win", [
    (64, 64, 0, 0), (1, 1024, 1023, 0), (100, 300, 200, 0), (129, 129, 0, 64),
    (200, 130, -70, 0), (31, 31, 40, 0), (150, 150, -20, 33), (1024, 1024, 0, 256),
])
def test_visible_pairs_match_the_oracle_mask(bench, Tq, Tk, off, win):
    assert bench.visible_pairs(Tq, Tk, off, win) == int(np.sum(A.visible(Tq, Tk, off, win)))


def test_traffic_is_reported_only_for_the_sources_it_was_taken_with(bench, tmp_path,
                                                                  monkeypatch):
    rec = {"source_sha": bench.source_sha(),
           "kernels": {"attn_bwd_dkdv": {"fetch_bytes": 100, "write_bytes": 23}}}
    path = tmp_path / "traffic_gpt2_124m.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    assert bench.measured_traffic("attn_bwd_dkdv", "gpt2_124m") == 123
    assert bench.measured_traffic("attn_fwd", "gpt2_124m") is None
    # another workload's counters are never reported
    assert bench.measured_traffic("attn_bwd_dkdv", "gpt3_2048") is None
    rec["source_sha"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("attn_bwd_dkdv", "gpt2_124m") is None


def test_source_hash_ignores_comments_only(bench):
    """Counter profiles stay valid across comment edits, not code edits."""
    a = "int f(int x) {  // twice\n  return 2 * x; /* doubled */ }\n"
    b = "/* header */\nint f(int x) {\n  return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }"
    assert bench.code_of(a) == bench.code_of(b) != bench.code_of(c)


def test_timing_event_flag_matches_the_hip_header(bench):
    """The timing events skip the system-scope fence: the flag is the one
    HIP's runtime header defines for that."""
    import re

    header = "/opt/rocm/include/hip/hip_runtime_api.h"
    if not os.path.exists(header):
        pytest.skip("no HIP runtime header here")
    m = re.search(r"#define\s+hipEventDisableSystemFence\s+(0x[0-9a-fA-F]+)", open(header).read())
    assert m and int(m.group(1), 16) == bench.HIP_EVENT_DISABLE_SYSTEM_FENCE


def test_rocm_smi_record_parsing(bench):
    """sclk and power come out of rocm-smi's JSON record of the first card."""
    rec = {"card0": {"sclk clock speed:": "(1972Mhz)", "sclk clock level:": "1",
                     "fclk clock speed:": "(2000Mhz)",
                     "Current Socket Graphics Package Power (W)": "871.0",
                     "Card Series": "AMD Instinct MI355X"},
           "card1": {"sclk clock speed:": "(100Mhz)"}}
    assert bench.parse_smi(rec) == ([1972], [871.0])
    assert bench.parse_smi({}) == ([], [])
    assert bench.parse_smi([]) == ([], [])
    rec = {"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": 248, "unit": "W"},
                                             "gfx_voltage": "N/A"}}]}
    assert bench.parse_amdsmi_power(rec) == [248.0]
    assert bench.parse_amdsmi_power({"gpu_data": []}) == []
    assert bench.parse_amdsmi_power({}) == []


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr


def test_traffic_counters_are_keyed_by_launch(tmp_path):
    """Counter rows map to the launch they belong to, whichever kernel
    variant served it."""
    from causal_self_attention_gptattn_amd import traffic

    rows = [("void gptattn::(anonymous namespace)::attn_fwd<64, false>(...)", 10.0),
            ("void gptattn::(anonymous namespace)::attn_bwd_dq16<64, false>(...)", 20.0),
            ("void gptattn::(anonymous namespace)::attn_bwd_dq<128, true>(...)", 40.0),
            ("void gptattn::(anonymous namespace)::attn_bwd_dkdv<64, 64>(...)", 30.0),
            ("void gptattn::(anonymous namespace)::attn_bwd_dkdv16w<128, false>(...)", 50.0),
            ("void gptattn::(anonymous namespace)::attn_bwd_dkdv64<4>(...)", 60.0),
            ("void gptattn::(anonymous namespace)::attn_bwd_dkdv64p<4>(...)", 70.0),
            ("void gptattn::(anonymous namespace)::attn_bwd_dkdv128p<8>(...)", 80.0),
            ("__amd_rocclr_copyBuffer", 7.0)]
    path = tmp_path / "c.csv"
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, v in rows:
            f.write('"%s",FETCH_SIZE,%g\n' % (name, v))
    got = traffic._per_kernel_kib(str(path), "FETCH_SIZE")
    assert got == {"attn_fwd": 10.0, "attn_bwd_dq": 30.0, "attn_bwd_dkdv": (30.0 + 50.0 + 60.0 + 70.0 + 80.0) / 5,
                   "__amd_rocclr_copyBuffer": 7.0}


def test_roofline_takes_the_tighter_roof(bench):
    """frac = max(F / peak_flops, B / peak_bw) / t, reported against the roof
    that term belongs to."""
    # the GPT-2 dK/dV launch: 29.0 GFLOP, 114.4 MB -> the HBM term is larger
    N, T, D = 144, 1024, 64
    k = bench.kernel_table(N, T, D)["attn_bwd_dkdv"]
    t = 50e-6
    r = bench.roofline(k["flops"], k["bytes"], t)
    f_term = k["flops"] / (bench.PEAK_BF16_TFLOPS * 1e12)
    b_term = k["bytes"] / (bench.PEAK_HBM_GBS * 1e9)
    assert b_term > f_term
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
    assert abs(r["frac"] - max(f_term, b_term) / t) < 1e-12
    assert abs(r["achieved"] - k["bytes"] / t / 1e9) < 1e-6
    # the GPT-3-shaped layer's dK/dV launch is matrix-bound
    k = bench.kernel_table(96, 2048, 128)["attn_bwd_dkdv"]
    r = bench.roofline(k["flops"], k["bytes"], 300e-6)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["frac"] - k["flops"] / (bench.PEAK_BF16_TFLOPS * 1e12) / 300e-6) < 1e-12


def test_float32_tensor_bytes(bench):
    t16 = bench.kernel_table(4, 64, 16)["attn_fwd"]["bytes"]
    t32 = bench.kernel_table(4, 64, 16, 4)["attn_fwd"]["bytes"]
    assert t32 - t16 == 4 * (4 * 64 * 16 * 2)


def test_per_kernel_pass_timing_with_fake_events(bench):
    """The per-kernel pass on the CPU with stand-in events: each kernel's mean
    is taken between the events at its launch boundaries, and each step's
    duration runs from the first event to the last."""
    clock = [0.0]

    class Event:
        def record(self, stream):
            self.t = clock[0]

        def elapsed_time(self, later):
            return later.t - self.t

        def synchronize(self):
            pass

    class Step:
        def __init__(self):
            self.n = 0

        def launch(self, i):
            clock[0] += (1.0, 2.0, 3.0)[i] + 0.5 * self.n
            if i == 2:
                self.n += 1

        def __call__(self):
            for i in range(3):
                self.launch(i)

    ev = [[Event() for _ in range(4)] for _ in range(4)]
    totals = []
    ks = bench.per_kernel_pass(Step(), 4, None, None, keep_busy=2, events=ev, step_times=totals)
    # step s adds 0.5 * s to each of its three launches
    assert ks == pytest.approx([1.75, 2.75, 3.75])
    assert totals == pytest.approx([6.0, 7.5, 9.0, 10.5])
