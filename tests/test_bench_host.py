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
    assert tab["attn_bwd_dq"]["bytes"] == 6 * t + 2 * r
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
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("attn_bwd_dkdv") == 123
    assert bench.measured_traffic("attn_fwd") is None
    rec["source_sha"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("attn_bwd_dkdv") is None


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
            ("__amd_rocclr_copyBuffer", 7.0)]
    path = tmp_path / "c.csv"
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, v in rows:
            f.write('"%s",FETCH_SIZE,%g\n' % (name, v))
    got = traffic._per_kernel_kib(str(path), "FETCH_SIZE")
    assert got == {"attn_fwd": 10.0, "attn_bwd_dq": 30.0, "attn_bwd_dkdv": 40.0,
                   "__amd_rocclr_copyBuffer": 7.0}
