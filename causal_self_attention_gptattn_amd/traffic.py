"""Turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs into per-launch HBM
bytes for each attention kernel.

The counters are calibrated against a device-to-device copy of known size
(``bench.py --copy-probe MIB`` profiled with the same counters): the factor
for each counter is (bytes the copy moves) / (bytes the counter reports).

Usage (from the repository root, after the four counter runs)::

    python -m causal_self_attention_gptattn_amd.traffic \\
        --fetch DIR/bench_counter_collection.csv --write DIR/bench_counter_collection.csv \\
        --copy-fetch DIR/copy_counter_collection.csv --copy-write DIR/copy_counter_collection.csv \\
        --copy-mib 256 --workload gpt2_124m --out profiles/traffic_gpt2_124m.json
"""

import argparse
import csv
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

KERNELS = ("attn_fwd", "attn_bwd_dq", "attn_bwd_dkdv")


def _per_kernel_kib(path, counter):
    """Average counter value (KiB) per dispatch for each kernel name."""
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            # the launch a kernel serves: attn_bwd_dq16<...>, attn_bwd_dkdv16w<...>
            # (16-row waves) and the head-size-64 kernels (attn_bwd_dkdv64<...>,
            # attn_bwd_dkdv64p<...>, attn_bwd_dkdv128p<...>) count as attn_bwd_dq /
            # attn_bwd_dkdv / attn_fwd
            m = re.search(r"::(attn_[a-z_]+?)(?:16w?|64p?|128p)?<", row["Kernel_Name"]) or re.search(
                r"(__amd_rocclr_copyBuffer)", row["Kernel_Name"])
            if not m:
                continue
            vals.setdefault(m.group(1), []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def _describe(name):
    from causal_self_attention_gptattn_amd import workloads as W

    w = W.WORKLOADS[name]
    return "%s (B=%d, H=%d, T=%d, D=%d, %s)" % (w.name, w.B, w.H, w.T, w.D, w.dtype)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--workload", default="gpt2_124m")
    ap.add_argument("--command", default="")
    args = ap.parse_args()

    import bench  # source hash of the kernels the counters describe

    copy_bytes = args.copy_mib << 20
    cf = _per_kernel_kib(args.copy_fetch, "FETCH_SIZE")["__amd_rocclr_copyBuffer"] * 1024
    cw = _per_kernel_kib(args.copy_write, "WRITE_SIZE")["__amd_rocclr_copyBuffer"] * 1024
    f_scale, w_scale = copy_bytes / cf, copy_bytes / cw
    fetch = _per_kernel_kib(args.fetch, "FETCH_SIZE")
    write = _per_kernel_kib(args.write, "WRITE_SIZE")
    rec = {
        "workload": _describe(args.workload),
        "source_sha": bench.source_sha(),
        "calibration": {"copy_bytes": copy_bytes, "fetch_scale": round(f_scale, 4),
                        "write_scale": round(w_scale, 4)},
        "command": args.command,
        "kernels": {},
    }
    for k in KERNELS:
        if k in fetch and k in write:
            rec["kernels"][k] = {
                "fetch_bytes": int(fetch[k] * 1024 * f_scale),
                "write_bytes": int(write[k] * 1024 * w_scale),
            }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
