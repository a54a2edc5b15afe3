#!/usr/bin/env python3
"""HBM traffic of the block-sparse prefill kernel, from rocprofv3 counters.

Runs, each as its own rocprofv3 pass (one counter per pass):
  * FETCH_SIZE, then WRITE_SIZE (KiB per dispatch) over ``bench.py`` on the
    named workload (without its decode and CPU-baseline legs), keeping the
    prefill kernel's dispatches;
  * the same two counters over a plain device copy of known size (a torch
    bf16 tensor copy), which calibrates KiB-as-counted to bytes moved.

Writes ``profiles/prefill_bf16_<workload>_traffic.json`` with the per-launch
bytes (read, written, total), the calibration factors, and a hash of the
kernel source, which ``bench.py`` checks before it reports the figure (a
changed kernel makes the record stale).  Usage, on a machine with the GPU:

    python bench_traffic.py [--config 3] [--out PATH]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import shutil
import statistics
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.abspath(__file__))
PREFILL_SRC = os.path.join(ROOT, "dynamic_sparse_attention_dhsa_amd", "csrc", "prefill_bf16.hip")
COPY_MIB = 1024

COPY_SNIPPET = f"""
import torch
x = torch.ones({COPY_MIB} * 1024 * 512, dtype=torch.bfloat16, device="cuda")
y = torch.empty_like(x)
for _ in range(3):
    y.copy_(x)
torch.cuda.synchronize()
print("copy done", flush=True)
"""


def rocprof_pass(counter: str, cmd: list[str], out_dir: str, timeout: int) -> list[dict]:
    env = dict(os.environ, TMPDIR="/tmp")
    full = ["timeout", "-s", "KILL", str(timeout), "rocprofv3", "--pmc", counter, "--output-format", "csv",
            "-d", out_dir, "-o", "run", "--"] + cmd
    print("[traffic] " + " ".join(full), flush=True)
    res = subprocess.run(full, cwd=ROOT, env=env, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout[-3000:] + res.stderr[-3000:])
        raise RuntimeError(f"rocprofv3 pass {counter} failed with exit code {res.returncode}")
    files = glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"no counter file under {out_dir}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def per_dispatch(rows: list[dict], counter: str, name_filter) -> list[float]:
    acc: dict[int, float] = {}
    for r in rows:
        if r["Counter_Name"] != counter or not name_filter(r["Kernel_Name"]):
            continue
        acc[int(r["Dispatch_Id"])] = acc.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    return [acc[k] for k in sorted(acc)]


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--timeout", type=int, default=240)
    ap.add_argument("--out", default=None, help="output path (default profiles/prefill_bf16_<workload>_traffic.json)")
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    from dynamic_sparse_attention_dhsa_amd import workloads as W
    name = W.make_config(args.config, layout_only=True).name

    work = tempfile.mkdtemp(prefix="dhsa_traffic_")
    bench = [sys.executable, "-u", "bench.py", "--config", str(args.config), "--steps", "2", "--warmup", "1",
             "--no-cpu-baseline", "--decode-batch", "0"]
    # bench.py's first 1 + 2 prefill launches are the step's (warm-up, then timed); the cold-cache
    # repetitions and the token-budget launches that follow run other lists or other cache states
    step_launches = 3
    copy = [sys.executable, "-u", "-c", COPY_SNIPPET]
    kib = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = rocprof_pass(counter, bench, os.path.join(work, "bench_" + counter), args.timeout)
        vals = per_dispatch(rows, counter, lambda k: "prefill_bf16_kernel" in k)[:step_launches]
        crow = rocprof_pass(counter, copy, os.path.join(work, "copy_" + counter), args.timeout)
        cvals = per_dispatch(crow, counter, lambda k: True)
        if not vals or not cvals:
            raise RuntimeError(f"{counter}: no prefill or copy dispatches found")
        kib[counter] = (statistics.median(vals), max(cvals), len(vals))
        print(f"[traffic] {counter}: prefill median {kib[counter][0]:.4g} KiB over {len(vals)} dispatches, "
              f"copy {kib[counter][1]:.4g} KiB", flush=True)
    copy_bytes = COPY_MIB * 1024 * 1024
    f_read = copy_bytes / (kib["FETCH_SIZE"][1] * 1024)
    f_write = copy_bytes / (kib["WRITE_SIZE"][1] * 1024)
    read_b = kib["FETCH_SIZE"][0] * 1024 * f_read
    write_b = kib["WRITE_SIZE"][0] * 1024 * f_write
    rec = {
        "workload": name,
        "kernel": "prefill_bf16_kernel",
        "kernel_source_sha256_16": hashlib.sha256(open(PREFILL_SRC, "rb").read()).hexdigest()[:16],
        "fetch_kib_per_dispatch": kib["FETCH_SIZE"][0],
        "write_kib_per_dispatch": kib["WRITE_SIZE"][0],
        "dispatches": kib["FETCH_SIZE"][2],
        "calibration": {"copy_bytes_each_way": copy_bytes, "copy_fetch_kib": kib["FETCH_SIZE"][1],
                        "copy_write_kib": kib["WRITE_SIZE"][1], "fetch_factor": f_read, "write_factor": f_write},
        "read_bytes_per_launch": read_b,
        "write_bytes_per_launch": write_b,
        "bytes_per_launch": read_b + write_b,
        "command": "python bench_traffic.py --config %d" % args.config,
    }
    path = args.out or os.path.join(ROOT, "profiles", f"prefill_bf16_{name}_traffic.json")
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec), flush=True)
    shutil.rmtree(work, ignore_errors=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
