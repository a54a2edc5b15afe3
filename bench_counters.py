#!/usr/bin/env python3
"""Matrix-core and instruction counters of the block-sparse prefill kernel, from rocprofv3.

Runs two rocprofv3 counter passes over ``bench.py`` on the named workload (without its decode and
CPU-baseline legs) and keeps the prefill kernel's dispatches of the step (warm-up and timed: the
first three), taking the median of each counter over them:

  * matrix pass: SQ_VALU_MFMA_BUSY_CYCLES, SQ_VALU_MFMA_COEXEC_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_INSTS_MFMA, SQ_WAVE_CYCLES, SQ_WAVES, GRBM_GUI_ACTIVE;
  * instruction pass: SQ_INSTS_VALU, SQ_INSTS_SALU, SQ_INSTS_LDS, SQ_INSTS_SMEM, SQ_ACTIVE_INST_VALU,
    SQ_ACTIVE_INST_SCA, SQ_ACTIVE_INST_LDS, SQ_ACTIVE_INST_ANY, GRBM_GUI_ACTIVE.

Derived (written beside the raw sums): the kernel's clock cycles (GRBM_GUI_ACTIVE summed over the
8 XCDs, divided by 8), the matrix pipe's busy share (MFMA busy cycles over clock cycles x 1024 SIMDs),
the effective clock over the bench's own K3 time, executed matrix FLOPs (MOPS x 512) against the
algorithmic kept FLOPs, instructions per wave-tile (MFMA count / MFMAs per wave-tile), and the share of
the two wave slots per SIMD holding a wave (SQ_WAVE_CYCLES, in quad-cycles).  Writes
``profiles/prefill_bf16_<workload>_counters.{json,md}``.  Usage, on a machine with the GPU:

    python bench_counters.py [--config 3]
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
sys.path.insert(0, ROOT)
from bench_traffic import per_dispatch  # noqa: E402  (sums a counter's rows per dispatch of the named kernels)
PREFILL_SRC = os.path.join(ROOT, "dynamic_sparse_attention_dhsa_amd", "csrc", "prefill_bf16.hip")
XCDS, SIMDS, WAVE_SLOTS = 8, 1024, 2          # MI355X: 8 XCDs, 256 CUs x 4 SIMDs; two prefill waves per SIMD
PASSES = {
    "matrix": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               "SQ_INSTS_MFMA", "SQ_WAVE_CYCLES", "SQ_WAVES", "GRBM_GUI_ACTIVE"],
    "instructions": ["SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_SMEM", "SQ_ACTIVE_INST_VALU",
                     "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE"],
}


def rocprof_pass(counters: list[str], cmd: list[str], out_dir: str, timeout: int):
    env = dict(os.environ, TMPDIR="/tmp")
    full = ["timeout", "-s", "KILL", str(timeout), "rocprofv3", "--pmc"] + counters + [
        "--output-format", "csv", "-d", out_dir, "-o", "run", "--"] + cmd
    print("[counters] " + " ".join(full), flush=True)
    res = subprocess.run(full, cwd=ROOT, env=env, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout[-3000:] + res.stderr[-3000:])
        raise RuntimeError(f"rocprofv3 pass failed with exit code {res.returncode}")
    files = glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"no counter file under {out_dir}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    bench = [line for line in res.stdout.splitlines() if line.startswith("{")]
    return rows, (json.loads(bench[-1]) if bench else None)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--timeout", type=int, default=240)
    args = ap.parse_args()
    from dynamic_sparse_attention_dhsa_amd import workloads as W
    w = W.make_config(args.config, layout_only=True)
    if w.dtype != "bf16":
        raise SystemExit("the counters cover the bf16 prefill kernel")
    bench = [sys.executable, "-u", "bench.py", "--config", str(args.config), "--steps", "2", "--warmup", "1",
             "--no-cpu-baseline", "--decode-batch", "0"]
    step_launches = 3
    work = tempfile.mkdtemp(prefix="dhsa_counters_")
    raw, t3_ms, algo = {}, [], None
    for name, counters in PASSES.items():
        rows, line = rocprof_pass(counters, bench, os.path.join(work, name), args.timeout)
        for c in counters:
            vals = per_dispatch(rows, c, lambda k: "prefill_bf16_kernel" in k)[:step_launches]
            if not vals:
                raise RuntimeError(f"{c}: no prefill dispatches found")
            raw[c if c != "GRBM_GUI_ACTIVE" else f"GRBM_GUI_ACTIVE[{name}]"] = statistics.median(vals)
        if line is not None:
            t3_ms.append(line["stages"]["t_prefill_ms"])
            algo = line["roofline"]["algorithmic_flops_per_launch"]
    shutil.rmtree(work, ignore_errors=True)

    d = w.head_dim
    mfma_per_tile = 2 * (d // 16) + (64 // 16) * (d // 32)   # 32-row waves: QK^T then PV per 64-key tile
    clocks = raw["GRBM_GUI_ACTIVE[matrix]"] / XCDS
    clocks_i = raw["GRBM_GUI_ACTIVE[instructions]"] / XCDS
    tiles = raw["SQ_INSTS_MFMA"] / mfma_per_tile
    t3 = statistics.median(t3_ms) if t3_ms else None
    derived = {
        "kernel_clock_cycles": clocks,
        "effective_clock_GHz": clocks / (t3 * 1e-3) / 1e9 if t3 else None,
        "mfma_busy_share": raw["SQ_VALU_MFMA_BUSY_CYCLES"] / (clocks * SIMDS),
        "mfma_coexec_share_of_busy": raw["SQ_VALU_MFMA_COEXEC_CYCLES"] / raw["SQ_VALU_MFMA_BUSY_CYCLES"],
        "executed_mfma_flops": raw["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512,
        "algorithmic_flops": algo,
        "executed_over_algorithmic": raw["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / algo if algo else None,
        "wave_slot_occupancy": raw["SQ_WAVE_CYCLES"] * 4 / (clocks * SIMDS * WAVE_SLOTS),
        "mfma_per_wave_tile": mfma_per_tile if d == 128 else None,
        "per_wave_tile": ({k: raw[k] / tiles for k in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS",
                                                          "SQ_INSTS_SMEM")} if d == 128 else None),
        "active_inst_share": {k: raw[k] * 4 / (clocks_i * SIMDS * WAVE_SLOTS)
                              for k in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_LDS",
                                        "SQ_ACTIVE_INST_ANY")},
        "t_prefill_ms_under_counters": t3,
    }
    rec = {
        "workload": w.name,
        "kernel": "prefill_bf16_kernel",
        "kernel_source_sha256_16": hashlib.sha256(open(PREFILL_SRC, "rb").read()).hexdigest()[:16],
        "dispatches": step_launches,
        "raw_median_over_dispatches": raw,
        "derived": derived,
        "command": "python bench_counters.py --config %d" % args.config,
    }
    base = os.path.join(ROOT, "profiles", f"prefill_bf16_{w.name}_counters")
    os.makedirs(os.path.dirname(base), exist_ok=True)
    with open(base + ".json", "w") as f:
        json.dump(rec, f, indent=1)
    pct = lambda x: "—" if x is None else f"{100 * x:.1f}%"
    md = [f"# Matrix-core and instruction counters of prefill_bf16_kernel on {w.name}", "",
          f"Command (from the repository root, on one MI355X): `{rec['command']}`", "",
          "Two rocprofv3 counter passes over `" + " ".join(["python"] + bench[1:]) + "`, the median of each "
          f"counter over the step's {step_launches} prefill dispatches (warm-up and two timed); the raw sums are in "
          f"`prefill_bf16_{w.name}_counters.json`.", "",
          "| Quantity | Value | From |", "|:--|--:|:--|",
          f"| kernel clock cycles | {clocks:.4g} | GRBM_GUI_ACTIVE / 8 XCDs |",
          f"| effective clock | {derived['effective_clock_GHz']:.2f} GHz | cycles over the bench's K3 time, {t3:.3f} ms |"
          if t3 else "| effective clock | — | |",
          f"| matrix pipe busy | {pct(derived['mfma_busy_share'])} | SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs) |",
          f"| VALU issued while the matrix pipe is busy | {pct(derived['mfma_coexec_share_of_busy'])} of busy cycles | SQ_VALU_MFMA_COEXEC_CYCLES |",
          f"| executed matrix FLOPs | {derived['executed_mfma_flops']:.4g} | SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 |",
          f"| over algorithmic kept FLOPs ({algo:.4g}) | {derived['executed_over_algorithmic']:.3f} | |"
          if algo else "| over algorithmic kept FLOPs | — | |",
          f"| wave slots holding a wave | {pct(derived['wave_slot_occupancy'])} | SQ_WAVE_CYCLES x 4 / (cycles x 1024 x 2) |"]
    if derived["per_wave_tile"]:
        pt = derived["per_wave_tile"]
        md.append(f"| per wave-tile (32 queries x 64 keys, {mfma_per_tile} MFMAs) | VALU {pt['SQ_INSTS_VALU']:.0f} "
                  f"(MFMAs included), SALU {pt['SQ_INSTS_SALU']:.0f}, LDS {pt['SQ_INSTS_LDS']:.0f}, SMEM "
                  f"{pt['SQ_INSTS_SMEM']:.1f} | SQ_INSTS_* / (SQ_INSTS_MFMA / {mfma_per_tile}) |")
    a = derived["active_inst_share"]
    md.append(f"| wave cycles issuing VALU / scalar / LDS / any | {pct(a['SQ_ACTIVE_INST_VALU'])} / "
              f"{pct(a['SQ_ACTIVE_INST_SCA'])} / {pct(a['SQ_ACTIVE_INST_LDS'])} / {pct(a['SQ_ACTIVE_INST_ANY'])} | "
              "SQ_ACTIVE_INST_* x 4 / (cycles x 1024 x 2) |")
    with open(base + ".md", "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
