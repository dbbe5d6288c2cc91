"""rocprofv3 harness for the attention kernels on one MI355X (gfx950).

Runs bench.py workloads under rocprofv3 in child processes and reports, for
the causal prefill kernel, achieved TFLOP/s and matrix-core (MFMA)
utilisation against the dense bf16 peak, and for the paged decode kernels
achieved HBM GB/s against the HBM peak, each with the HBM bytes the hardware
counters saw per launch.

    python3 transformer_attention_tiled_amd/rocprof_harness.py --out DIR [--update-profiles]
    python3 transformer_attention_tiled_amd/rocprof_harness.py --record DIR/summary.json

Passes (each its own rocprofv3 run, under its own time limit):
  trace_c3, trace_c4       --kernel-trace --stats: per-launch durations of
                           the prefill (B=1, Hq=32, Hkv=8, T=16384, d=128)
                           and of the decode split and merge kernels (64
                           sequences, Hq=12, Hkv=2, 8 rotated KV pools)
  fetch_*, write_*         --pmc FETCH_SIZE, then --pmc WRITE_SIZE (one
                           counter per run) for a plain 1 GiB device copy
                           (the calibration), the prefill and the decode
  mfma_c3                  --pmc with eight SQ counters (waves, busy CU
                           cycles, MFMA busy cycles, MFMA / VALU / LDS
                           instruction counts, LDS bank conflicts, LDS waits)

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch; each is scaled by
what it reads for the copy of known size (bytes moved / counter bytes).
Achieved rates use the algorithmic work bench.py reports (credited causal
FLOPs; every valid K/V element once plus q, o, table entries and lengths)
over the mean kernel duration of the timed launches (the last `steps`
launches of each kernel in the trace).

The harness itself never touches the GPU (it does not import torch): the
profiled program is bench.py, started by rocprofv3 as its direct child, from
/tmp with TMPDIR=/tmp. Results go to DIR/summary.json and DIR/summary.md;
with --update-profiles the calibrated byte counts are also written to
profiles/hbm_traffic.json, keyed with a hash of each kernel's source file
(bench.py reports `traffic` only while that hash matches); --record does the
same later from a run's summary.json.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
BENCH = os.path.join(ROOT, "bench.py")
PROFILES = os.path.join(ROOT, "profiles")

PEAK_BF16_TFLOPS = 2516.6  # dense bf16 MFMA, 256 CUs x 2.4 GHz
PEAK_HBM_GBS = 8000.0
N_CU = 256
SIMD_PER_CU = 4
COPY_BYTES = 1 << 30       # bench.py --workload copy moves 1 GiB each way

KERNELS = {
    "prefill": "prefill_pp_kernel<128, true>",
    "decode": "decode_kernel<128>",
    "merge": "decode_merge_kernel<128>",
    "copy": "__amd_rocclr_copyBuffer",
}
SQ_COUNTERS = ["SQ_WAVES", "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
               "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS"]
TRAFFIC_KEYS = {
    "prefill": "prefill_pp_kernel<128,true> B=1 Hq=32 Hkv=8 T=16384",
    "decode": "decode_kernel<128> 64 seqs Hq=12 Hkv=2 (mean of 8 rotated pools)",
}
SOURCES = {"prefill": "prefill_bf16.hip", "decode": "decode_paged.hip"}


# ---------------------------------------------------------------- parsing

def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_durations(trace_csv, name):
    """Durations in microseconds of every launch of the kernel whose name
    contains `name`, in dispatch order."""
    rows = []
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            if name in r["Kernel_Name"]:
                rows.append((int(r["Dispatch_Id"]),
                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0))
    return [us for _, us in sorted(rows)]


def counter_values(counter_csv, name, counter):
    """Per-dispatch values of `counter` for the kernel whose name contains
    `name`, in dispatch order (values of one dispatch are summed if the file
    lists them per instance)."""
    per = {}
    with open(counter_csv, newline="") as f:
        for r in csv.DictReader(f):
            if name in r["Kernel_Name"] and r["Counter_Name"] == counter:
                k = int(r["Dispatch_Id"])
                per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def mean(xs):
    if not xs:
        raise ValueError("no samples")
    return sum(xs) / len(xs)


def timed_stats(durs, steps):
    t = durs[-steps:] if steps and len(durs) >= steps else durs
    return {"launches": len(durs), "timed": len(t), "mean_us": mean(t), "min_us": min(t),
            "max_us": max(t)}


# ------------------------------------------------------------- arithmetic

def calibration(copy_fetch_kib, copy_write_kib, copy_bytes=COPY_BYTES):
    """Scale factors from counter KiB to bytes moved, from a copy of known size."""
    return {"fetch_scale": copy_bytes / (copy_fetch_kib * 1024.0),
            "write_scale": copy_bytes / (copy_write_kib * 1024.0)}


def traffic_bytes(fetch_kib, write_kib, cal):
    return fetch_kib * 1024.0 * cal["fetch_scale"] + write_kib * 1024.0 * cal["write_scale"]


def mfma_utilisation(mfma_busy_cycles, busy_cu_cycles):
    """Fraction of the CUs' busy cycles in which a SIMD's matrix core was
    busy: the MFMA busy count is summed over the 1024 SIMDs, the busy-CU
    count over the 256 CUs."""
    return (mfma_busy_cycles / (N_CU * SIMD_PER_CU)) / (busy_cu_cycles / N_CU)


def summarise(res):
    """res: raw measurements (see main); returns the report dictionary."""
    cal = calibration(res["copy_fetch_kib"], res["copy_write_kib"])
    p_us = res["prefill_trace"]["mean_us"]
    p_tflops = res["prefill_flops"] / (p_us * 1e-6) / 1e12
    d_us = res["decode_trace"]["mean_us"]
    m_us = res["merge_trace"]["mean_us"]
    by = res["decode_bytes"]
    out = {
        "calibration": {**cal, "copy_fetch_kib": res["copy_fetch_kib"],
                        "copy_write_kib": res["copy_write_kib"], "copy_bytes": COPY_BYTES},
        "prefill": {
            "kernel": KERNELS["prefill"], **res["prefill_trace"],
            "flops": res["prefill_flops"],
            "tflops": p_tflops, "frac_bf16_peak": p_tflops / PEAK_BF16_TFLOPS,
            "fetch_kib": res["prefill_fetch_kib"], "write_kib": res["prefill_write_kib"],
            "hbm_bytes": traffic_bytes(res["prefill_fetch_kib"], res["prefill_write_kib"], cal),
        },
        "decode": {
            "kernels": [KERNELS["decode"], KERNELS["merge"]],
            "split": res["decode_trace"], "merge": res["merge_trace"],
            "bytes": by,
            "gbs_split": by / (d_us * 1e-6) / 1e9,
            "gbs_split_plus_merge": by / ((d_us + m_us) * 1e-6) / 1e9,
            "fetch_kib": res["decode_fetch_kib"], "write_kib": res["decode_write_kib"],
            "merge_fetch_kib": res["merge_fetch_kib"], "merge_write_kib": res["merge_write_kib"],
            "hbm_bytes": traffic_bytes(res["decode_fetch_kib"], res["decode_write_kib"], cal),
        },
    }
    out["decode"]["frac_hbm_split_plus_merge"] = out["decode"]["gbs_split_plus_merge"] / PEAK_HBM_GBS
    sq = res.get("prefill_sq")
    if sq:
        out["prefill"]["sq"] = sq
        out["prefill"]["mfma_util"] = mfma_utilisation(sq["SQ_VALU_MFMA_BUSY_CYCLES"],
                                                       sq["SQ_BUSY_CU_CYCLES"])
    return out


def markdown(rep, cmd):
    p, d, c = rep["prefill"], rep["decode"], rep["calibration"]
    lines = [
        "# rocprofv3 harness: causal prefill (B=1 Hq=32 Hkv=8 T=16384 d=128) and paged decode "
        "(64 seqs Hq=12 Hkv=2 d=128)",
        "",
        "Command (from the repository root on one MI355X):",
        "",
        "```",
        cmd,
        "```",
        "",
        "| kernel | timed launches | mean µs | min µs | max µs | achieved | of peak |",
        "|---|---|---|---|---|---|---|",
        f"| `{p['kernel']}` | {p['timed']} | {p['mean_us']:.2f} | {p['min_us']:.2f} | "
        f"{p['max_us']:.2f} | {p['tflops']:.1f} TFLOP/s | {100 * p['frac_bf16_peak']:.1f}% of "
        f"{PEAK_BF16_TFLOPS} TFLOP/s |",
        f"| `{d['kernels'][0]}` | {d['split']['timed']} | {d['split']['mean_us']:.2f} | "
        f"{d['split']['min_us']:.2f} | {d['split']['max_us']:.2f} | {d['gbs_split']:.0f} GB/s | "
        f"{100 * d['gbs_split'] / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f} GB/s |",
        f"| `{d['kernels'][1]}` | {d['merge']['timed']} | {d['merge']['mean_us']:.2f} | "
        f"{d['merge']['min_us']:.2f} | {d['merge']['max_us']:.2f} | split + merge: "
        f"{d['gbs_split_plus_merge']:.0f} GB/s | {100 * d['frac_hbm_split_plus_merge']:.1f}% |",
        "",
        f"Algorithmic work: prefill {p['flops'] / 1e12:.4f} TFLOP per launch (credited causal "
        f"FLOPs); decode {d['bytes'] / 1e6:.1f} MB per call (K/V once, q, o, table, lengths).",
        "",
        f"HBM counters (calibration: a 1 GiB copy reads FETCH_SIZE {c['copy_fetch_kib']:.1f} KiB "
        f"and WRITE_SIZE {c['copy_write_kib']:.1f} KiB, scale {c['fetch_scale']:.3f} and "
        f"{c['write_scale']:.3f}):",
        "",
        "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated HBM bytes |",
        "|---|---|---|---|",
        f"| `{p['kernel']}` | {p['fetch_kib']:.1f} | {p['write_kib']:.1f} | "
        f"{p['hbm_bytes'] / 1e6:.1f} MB |",
        f"| `{d['kernels'][0]}` | {d['fetch_kib']:.1f} | {d['write_kib']:.1f} | "
        f"{d['hbm_bytes'] / 1e6:.1f} MB |",
        f"| `{d['kernels'][1]}` | {d['merge_fetch_kib']:.1f} | {d['merge_write_kib']:.1f} | — |",
    ]
    if "mfma_util" in p:
        lines += ["", "Prefill shader counters (mean per dispatch):", "",
                  "| counter | value |", "|---|---|"]
        lines += [f"| {k} | {v:.0f} |" for k, v in p["sq"].items()]
        lines += ["", f"Matrix cores busy {100 * p['mfma_util']:.1f}% of the busy cycles "
                      "(SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over SQ_BUSY_CU_CYCLES / 256 CUs)."]
    return "\n".join(lines) + "\n"


# --------------------------------------------------------------- running

def run_pass(out, name, prof_args, workload, steps, warmup, limit):
    """One rocprofv3 run of bench.py; returns (output dir, bench's JSON line)."""
    d = os.path.join(out, name)
    cmd = ["timeout", "-s", "KILL", str(limit), "rocprofv3", *prof_args, "--output-format",
           "csv", "-d", d, "-o", "r", "--", sys.executable, BENCH, "--workload", workload,
           "--steps", str(steps), "--warmup", str(warmup)]
    print("[harness] " + " ".join(cmd), flush=True)
    log = os.path.join(out, name + ".log")
    with open(log, "w") as f:
        r = subprocess.run(cmd, cwd="/tmp", env=dict(os.environ, TMPDIR="/tmp"), stdout=f,
                           stderr=subprocess.STDOUT)
    text = open(log).read()
    js = [l for l in text.splitlines() if l.startswith("{")]
    if r.returncode != 0:
        # rocprofv3 can exit with a segmentation fault after the program has
        # finished and its results are complete; accept that case only
        if not (r.returncode in (139, -11) and js):
            raise SystemExit(f"[harness] pass {name} failed with status {r.returncode}; see {log}")
        print(f"[harness] pass {name}: rocprofv3 exited {r.returncode} after the program "
              "finished; results kept", flush=True)
    if not js:
        raise SystemExit(f"[harness] pass {name}: bench.py printed no result; see {log}")
    return d, json.loads(js[-1])


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", help="output directory (created)")
    ap.add_argument("--record", metavar="SUMMARY_JSON",
                    help="only write profiles/hbm_traffic.json from an earlier run's summary.json")
    ap.add_argument("--steps", type=int, default=16, help="timed steps in the trace passes")
    ap.add_argument("--limit", type=int, default=180, help="seconds allowed per pass")
    ap.add_argument("--no-sq", action="store_true", help="skip the shader-counter pass")
    ap.add_argument("--update-profiles", action="store_true",
                    help="write the calibrated bytes to profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.record:
        with open(args.record) as f:
            update_traffic(json.load(f))
        return
    if not args.out:
        ap.error("--out is required")
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    res = {}

    d, js = run_pass(out, "trace_c3", ["--kernel-trace", "--stats"], "c3", args.steps, 5,
                     args.limit)
    res["prefill_flops"] = js["flops"]
    res["prefill_trace"] = timed_stats(
        kernel_durations(_find(d, "kernel_trace.csv"), KERNELS["prefill"]), args.steps)
    d, js = run_pass(out, "trace_c4", ["--kernel-trace", "--stats"], "c4", args.steps, 8,
                     args.limit)
    res["decode_bytes"] = js["bytes"]
    tr = _find(d, "kernel_trace.csv")
    res["decode_trace"] = timed_stats(kernel_durations(tr, KERNELS["decode"]), args.steps)
    res["merge_trace"] = timed_stats(kernel_durations(tr, KERNELS["merge"]), args.steps)

    for ctr, key in (("FETCH_SIZE", "fetch_kib"), ("WRITE_SIZE", "write_kib")):
        tag = ctr.split("_")[0].lower()
        d, _ = run_pass(out, f"{tag}_copy", ["--pmc", ctr], "copy", 3, 1, args.limit)
        res[f"copy_{key}"] = mean(counter_values(_find(d, "counter_collection.csv"),
                                                 KERNELS["copy"], ctr)[-3:])
        d, _ = run_pass(out, f"{tag}_c3", ["--pmc", ctr], "c3", 3, 1, args.limit)
        res[f"prefill_{key}"] = mean(counter_values(_find(d, "counter_collection.csv"),
                                                    KERNELS["prefill"], ctr))
        d, _ = run_pass(out, f"{tag}_c4", ["--pmc", ctr], "c4", 8, 0, args.limit)
        cc = _find(d, "counter_collection.csv")
        res[f"decode_{key}"] = mean(counter_values(cc, KERNELS["decode"], ctr))
        res[f"merge_{key}"] = mean(counter_values(cc, KERNELS["merge"], ctr))

    if not args.no_sq:
        d, _ = run_pass(out, "mfma_c3", ["--pmc", *SQ_COUNTERS], "c3", 3, 1, args.limit)
        cc = _find(d, "counter_collection.csv")
        res["prefill_sq"] = {c: mean(counter_values(cc, KERNELS["prefill"], c))
                             for c in SQ_COUNTERS}

    rep = summarise(res)
    rep["raw"] = res
    cmd = "python3 transformer_attention_tiled_amd/rocprof_harness.py --out " + args.out + (
        " --update-profiles" if args.update_profiles else "")
    with open(os.path.join(out, "summary.json"), "w") as f:
        json.dump(rep, f, indent=1)
    md = markdown(rep, cmd)
    with open(os.path.join(out, "summary.md"), "w") as f:
        f.write(md)
    print(md, flush=True)
    if args.update_profiles:
        update_traffic(rep)


def update_traffic(rep, path=None):
    """Record the calibrated bytes per launch with each kernel's source hash."""
    path = path or os.path.join(PROFILES, "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        rec = {}
    c = rep["calibration"]
    rec["calibration"] = {"copy_bytes": c["copy_bytes"], "fetch_kib": c["copy_fetch_kib"],
                          "write_kib": c["copy_write_kib"], "fetch_scale": c["fetch_scale"],
                          "write_scale": c["write_scale"]}
    for part in ("prefill", "decode"):
        r = rep[part]
        src = SOURCES[part]
        with open(os.path.join(PKG, "csrc", src), "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()[:16]
        e = {"source": src, "source_sha256_16": h, "fetch_kib": r["fetch_kib"],
             "write_kib": r["write_kib"],
             "fetch_bytes": r["fetch_kib"] * 1024.0 * c["fetch_scale"],
             "write_bytes": r["write_kib"] * 1024.0 * c["write_scale"]}
        if part == "decode":
            e["merge_kernel_fetch_kib"] = r["merge_fetch_kib"]
            e["merge_kernel_write_kib"] = r["merge_write_kib"]
        rec[TRAFFIC_KEYS[part]] = e
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"[harness] updated {path}", flush=True)


if __name__ == "__main__":
    main()
