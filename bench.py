"""Benchmark of the fused attention hot path on one MI355X.

One step = one pass over the whole path on one batch of synthetic input:
  * causal prefill, bf16, B=1, Hq=32, Hkv=8 (GQA 4), T=16384, d=128
    (attn_prefill), and
  * paged decode, bf16, 64 sequences x 1 query, Hq=12, Hkv=2, d=128,
    block 16, lengths uniform in [256, 4096] (attn_decode_paged).
Inputs are resident in HBM before the timed region. The decode batch cycles
through 8 independently drawn KV pools (about 1.2 GB), so that the 256 MB
last-level cache cannot serve it from a previous step.

Printed: one JSON line. ``value`` is the prefill throughput in TFLOP/s
(algorithmic causal FLOPs 4*B*Hq*d*T(T+1)/2 over the prefill call's time,
HIP events on its stream); ``decode`` carries the decode HBM throughput
(algorithmic bytes: every valid K/V element once, q, o, used table entries
and lengths, over the decode call's time). ``roofline`` is for the prefill
kernel against the dense bf16 MFMA peak; ``roofline_decode`` for the decode
call (split kernel + merge kernel) against the HBM peak. ``cpu_baseline`` is
the CPU oracle timed on this host on half of the prefill's query heads.

Other workloads (parity configurations, the mixed paged batch) can be timed
with --workload; only the default is the headline line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import transformer_attention_tiled_amd as attn  # noqa: E402
from transformer_attention_tiled_amd import inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA, MI355X
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "causal prefill TFLOP/s + paged-decode HBM GB/s on 1 MI355X (% of roofline)"
ROTATE = 8


def causal_flops(B, Hq, T, d):
    return 4.0 * B * Hq * d * T * (T + 1) / 2


def decode_bytes(b, Hq, Hkv, d):
    lens = b["seq_lens_host"]
    kv = sum(lens) * Hkv * d * 2 * 2              # each valid K and V element once (bf16)
    qo = len(lens) * Hq * d * 2 * 2               # q in, o out
    table = sum(math.ceil(L / 16) for L in lens) * 4 + len(lens) * 4
    return kv + qo + table


class Timer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self):
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record(torch.cuda.current_stream())
        return e

    def stop(self, e0):
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(torch.cuda.current_stream())
        self.pairs.append((e0, e1))

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))


def make_prefill(cfg, dev):
    B, Hq, Hkv, T, d, dtype, seed = cfg
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, T, d, dtype, seed=seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    return dict(cpu=(q, k, v), q=qd, k=kd, v=vd, o=o, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, dtype=dtype)


def run_prefill(p):
    attn.prefill(p["q"], p["k"], p["v"], p["o"], causal=True)


def make_decode_sets(n_sets, num_seqs, Hq, Hkv, d, lo, hi, seed, dev, q_lens=None, gen_dev="cpu"):
    sets = []
    for r in range(n_sets):
        b = inputs.paged_inputs(num_seqs, Hq, Hkv, d, seq_len_range=(lo, hi), q_lens=q_lens,
                                seed=seed + 1000 * r, device=gen_dev)
        bd = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in b.items()}
        bd["o"] = torch.empty_like(bd["q"])
        bd["ws"] = torch.empty(max(1, attn.decode_paged_workspace_size(
            num_seqs, Hq, Hkv, d, b["max_seq_len"], PARTITION)), dtype=torch.uint8, device=dev)
        bd["cpu"] = b if r == 0 else None
        sets.append(bd)
    return sets


PARTITION = 0  # split-KV partition length for the decode calls (0 = the library's choice)


def run_decode(bd, with_qsl=False):
    attn.decode_paged(bd["q"], bd["k_cache"], bd["v_cache"], bd["block_table"], bd["seq_lens"],
                      max_seq_len=bd["max_seq_len"], max_query_len=bd["max_query_len"],
                      query_start_loc=bd["query_start_loc"] if with_qsl else None,
                      o=bd["o"], workspace=bd["ws"], partition_size=PARTITION)


def measured_traffic(kernel_key):
    """Calibrated HBM bytes per launch recorded under profiles/ for a kernel,
    or None when the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))[kernel_key]
        src = os.path.join(ROOT, "transformer_attention_tiled_amd", "csrc", rec["source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != rec["source_sha256_16"]:
            return None
        return int(rec["fetch_bytes"] + rec["write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline_prefill(p, heads=(0,)):
    """Time the oracle on whole query heads of the prefill; also return the
    parity of the GPU output on those heads."""
    import oracle

    q, k, v = p["cpu"]
    t0 = time.perf_counter()
    ref, _ = oracle.prefill(q, k, v, 1.0 / math.sqrt(p["d"]), causal=True, heads=list(heads))
    dt = time.perf_counter() - t0
    flops = causal_flops(p["B"], len(heads), p["T"], p["d"])
    got = p["o"].cpu().double().numpy()[:, list(heads)]
    err = np.abs(got - ref[:, list(heads)])
    return flops / dt / 1e12, dt, float(err.max()), float(err.mean())


def decode_parity(bd):
    import oracle

    b = bd["cpu"]
    ref, _ = oracle.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                                 b["seq_lens"], 1.0 / math.sqrt(b["q"].shape[-1]))
    err = np.abs(bd["o"].cpu().double().numpy() - ref)
    return float(err.max()), float(err.mean())


def machine_info(dev):
    """GPU name and compute units as the runtime reports them; XCDs derived
    from the compute units."""
    pr = torch.cuda.get_device_properties(dev)
    info = {"gpu": pr.name, "arch": getattr(pr, "gcnArchName", ""),
            "compute_units": pr.multi_processor_count,
            "hbm_gib": round(pr.total_memory / 2**30, 1)}
    # 32 compute units per XCD on MI355X
    info["xcds"] = max(1, pr.multi_processor_count // 32)
    return info


def probe_clock(dev, iters=20000):
    """Shader clock under dense bf16 MFMA load, from s_memtime / s_memrealtime
    (constant 100 MHz) of a pure MFMA loop on every SIMD, and the MFMA rate
    that loop reaches (libattn_probe.so; not the attention library)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "transformer_attention_tiled_amd", "libattn_probe.so"))
    lib.attn_probe_mfma_clock.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.zeros(3 * blocks * 4, dtype=torch.int64, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    res = None
    for _ in range(2):  # the first run warms the clock up
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        if lib.attn_probe_mfma_clock(ctypes.c_void_p(out.data_ptr()), blocks, iters, stream) != 0:
            return None
        e1.record()
        torch.cuda.synchronize()
        res = out.view(-1, 3).cpu().numpy()
        ms = e0.elapsed_time(e1)
    dt, dr = res[:, 0].astype(np.float64), res[:, 1].astype(np.float64)
    clock_ghz = float(dt.sum() / dr.sum() * 0.1)      # s_memrealtime counts at 100 MHz
    loop_s = float(dr.max()) / 1e8
    flops = blocks * 4 * iters * 8 * 2.0 * 32 * 32 * 16
    return {"mfma_loaded_clock_ghz": round(clock_ghz, 3),
            "mfma_loop_tflops": round(flops / loop_s / 1e12, 1),
            "mfma_loop_frac_of_2516": round(flops / loop_s / 1e12 / PEAK_BF16_TFLOPS, 4),
            "probe_ms_events": round(ms, 3), "probe_ms_realtime": round(loop_s * 1e3, 3)}


def copy_bandwidth(dev, nbytes=1 << 30, reps=5):
    """Read + write GB/s of a plain device-to-device copy of nbytes."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t = Timer()
    for _ in range(reps):
        e = t.start()
        dst.copy_(src)
        t.stop(e)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def measure_c2(dev, steps=50, warmup=10):
    """Causal prefill bf16, B=4, Hq=Hkv=16, T=2048, d=128 alone."""
    cfg = (4, 16, 16, 2048, 128, torch.bfloat16, 2)
    p = make_prefill(cfg, dev)
    for _ in range(warmup):
        run_prefill(p)
    torch.cuda.synchronize()
    t = Timer()
    for _ in range(steps):
        e = t.start()
        run_prefill(p)
        t.stop(e)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    tf = causal_flops(4, 16, 2048, 128) / (ms * 1e-3) / 1e12
    return {"workload": "causal prefill bf16 B=4 Hq=Hkv=16 T=2048 d=128", "ms": round(ms, 5),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": None}}


def measure_mixed(dev, ctx, steps=20, warmup=5):
    """The mixed paged batch: 8 chunks of 512 new tokens + 256 decodes with
    lengths uniform in [1024, 32768], Hq=32, Hkv=8, d=128, one attn_decode_paged
    call. ctx: each chunk also follows L - 512 cached tokens (L uniform in
    [1024, 32768]). Reported against the sum of the chunks' MFMA time and the
    K/V bytes' HBM time at peak (the step bound)."""
    n_chunks, n_dec = 8, 256
    b = inputs.mixed_batch_inputs(n_chunks, 512, n_dec, (1024, 32768), 32, 8, 128,
                                  seed=7 if ctx else 5, device=dev,
                                  chunk_len_range=(1024, 32768) if ctx else None)
    dec_lens = b["seq_lens_host"][n_chunks:]
    chunk_lens = b["seq_lens_host"][:n_chunks]
    b["o"] = torch.empty_like(b["q"])
    b["ws"] = torch.empty(attn.paged_workspace_size(
        n_chunks + n_dec, b["q"].shape[0], 32, 8, 128, b["max_seq_len"], b["max_query_len"],
        PARTITION), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        run_decode(b, with_qsl=True)
    torch.cuda.synchronize()
    t = Timer()
    for _ in range(steps):
        e = t.start()
        run_decode(b, with_qsl=True)
        t.stop(e)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    fl = sum(4.0 * 32 * 128 * (512 * (L - 512) + 512 * 513 / 2) for L in chunk_lens)
    kv = (sum(dec_lens) + sum(chunk_lens)) * 8 * 128 * 2 * 2
    qo = (n_chunks * 512 + n_dec) * 32 * 128 * 2 * 2
    bound_s = fl / (PEAK_BF16_TFLOPS * 1e12) + (kv + qo) / (PEAK_HBM_GBS * 1e9)
    del b
    torch.cuda.empty_cache()
    name = ("mixed paged batch bf16: 8 chunks x 512 new tokens" +
            (" after 512..32256 cached tokens" if ctx else "") +
            " + 256 decodes L~U[1024,32768], Hq=32 Hkv=8 d=128")
    return {"workload": name, "ms": round(ms, 4), "chunk_gflop": round(fl / 1e9, 2),
            "kv_gbytes": round(kv / 1e9, 3),
            "kv_gbs_whole_call": round(kv / (ms * 1e-3) / 1e9, 1),
            "roofline": {"bound": "mfma+hbm", "achieved": round(bound_s * 1e3, 4),
                         "peak": round(ms, 4), "unit": "ms (step bound at peak / measured)",
                         "frac": round(bound_s * 1e3 / ms, 4), "traffic": None}}


def headline(args, dev):
    P_CFG = (1, 32, 8, 16384, 128, torch.bfloat16, 3)
    D_CFG = dict(num_seqs=64, Hq=12, Hkv=2, d=128, lo=256, hi=4096, seed=4)
    p = make_prefill(P_CFG, dev)
    dsets = make_decode_sets(ROTATE, D_CFG["num_seqs"], D_CFG["Hq"], D_CFG["Hkv"], D_CFG["d"],
                             D_CFG["lo"], D_CFG["hi"], D_CFG["seed"], dev)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        run_prefill(p)
        run_decode(dsets[i % ROTATE])
    torch.cuda.synchronize()

    tp, td = Timer(), Timer()
    t_start = time.perf_counter()
    for i in range(args.steps):
        e = tp.start()
        run_prefill(p)
        tp.stop(e)
        e = td.start()
        run_decode(dsets[i % ROTATE])
        td.stop(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    ms_p, ms_d = tp.mean_ms(), td.mean_ms()
    fl = causal_flops(1, 32, 16384, 128)
    tflops = fl / (ms_p * 1e-3) / 1e12
    # decode: algorithmic bytes averaged over the rotated sets actually timed
    used = [dsets[i % ROTATE] for i in range(args.steps)]
    by = sum(decode_bytes(bd, 12, 2, 128) for bd in used) / len(used)
    gbs = by / (ms_d * 1e-3) / 1e9

    # parity on the timed outputs, and the oracle baseline (rank 0, N=1)
    run_decode(dsets[0])
    torch.cuda.synchronize()
    dmax, dmean = decode_parity(dsets[0])
    heads = tuple(range(0, 32, 2))  # 16 of the 32 query heads, every KV group
    cpu_tflops, cpu_s, pmax, pmean = cpu_baseline_prefill(p, heads=heads)

    # outside the timed region: the run's machine, its clock under MFMA load,
    # a plain copy's bandwidth, and the other configurations of the workload
    part = attn.decode_paged_partition_size(64, 2, max(bd["max_seq_len"] for bd in dsets))
    del dsets
    torch.cuda.empty_cache()
    meta = machine_info(dev)
    meta["copy_gbs_read_plus_write"] = copy_bandwidth(dev)
    clk = probe_clock(dev)
    if clk is not None:
        meta.update(clk)
    extra = {"c2": measure_c2(dev), "c5": measure_mixed(dev, ctx=False),
             "c5ctx": measure_mixed(dev, ctx=True)}

    return {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill bf16 B=1 Hq=32 Hkv=8 T=16384 d=128 + paged decode bf16 "
                        "64 seqs x 1 query Hq=12 Hkv=2 d=128 block 16 L~U[256,4096] "
                        f"({ROTATE} rotated KV pools)",
            "prefill": {"B": 1, "Hq": 32, "Hkv": 8, "T": 16384, "d": 128, "causal": True},
            "decode": {"num_seqs": 64, "Hq": 12, "Hkv": 2, "d": 128, "block_size": 16,
                       "seq_len_range": [256, 4096],
                       "partition_size": part},
        },
        "prefill": {"ms": round(ms_p, 4), "tflops": round(tflops, 2),
                    "frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                    "max_abs_err_sampled_heads": pmax, "mean_abs_err_sampled_heads": pmean},
        "decode": {"value": round(gbs, 1), "unit": "GB/s", "ms": round(ms_d, 5),
                   "bytes": int(by), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                   "max_abs_err": dmax, "mean_abs_err": dmean},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(
                         "prefill_pp_kernel<128,true> B=1 Hq=32 Hkv=8 T=16384")},
        "roofline_decode": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "traffic": measured_traffic(
                                "decode_kernel<128> 64 seqs Hq=12 Hkv=2 (mean of 8 rotated pools)")},
        "machine": meta,
        "other_configs": extra,
        "cpu_baseline": {"value": round(cpu_tflops, 5), "unit": "TFLOP/s", "cores": blas_threads(),
                         "kind": "oracle",
                         "sample": f"fp64 numpy oracle on the even query heads of the prefill "
                                   f"({len(heads)} of 32 heads, all 16384 rows each), "
                                   f"{cpu_s:.1f} s; credited causal FLOPs only"},
    }


def single(args, dev):
    """Time one configuration alone (prefill configs 1-3, decode 4, mixed 5)."""
    w = args.workload
    if w in ("c1", "c2", "c3"):
        cfg = {"c1": (1, 2, 2, 128, 64, torch.float32, 1),
               "c2": (4, 16, 16, 2048, 128, torch.bfloat16, 2),
               "c3": (1, 32, 8, 16384, 128, torch.bfloat16, 3)}[w]
        p = make_prefill(cfg, dev)
        for _ in range(args.warmup):
            run_prefill(p)
        torch.cuda.synchronize()
        t = Timer()
        for _ in range(args.steps):
            e = t.start()
            run_prefill(p)
            t.stop(e)
        torch.cuda.synchronize()
        ms = t.mean_ms()
        fl = causal_flops(cfg[0], cfg[1], cfg[3], cfg[4])
        peak = PEAK_F32_TFLOPS if cfg[5] == torch.float32 else PEAK_BF16_TFLOPS
        tf = fl / (ms * 1e-3) / 1e12
        return {"workload": w, "ms": round(ms, 5), "tflops": round(tf, 3),
                "frac_peak": round(tf / peak, 4), "flops": fl,
                "dtype": str(cfg[5]).replace("torch.", "")}
    if w == "c4":
        dsets = make_decode_sets(ROTATE, 64, 12, 2, 128, 256, 4096, 4, dev)
        for i in range(args.warmup):
            run_decode(dsets[i % ROTATE])
        torch.cuda.synchronize()
        t = Timer()
        for i in range(args.steps):
            e = t.start()
            run_decode(dsets[i % ROTATE])
            t.stop(e)
        torch.cuda.synchronize()
        ms = t.mean_ms()
        used = [dsets[i % ROTATE] for i in range(args.steps)]
        by = sum(decode_bytes(bd, 12, 2, 128) for bd in used) / len(used)
        gbs = by / (ms * 1e-3) / 1e9
        return {"workload": w, "ms": round(ms, 5), "gbs": round(gbs, 1),
                "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": int(by),
                "partition_size": PARTITION or
                attn.decode_paged_partition_size(64, 2, max(bd["max_seq_len"] for bd in dsets))}
    if w in ("c5", "c5ctx"):
        # 8 chunks of 512 new tokens + 256 decodes, lengths uniform in
        # [1024, 32768]; one shuffled pool on the GPU. c5: the chunks have no
        # prior context; c5ctx: each chunk's sequence is also 1024..32768
        # long, so it follows L - 512 cached tokens.
        n_chunks, n_dec = 8, 256
        ctx = w == "c5ctx"
        b = inputs.mixed_batch_inputs(n_chunks, 512, n_dec, (1024, 32768), 32, 8, 128,
                                      seed=7 if ctx else 5, device=dev,
                                      chunk_len_range=(1024, 32768) if ctx else None)
        dec_lens = b["seq_lens_host"][n_chunks:]
        chunk_lens = b["seq_lens_host"][:n_chunks]
        b["o"] = torch.empty_like(b["q"])
        b["ws"] = torch.empty(attn.paged_workspace_size(
            n_chunks + n_dec, b["q"].shape[0], 32, 8, 128, b["max_seq_len"], b["max_query_len"],
            PARTITION), dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            run_decode(b, with_qsl=True)
        torch.cuda.synchronize()
        t = Timer()
        for _ in range(args.steps):
            e = t.start()
            run_decode(b, with_qsl=True)
            t.stop(e)
        torch.cuda.synchronize()
        ms = t.mean_ms()
        # chunk flops: row i of a chunk after c cached tokens sees c + i + 1 keys
        fl = sum(4.0 * 32 * 128 * (512 * (L - 512) + 512 * 513 / 2) for L in chunk_lens)
        kv = (sum(dec_lens) + sum(chunk_lens)) * 8 * 128 * 2 * 2
        dec_kv = sum(dec_lens) * 8 * 128 * 2 * 2
        return {"workload": w, "ms": round(ms, 4), "partition_size": PARTITION,
                "chunk_gflop": round(fl / 1e9, 2), "chunk_flops": fl,
                "decode_kv_bytes": dec_kv, "chunk_kv_bytes": kv - dec_kv,
                "kv_gbytes": round(kv / 1e9, 3), "kv_gbs_whole_call": round(kv / (ms * 1e-3) / 1e9, 1)}
    if w in ("append", "append_decode"):
        # paged-cache append: "append" writes the mixed batch's new rows (8
        # chunks x 512 + 256 decodes, Hkv=8, d=128) into its ~17.9 GB pool;
        # "append_decode" one row per sequence of the 64-sequence decode batch
        # (Hkv=2, d=128, lengths uniform in [256, 4096]), 8 rotated pools.
        if w == "append":
            pools = [inputs.mixed_batch_inputs(8, 512, 256, (1024, 32768), 32, 8, 128, seed=5,
                                               device=dev)]
            Hkv = 8
        else:
            pools = make_decode_sets(ROTATE, 64, 12, 2, 128, 256, 4096, 4, dev)
            Hkv = 2
        rows = [inputs.new_kv_rows(b["q"].shape[0], Hkv, 128, 105 + i, device=dev)
                for i, b in enumerate(pools)]
        with_qsl = w == "append"

        def call(j):
            b, (kn, vn) = pools[j], rows[j]
            attn.kv_append(kn, vn, b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                           max_query_len=b["max_query_len"] if with_qsl else 1,
                           query_start_loc=b["query_start_loc"] if with_qsl else None)
        # the kernel is shorter than a Python-level call, so the calls are
        # captured in a HIP graph (static addresses, one submission per
        # replay) and the graph is replayed: the events then see GPU time
        per_graph = 8 * len(pools) if len(pools) > 1 else 16
        for j in range(len(pools)):
            call(j)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in range(per_graph):
                call(c % len(pools))
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t = Timer()
        for _ in range(args.steps):
            e = t.start()
            graph.replay()
            t.stop(e)
        torch.cuda.synchronize()
        ms = t.mean_ms() / per_graph
        nt = pools[0]["q"].shape[0]
        by = 2 * (2 * nt * Hkv * 128 * 2)  # K and V rows, each read once and written once
        return {"workload": w, "ms": round(ms, 5), "rows": nt, "bytes": by,
                "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if w in ("addnorm", "addnorm_decode"):
        # residual add + RMSNorm, bf16, hidden 4096 (32 heads x 128): 4096 rows
        # (a prefill chunk) or 256 rows (a decode batch); 4 rotated buffer sets
        # (~0.5 GB for 4096 rows, beyond the last-level cache). The calls are
        # replayed from a HIP graph, so the events see GPU time.
        rows, hidden = (4096, 4096) if w == "addnorm" else (256, 4096)
        sets = []
        for i in range(4):
            x, r, wt = inputs.norm_inputs(rows, hidden, 140 + i, device=dev)
            sets.append((x, r, wt, torch.empty_like(x), torch.empty_like(x)))

        def call(j):
            x, r, wt, y, h = sets[j]
            attn.add_rmsnorm(x, r, wt, 1e-6, out=y, residual_out=h)
        for j in range(4):
            call(j)
        torch.cuda.synchronize()
        per_graph = 16
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in range(per_graph):
                call(c % 4)
        for _ in range(max(1, args.warmup // 4)):
            graph.replay()
        torch.cuda.synchronize()
        t = Timer()
        for _ in range(max(1, args.steps // 4)):
            e = t.start()
            graph.replay()
            t.stop(e)
        torch.cuda.synchronize()
        ms = t.mean_ms() / per_graph
        by = 4 * rows * hidden * 2 + hidden * 2  # x, residual read; out, residual_out written
        return {"workload": w, "ms": round(ms, 5), "rows": rows, "hidden": hidden, "bytes": by,
                "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if w == "decode_step":
        # one serving decode step on the 64-sequence batch (Hq=12, Hkv=2,
        # d=128, lengths uniform in [256, 4096]): append the 64 new K/V rows
        # to the paged cache, then paged attention; 8 rotated pools. Timed
        # eagerly (events per step) and as a HIP graph of 8 steps (one per
        # pool) replayed.
        dsets = make_decode_sets(ROTATE, 64, 12, 2, 128, 256, 4096, 4, dev)
        rows = [inputs.new_kv_rows(64, 2, 128, 105 + i, device=dev) for i in range(ROTATE)]

        def step(j):
            bd, (kn, vn) = dsets[j], rows[j]
            attn.kv_append(kn, vn, bd["k_cache"], bd["v_cache"], bd["block_table"],
                           bd["seq_lens"])
            run_decode(bd)
        for i in range(args.warmup):
            step(i % ROTATE)
        torch.cuda.synchronize()
        t = Timer()
        for i in range(args.steps):
            e = t.start()
            step(i % ROTATE)
            t.stop(e)
        torch.cuda.synchronize()
        ms_eager = t.mean_ms()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for j in range(ROTATE):
                step(j)
        for _ in range(max(1, args.warmup // ROTATE)):
            graph.replay()
        torch.cuda.synchronize()
        t = Timer()
        reps = max(1, args.steps // ROTATE)
        for _ in range(reps):
            e = t.start()
            graph.replay()
            t.stop(e)
        torch.cuda.synchronize()
        ms_graph = t.mean_ms() / ROTATE
        by = sum(decode_bytes(bd, 12, 2, 128) for bd in dsets) / ROTATE + 2 * (2 * 64 * 2 * 128 * 2)
        return {"workload": w, "ms_eager": round(ms_eager, 5), "ms_graph": round(ms_graph, 5),
                "bytes": by, "gbs_graph": round(by / (ms_graph * 1e-3) / 1e9, 1),
                "frac_hbm_graph": round(by / (ms_graph * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if w == "copy":
        # plain 1 GiB device-to-device copy: the calibration for the HBM byte
        # counters (what FETCH_SIZE / WRITE_SIZE read for a known size)
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t = Timer()
        for _ in range(args.steps):
            e = t.start()
            dst.copy_(src)
            t.stop(e)
        torch.cuda.synchronize()
        ms = t.mean_ms()
        return {"workload": w, "bytes_each_way": n, "ms": round(ms, 4),
                "gbs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}
    raise SystemExit(f"unknown workload {w}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "c1", "c2", "c3", "c4", "c5", "c5ctx", "append",
                             "append_decode", "decode_step", "addnorm", "addnorm_decode",
                             "copy"])
    ap.add_argument("--partition-size", type=int, default=0,
                    help="split-KV partition length for decode (0: the library's choice)")
    args = ap.parse_args()
    global PARTITION
    PARTITION = args.partition_size
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the path is not sharded "
              "(see the multi-GPU design notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    attn.load_library()
    dev = torch.device("cuda:0")
    if args.workload == "headline":
        out = headline(args, dev)
    else:
        out = single(args, dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
