"""Per-configuration report: GPU time, throughput, fraction of the roofline,
max / mean absolute error against the oracle and the oracle's own time on
this host, one JSON line per configuration.

    python tests/report_configs.py [c1 c2 c3 c4 c5]

c1-c3: contiguous causal prefill (fp32 B=1 Hq=Hkv=2 T=128 d=64; bf16 B=4
Hq=Hkv=16 T=2048 d=128; bf16 B=1 Hq=32 Hkv=8 T=16384 d=128, oracle on query
heads 0, 3, 4, 31, its time scaled to all 32 heads). c4: paged decode, 64
sequences, Hq=12 Hkv=2 d=128, lengths uniform in [256, 4096], 8 rotated
pools. c5: one mixed call, 8 chunks of 512 new tokens + 256 decodes with
lengths uniform in [1024, 32768], Hq=32 Hkv=8 d=128; the oracle checks every
chunk and 16 decode sequences (shortest, longest, 14 seeded), its decode time
scaled by the ratio of summed lengths. Needs a GPU.
"""
import json, math, os, sys, time
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))
import numpy as np
import torch
import bench
import oracle
import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import inputs

dev = torch.device("cuda")
cores = len(os.sched_getaffinity(0))
print("cores", cores, flush=True)


def timed(fn, warm, steps):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t = bench.Timer()
    for _ in range(steps):
        e = t.start()
        fn()
        t.stop(e)
    torch.cuda.synchronize()
    return t.mean_ms()


which = sys.argv[1:] or ["c1", "c2", "c3", "c4", "c5"]
for w in which:
    if w in ("c1", "c2", "c3"):
        cfg = {"c1": (1, 2, 2, 128, 64, torch.float32, 1),
               "c2": (4, 16, 16, 2048, 128, torch.bfloat16, 2),
               "c3": (1, 32, 8, 16384, 128, torch.bfloat16, 3)}[w]
        heads = [0, 3, 4, 31] if w == "c3" else None
        p = bench.make_prefill(cfg, dev)
        ms = timed(lambda: bench.run_prefill(p), 10, 100 if w != "c3" else 30)
        fl = bench.causal_flops(cfg[0], cfg[1], cfg[3], cfg[4])
        peak = bench.PEAK_F32_TFLOPS if cfg[5] == torch.float32 else bench.PEAK_BF16_TFLOPS
        tf = fl / (ms * 1e-3) / 1e12
        q, k, v = p["cpu"]
        t0 = time.perf_counter()
        ref, _ = oracle.prefill(q, k, v, 1.0 / math.sqrt(cfg[4]), causal=True, heads=heads)
        dt = time.perf_counter() - t0
        got = p["o"].float().cpu().double().numpy()
        if heads is not None:
            got, ref = got[:, heads], ref[:, heads]
            dt_full = dt * cfg[1] / len(heads)
        else:
            dt_full = dt
        err = np.abs(got - ref)
        print(json.dumps({"config": w, "ms": round(ms, 5), "tflops": round(tf, 2),
                          "frac": round(tf / peak, 4), "max_err": float(err.max()),
                          "mean_err": float(err.mean()), "oracle_s": round(dt, 2),
                          "oracle_s_full": round(dt_full, 2),
                          "oracle_sample": "heads %s" % heads if heads else "full"}), flush=True)
        del p
        torch.cuda.empty_cache()
    elif w == "c4":
        dsets = bench.make_decode_sets(8, 64, 12, 2, 128, 256, 4096, 4, dev)
        i = [0]

        def one():
            bench.run_decode(dsets[i[0] % 8])
            i[0] += 1
        ms = timed(one, 16, 400)
        by = sum(bench.decode_bytes(bd, 12, 2, 128) for bd in dsets) / 8
        bench.run_decode(dsets[0])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        mx, mean = bench.decode_parity(dsets[0])
        dt = time.perf_counter() - t0
        gbs = by / (ms * 1e-3) / 1e9
        print(json.dumps({"config": w, "ms": round(ms, 5), "gbs": round(gbs, 1),
                          "frac": round(gbs / bench.PEAK_HBM_GBS, 4), "bytes": by,
                          "max_err": mx, "mean_err": mean, "oracle_s": round(dt, 2)}), flush=True)
        del dsets
        torch.cuda.empty_cache()
    elif w == "c5":
        b = inputs.mixed_batch_inputs(8, 512, 256, (1024, 32768), 32, 8, 128, seed=5, device=dev)
        o = torch.empty_like(b["q"])
        lse = torch.full(tuple(b["q"].shape[:2]), float("nan"), device=dev)
        ws = torch.empty(attn.decode_paged_workspace_size(264, 32, 8, 128, b["max_seq_len"], 0),
                         dtype=torch.uint8, device=dev)

        def one():
            attn.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                              max_seq_len=b["max_seq_len"], max_query_len=b["max_query_len"],
                              query_start_loc=b["query_start_loc"], o=o, lse=lse, workspace=ws)
        ms = timed(one, 3, 20)
        torch.cuda.synchronize()
        lens = b["seq_lens_host"]
        dec = list(range(8, 264))
        kv = sum(lens[8:]) * 8 * 128 * 2 * 2 + 8 * 512 * 8 * 128 * 2 * 2
        rng = np.random.default_rng(5)
        pick = {min(dec, key=lambda n: lens[n]), max(dec, key=lambda n: lens[n])}
        pick |= set(int(x) for x in rng.choice(dec, 14, replace=False))
        seqs = list(range(8)) + sorted(pick)
        kc, vc, table, sl, q, qsl = inputs.compact_sequences(b, seqs)
        t0 = time.perf_counter()
        ro, rl = oracle.decode_paged(q, kc, vc, table, sl, 1.0 / math.sqrt(128),
                                     query_start_loc=qsl, seqs=list(range(8)))
        t_chunks = time.perf_counter() - t0
        t0 = time.perf_counter()
        ro2, _ = oracle.decode_paged(q, kc, vc, table, sl, 1.0 / math.sqrt(128),
                                     query_start_loc=qsl, seqs=list(range(8, len(seqs))))
        t_dec = time.perf_counter() - t0
        ro[np.isnan(ro)] = ro2[np.isnan(ro)]
        qsl_full = b["query_start_loc"].cpu()
        rows = torch.cat([torch.arange(int(qsl_full[n]), int(qsl_full[n + 1])) for n in seqs])
        got = o[rows.to(dev)].float().cpu().double().numpy()
        err = np.abs(got - ro)
        sampled_L = sum(lens[n] for n in sorted(pick))
        dt_full = t_chunks + t_dec * sum(lens[8:]) / sampled_L
        print(json.dumps({"config": w, "ms": round(ms, 4), "kv_gbytes": round(kv / 1e9, 3),
                          "kv_gbs": round(kv / (ms * 1e-3) / 1e9, 1),
                          "frac": round(kv / (ms * 1e-3) / 1e9 / bench.PEAK_HBM_GBS, 4),
                          "chunk_gflop": round(8 * bench.causal_flops(1, 32, 512, 128) / 1e9, 2),
                          "max_err": float(err.max()), "mean_err": float(err.mean()),
                          "oracle_s_chunks": round(t_chunks, 2), "oracle_s_dec16": round(t_dec, 2),
                          "oracle_s_full_extrap": round(dt_full, 2)}), flush=True)
        del b
        torch.cuda.empty_cache()
