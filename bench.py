"""Benchmark of the paged KV write + paged attention path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the
step's KV_CACHE_WRITE followed by its PAGED_ATTENTION call (decode or prefill).
The headline line is the Llama-3-8B-shaped decode layer (64 sequences, 8 KV heads
of 128, pages of 16 tokens, bf16 KV, contexts U[512, 8192]) in KV GB/s; the
other configurations (batched and long-context prefill in f32 TFLOP/s, fp8 KV
decode in GB/s) are measured in the same run and reported under "secondary".

Inputs are resident in HBM before the timed region.  Each configuration:
W untimed warm-up steps, then exactly K timed steps bracketed by
torch.cuda.synchronize(); the attention call is also bracketed by HIP events on
the stream it runs on, which gives the dominant kernels' average duration for the
roofline object.  The CPU oracle is timed on a bounded sample of the headline
workload on this host ("cpu_baseline").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode KV GB/s + prefill f32 TFLOP/s, % of MI355X roofline"
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X dense f32 matrix, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "paged_kv_attention_cache_amd", "csrc"))):
        with open(os.path.join(ROOT, "paged_kv_attention_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(cfg: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if taken on this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(cfg)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def run_config(name: str, steps: int, warmup: int):
    import torch
    from paged_kv_attention_cache_amd import accounting as A
    from paged_kv_attention_cache_amd import runner as R
    from paged_kv_attention_cache_amd import workloads as W

    wl = W.make(name)
    t0 = time.time()
    pool = R.make_pool(wl, fill_byte=None)
    hist = R.write_history(pool, wl)
    step = R.DecodeStep(wl, pool) if wl.kind == "decode" else R.PrefillStep(wl, pool)
    torch.cuda.synchronize()
    log(f"[bench] {name}: pool {pool.nbytes() / 2**30:.2f} GiB, {hist} history tokens written "
        f"({time.time() - t0:.1f} s setup)")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step.write()
        ev[i][0].record(stream)
        step.attend()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ms_step = wall * 1e3 / steps

    if wl.kind == "decode":
        attn_bytes = A.decode_bytes(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size,
                                    wl.kv_dtype, wl.window)
        wr_bytes = A.write_bytes(step.slots.cpu().numpy(), wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
        res = {
            "workload": wl.name, "kind": "decode", "batch": wl.batch, "kv_dtype": wl.kv_dtype,
            "ms_per_step": ms_step, "attn_ms": attn_ms,
            "step_GBps": (attn_bytes + wr_bytes) / (ms_step * 1e-3) / 1e9,
            "attn_GBps": attn_bytes / (attn_ms * 1e-3) / 1e9,
            "attn_bytes": attn_bytes, "write_bytes": wr_bytes,
            "flops": A.decode_flops(wl.seq_lens, wl.num_q_heads, wl.head_dim, wl.window),
        }
        res["hbm_frac"] = res["attn_GBps"] / HBM_PEAK_GBPS
    else:
        pos = wl.row_positions()
        flops = A.prefill_flops(pos, wl.num_q_heads, wl.head_dim, wl.window)
        wr_bytes = A.write_bytes(step.slots.cpu().numpy(), wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
        res = {
            "workload": wl.name, "kind": "prefill", "batch": wl.batch, "tokens_per_row": wl.tokens_per_row,
            "window": wl.window, "kv_dtype": wl.kv_dtype, "ms_per_step": ms_step, "attn_ms": attn_ms,
            "flops": flops, "write_bytes": wr_bytes,
            "attn_TFLOPs": flops / (attn_ms * 1e-3) / 1e12,
            "step_TFLOPs": flops / (ms_step * 1e-3) / 1e12,
        }
        res["mfma_frac"] = res["attn_TFLOPs"] / MFMA_F32_PEAK_TFLOPS
    del step, pool
    torch.cuda.empty_cache()
    return wl, res


def cpu_baseline(seqs: int = 6):
    """The oracle on a bounded sample of the headline decode workload, on this host."""
    from threadpoolctl import threadpool_limits

    import oracle
    from paged_kv_attention_cache_amd import accounting as A
    from paged_kv_attention_cache_amd import workloads as W

    wl = W.make("c2")
    picks = list(range(seqs))
    lens = wl.seq_lens[picks]
    # inputs are drawn before the timer starts
    kv = [wl.seq_kv(b) for b in picks]
    q = wl.decode_q()
    with threadpool_limits(1):
        t0 = time.perf_counter()
        pool = oracle.KVPool(wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
        for b, (k, v) in zip(picks, kv):
            pool.write(k, v, wl.slots_for(b, np.arange(int(wl.seq_lens[b]))))
        oracle.decode(pool, q, wl.block_tables, wl.seq_lens, 0, wl.scale, seqs=picks)
        dt = time.perf_counter() - t0
    nbytes = A.decode_bytes(lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.kv_dtype)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{seqs} of the 64 sequences of the headline decode workload ({int(lens.sum())} positions): "
                      f"pool write of their K/V then decode attention, numpy f64, one thread; {dt:.1f} s",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--configs", default="c2,c3,c4,c4w,c5",
                    help="comma list; the first is the headline (default c2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the kernels would shard by sequence or KV head with no exchange); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import paged_kv_attention_cache_amd as tl
    tl.lib()

    names = [c.strip() for c in args.configs.split(",") if c.strip()]
    results = {}
    for n in names:
        wl, r = run_config(n, args.steps, args.warmup)
        results[n] = (wl, r)
        log(f"[bench] {n}: " + json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}))

    head_wl, head = results[names[0]]
    if head["kind"] == "decode":
        value, unit = head["step_GBps"], "GB/s"
        per_launch = head["attn_bytes"]
        roof = {"bound": "hbm", "achieved": head["attn_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": head["attn_GBps"] / HBM_PEAK_GBPS,
                "kernel": "decode split + merge kernels (one tl_paged_attn_decode call)",
                "per_launch_bytes": per_launch}
    else:
        value, unit = head["step_TFLOPs"], "TFLOP/s"
        roof = {"bound": "mfma", "achieved": head["attn_TFLOPs"], "peak": MFMA_F32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": head["attn_TFLOPs"] / MFMA_F32_PEAK_TFLOPS,
                "kernel": "prefill kernel (one tl_paged_attn_prefill call)", "per_launch_flops": head["flops"]}
    roof["traffic"] = traffic_record(names[0])

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": head_wl.name, "batch": head_wl.batch, "num_q_heads": head_wl.num_q_heads,
                   "num_kv_heads": head_wl.num_kv_heads, "head_dim": head_wl.head_dim,
                   "page_size": head_wl.page_size, "kv_dtype": head_wl.kv_dtype, "parallelism": "none"},
        "roofline": roof,
    }
    line["secondary"] = {n: r for n, (_, r) in results.items() if n != names[0]}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
