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


KERNEL_SOURCES = ("tl_decode.hip", "tl_prefill.hip", "tl_write.hip", "tl_gdn.hip", "tl_internal.h")


def kernel_source_hash() -> str:
    """Hash of the sources of the measured kernels (the traffic record is valid while it matches)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
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

    hist_write = history_write_rate(wl, pool) if wl.kind == "decode" else None

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
        res.update(hist_write)
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


def run_gdn(name: str, steps: int, warmup: int):
    """GATED_DELTA_RULE decode steps over the workload's state pool (each step reads and
    writes every live row's [H, 128, 128] f32 state): KV-style GB/s of the call."""
    import torch
    from paged_kv_attention_cache_amd import tl_gated_delta_rule_decode
    from paged_kv_attention_cache_amd import workloads as W
    wl = W.make(name)
    pool = torch.from_numpy(wl.initial_pool()).cuda()
    slots, pos = wl.slots_positions()
    ins = [torch.from_numpy(x).cuda() for x in wl.step_inputs(0)]
    st, pt = torch.from_numpy(slots).cuda(), torch.from_numpy(pos).cuda()
    out = torch.empty_like(ins[2])
    for _ in range(warmup):
        tl_gated_delta_rule_decode(pool, *ins, st, pt, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        tl_gated_delta_rule_decode(pool, *ins, st, pt, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    live = int(np.count_nonzero(slots >= 0))
    fresh = int(np.count_nonzero((slots >= 0) & (pos == 0)))
    D, H = wl.head_dim, wl.num_heads
    # state read (not for fresh rows) and written, q k v read and o written, g and beta, slots, positions
    nbytes = (live * 2 - fresh) * H * D * D * 4 + wl.batch * H * (4 * D * 4 + 8) + wl.batch * 8
    return wl, {"kind": "gdn", "workload": wl.name, "attn_ms": ms, "attn_bytes": nbytes,
                "attn_GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "ms_per_step": wall * 1e3 / steps}


def history_write_rate(wl, pool, reps: int = 10):
    """KV_CACHE_WRITE throughput on the workload's first history chunk (up to 64K tokens):
    the same rows rewritten to the same slots, timed with HIP events."""
    import torch
    from paged_kv_attention_cache_amd import accounting as A
    from paged_kv_attention_cache_amd import runner as R
    from paged_kv_attention_cache_amd import tl_kv_cache_write
    k, v, slots = next(wl.history_batches())
    dk, dv, ds = R._t(k, "cuda"), R._t(v, "cuda"), R._t(slots, "cuda")
    for _ in range(2):
        tl_kv_cache_write(pool, dk, dv, ds)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        tl_kv_cache_write(pool, dk, dv, ds)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = A.write_bytes(slots, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    return {"hist_write_tokens": int(len(slots)), "hist_write_bytes": nbytes, "hist_write_ms": ms,
            "hist_write_GBps": nbytes / (ms * 1e-3) / 1e9}


def cpu_baseline(target_s: float = 12.0, cap_s: float = 30.0):
    """The oracle on a time-bounded sample of the headline decode workload, on this host.

    Sequences of the workload are processed in order, each one's pool write then its
    decode attention, until about target_s seconds of CPU work (passes over the whole
    batch repeat if one pass is shorter); the rate uses the same algorithmic bytes as
    the GPU figure."""
    from threadpoolctl import threadpool_limits

    import oracle
    from paged_kv_attention_cache_amd import accounting as A
    from paged_kv_attention_cache_amd import workloads as W

    wl = W.make("c2")
    q = wl.decode_q()
    done, positions, nbytes, dt = 0, 0, 0, 0.0
    pool = oracle.KVPool(wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)  # resident, untimed
    with threadpool_limits(1):
        while dt < target_s and dt < cap_s:
            b = done % wl.batch
            k, v = wl.seq_kv(b)  # inputs are drawn outside the timed part
            t0 = time.perf_counter()
            pool.write(k, v, wl.slots_for(b, np.arange(int(wl.seq_lens[b]))))
            oracle.decode(pool, q, wl.block_tables, wl.seq_lens, 0, wl.scale, seqs=[b])
            dt += time.perf_counter() - t0
            done += 1
            positions += int(wl.seq_lens[b])
            nbytes += A.decode_bytes(wl.seq_lens[b:b + 1], wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                     wl.page_size, wl.kv_dtype)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} sequence-steps of the headline decode workload (sequences in order, "
                      f"{positions} positions): each one's pool write then its decode attention, numpy f64, "
                      f"one thread; {dt:.1f} s",
            "seconds": dt}


# ------------------------------------------------------------------ rocprofv3 summaries
# These modes make no GPU call except --copy-calibration; they turn the CSV output of
# rocprofv3 runs of this file into the short text summaries kept under profiles/.

ATTN_KERNELS = ("decode_split_kernel", "decode_merge_kernel", "prefill_kernel", "gdn_decode_kernel")


def _short_name(name: str) -> str:
    for k in ATTN_KERNELS + ("write_kernel", "gather_kernel"):
        if k in name:
            return name[name.index(k):].split("(tl::")[0]
    return name[:60]


def _find_csv(d: str, suffix: str) -> str:
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _counter_means(d: str, counter: str):
    """Mean counter value (KiB) and dispatch count per kernel name in one --pmc run."""
    import csv
    acc = {}
    for r in csv.DictReader(open(_find_csv(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def copy_calibration(gib: int = 1, reps: int = 3):
    """A plain device-to-device copy of known size, run under rocprofv3 --pmc to scale
    FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    n = gib << 28
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    x.fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "reps": reps}), flush=True)


def traffic_summary(cfg: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                    command: str):
    """Scale FETCH_SIZE / WRITE_SIZE of the attention kernels by the copy calibration and
    record bytes per attention call in profiles/traffic.json (keyed by workload)."""
    copy_bytes = 1 << 30
    cf = max(v[0] for v in _counter_means(copy_fetch_dir, "FETCH_SIZE").values()) * 1024
    cw = max(v[0] for v in _counter_means(copy_write_dir, "WRITE_SIZE").values()) * 1024
    f_fetch, f_write = copy_bytes / cf, copy_bytes / cw
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    lines = [f"# HBM traffic per attention call, workload {cfg}", "",
             f"command (FETCH_SIZE, then again with WRITE_SIZE): {command}",
             f"calibration: a 1 GiB device copy (python bench.py --copy-calibration under the same "
             f"rocprofv3 --pmc) reads {cf / 1024:.0f} KiB and writes {cw / 1024:.0f} KiB per dispatch -> "
             f"FETCH_SIZE x {f_fetch:.3f}, WRITE_SIZE x {f_write:.3f}", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (scaled) | written bytes (scaled) |",
             "|---|---|---|---|---|---|"]
    total_r = total_w = 0.0
    for name in sorted(fetch):
        short = _short_name(name)
        if not any(k in name for k in ATTN_KERNELS):
            continue
        fr, n = fetch[name]
        wr = write.get(name, (0.0, 0))[0]
        rb, wb = fr * 1024 * f_fetch, wr * 1024 * f_write
        total_r += rb
        total_w += wb
        lines.append(f"| {short} | {n} | {fr:.0f} | {wr:.0f} | {rb / 1e9:.4f} GB | {wb / 1e9:.4f} GB |")
    lines.append(f"| attention call total | | | | {total_r / 1e9:.4f} GB | {total_w / 1e9:.4f} GB |")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec[cfg] = {"source_hash": kernel_source_hash(), "bytes_per_launch": total_r + total_w,
                "read_bytes": total_r, "written_bytes": total_w,
                "fetch_factor": f_fetch, "write_factor": f_write}
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print("\n".join(lines))


def stats_summary(d: str, configs: str, calls: str, command: str):
    """Per-kernel durations from rocprofv3 --kernel-trace of one bench run, per workload.

    The run executes the workloads in the order given, each making `calls` attention
    calls (warm-up + timed); dispatches of the attention kernels are assigned to the
    workloads in that order."""
    import csv
    rows = sorted(csv.DictReader(open(_find_csv(d, "kernel_trace.csv"))), key=lambda r: int(r["Start_Timestamp"]))
    n = int(calls)
    att = [r for r in rows if any(k in r["Kernel_Name"] for k in ATTN_KERNELS)]
    mains = [i for i, r in enumerate(att) if any(k in r["Kernel_Name"] for k in
                                                 ("decode_split_kernel", "prefill_kernel", "gdn_decode_kernel"))]
    print(f"command: {command}\n")
    print("Durations from the kernel trace (rocprofv3 --kernel-trace --stats), grouped by workload.\n")
    print("| workload | kernel | calls | average us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for ci, cfg in enumerate(configs.split(",")):
        blk = mains[ci * n:(ci + 1) * n]
        if not blk:
            break
        lo = blk[0]
        hi = mains[(ci + 1) * n] if (ci + 1) * n < len(mains) else len(att)
        per = {}
        for r in att[lo:hi]:
            per.setdefault(_short_name(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        call_total = 0.0
        for k, v in per.items():
            call_total += sum(v) / len(v)
            print(f"| {cfg} | {k} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
        print(f"| {cfg} | whole attention call (sum of averages) | | {call_total:.1f} | | |")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-summary":
        traffic_summary(*sys.argv[2:8])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--stats-summary":
        stats_summary(*sys.argv[2:6])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--copy-calibration":
        copy_calibration()
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--configs", default="c2,c3,c4,c4w,c5,c2r,c5u,c2i,c6",
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
        wl, r = run_gdn(n, args.steps, args.warmup) if n == "c6" else run_config(n, args.steps, args.warmup)
        results[n] = (wl, r)
        log(f"[bench] {n}: " + json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}))

    head_wl, head = results[names[0]]
    if head["kind"] == "gdn":  # (only when the state-pool workload is run first)
        value, unit = head["attn_bytes"] / (head["ms_per_step"] * 1e-3) / 1e9, "GB/s"
        roof = {"bound": "hbm", "achieved": head["attn_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": head["attn_GBps"] / HBM_PEAK_GBPS, "kernel": "gdn_decode_kernel",
                "per_launch_bytes": head["attn_bytes"]}
    elif head["kind"] == "decode":
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
        "config": ({"workload": head_wl.name, "batch": head_wl.batch, "num_heads": head_wl.num_heads,
                    "head_dim": head_wl.head_dim, "num_slots": head_wl.num_slots, "parallelism": "none"}
                   if head["kind"] == "gdn" else
                   {"workload": head_wl.name, "batch": head_wl.batch, "num_q_heads": head_wl.num_q_heads,
                    "num_kv_heads": head_wl.num_kv_heads, "head_dim": head_wl.head_dim,
                    "page_size": head_wl.page_size, "kv_dtype": head_wl.kv_dtype, "parallelism": "none"}),
        "roofline": roof,
    }
    line["secondary"] = {n: r for n, (_, r) in results.items() if n != names[0]}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
