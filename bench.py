"""Benchmark of the paged KV write + paged attention path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the
step's KV_CACHE_WRITE followed by its PAGED_ATTENTION call (decode or prefill).
The headline line is the Llama-3-8B-shaped decode layer (64 sequences, 8 KV heads
of 128, pages of 16 tokens, bf16 KV, contexts U[512, 8192]) in KV GB/s; the
other configurations (batched and long-context prefill in f32 TFLOP/s, fp8 KV
decode in GB/s) are measured in the same run and reported under "secondary".

Inputs are resident in HBM before the timed region.  Each configuration:
W untimed warm-up steps, then exactly K timed steps back to back, bracketed by
torch.cuda.synchronize() (wall clock: "value" and "ms_per_step"; a decode step is
captured once as a HIP graph of its two launches and replayed, as a serving loop
does, and the eagerly launched steps' time is reported beside it), then K more
attention calls each timed alone with HIP events on the stream it runs on, after a
512 MiB cache-evicting read: their median gives the roofline object (the
back-to-back mean is reported beside it).  The CPU oracle is timed on a bounded
sample of the headline workload on this host's cores ("cpu_baseline").
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
    """Hash of the sources of the measured kernels and of the flags they are built with
    (the traffic record is valid while it matches)."""
    from paged_kv_attention_cache_amd import _build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_attention_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(_build.HIP_FLAGS).encode())
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


FLUSH_BYTES = 512 << 20  # larger than the 256 MB last-level cache (MALL) plus the L2s


def timed_steps(write, attend, steps: int):
    """The contract loop: exactly `steps` back-to-back steps (the step's write, then its
    attention call) between synchronisations, wall clock; the attention calls are also
    bracketed by HIP events on their stream.  Returns (ms per step, mean attention ms)."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if write is not None:
            write()
        ev[i][0].record(stream)
        attend()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, float(np.mean([a.elapsed_time(b) for a, b in ev]))


def graph_steps(graph, steps: int):
    """The contract loop with each step replayed as one captured HIP graph (the step's
    write, then its attention call), as a serving loop replays a captured decode step:
    exactly `steps` replays between synchronisations, wall clock, ms per step."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def capture_step(step):
    """Capture step.run() in a graph and check that a replay gives the eager step's
    output bit for bit (the step is idempotent: the same rows to the same slots)."""
    import torch
    step.run()
    torch.cuda.synchronize()
    ref = step.out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    step.out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(step.out, ref):
        raise RuntimeError("graph replay of the decode step differs from the eager step")
    return graph


_flush = None


def _flush_caches():
    """Read FLUSH_BYTES of scratch with plain (cache-allocating) loads: every line an
    earlier call left in the L2s or the MALL is evicted, and dirty ones are written
    back now, not during the next timed call (a flush that wrote its scratch would
    leave its own dirty lines to be written back inside the timed call)."""
    import ctypes
    import torch
    global _flush
    if _flush is None:
        from paged_kv_attention_cache_amd import _build
        L = ctypes.CDLL(_build.STREAM_LIB)
        L.tl_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
        _flush = (L, torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda"),
                  torch.zeros(1, dtype=torch.int32, device="cuda"))
    L, buf, sink = _flush
    rc = L.tl_stream_read(buf.data_ptr(), FLUSH_BYTES, sink.data_ptr(), 0, 2048, torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"tl_stream_read: HIP error {rc}")


def flushed_calls(attend, calls: int):
    """Each attention call timed alone with HIP events on its stream, after FLUSH_BYTES of
    scratch have been read (untimed), so that no input is served from a cache the
    previous call filled.  Returns median, min and mean milliseconds."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for i in range(calls):
        _flush_caches()
        ev[i][0].record(stream)
        attend()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median_ms": float(np.median(ms)), "min_ms": float(ms.min()), "mean_ms": float(ms.mean()),
            "calls": calls}


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
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    ms_step_eager, attn_back_to_back = timed_steps(step.write, step.attend, steps)
    ms_step, step_mode = ms_step_eager, "eager"
    if wl.kind == "decode":  # launch-bound: the step runs as one replayed graph
        try:
            graph = capture_step(step)
            for _ in range(warmup):
                graph.replay()
            ms_step, step_mode = graph_steps(graph, steps), "graph"
            del graph
        except RuntimeError as e:  # reported, and the eager steps stand
            log(f"[bench] {name}: graph capture not used ({e}); eager steps")
            step.run()
            torch.cuda.synchronize()
    attn = flushed_calls(step.attend, steps)
    attn_ms = attn["median_ms"]

    hist_write = history_write_rate(wl, pool) if wl.kind == "decode" else None

    if wl.kind == "decode":
        attn_bytes = A.decode_bytes(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size,
                                    wl.kv_dtype, wl.window)
        wr_bytes = A.write_bytes(step.slots.cpu().numpy(), wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
        res = {
            "workload": wl.name, "kind": "decode", "batch": wl.batch, "kv_dtype": wl.kv_dtype,
            "ms_per_step": ms_step, "ms_per_step_eager": ms_step_eager, "step_mode": step_mode, "attn_ms": attn_ms,
            "attn_ms_min": attn["min_ms"], "attn_ms_back_to_back": attn_back_to_back,
            "step_GBps": (attn_bytes + wr_bytes) / (ms_step * 1e-3) / 1e9,
            "attn_GBps": attn_bytes / (attn_ms * 1e-3) / 1e9,
            "attn_bytes": attn_bytes, "write_bytes": wr_bytes,
            "flops": A.decode_flops(wl.seq_lens, wl.num_q_heads, wl.head_dim, wl.window),
        }
        res["hbm_frac"] = res["attn_GBps"] / HBM_PEAK_GBPS
        res["hbm_frac_min"] = attn_bytes / (attn["min_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS
        res["hbm_frac_back_to_back"] = attn_bytes / (attn_back_to_back * 1e-3) / 1e9 / HBM_PEAK_GBPS
        res.update(hist_write)
    else:
        pos = wl.row_positions()
        flops = A.prefill_flops(pos, wl.num_q_heads, wl.head_dim, wl.window)
        wr_bytes = A.write_bytes(step.slots.cpu().numpy(), wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
        res = {
            "workload": wl.name, "kind": "prefill", "batch": wl.batch, "tokens_per_row": wl.tokens_per_row,
            "window": wl.window, "kv_dtype": wl.kv_dtype, "ms_per_step": ms_step, "attn_ms": attn_ms,
            "attn_ms_min": attn["min_ms"], "attn_ms_back_to_back": attn_back_to_back,
            "flops": flops, "write_bytes": wr_bytes,
            "attn_TFLOPs": flops / (attn_ms * 1e-3) / 1e12,
            "step_TFLOPs": flops / (ms_step * 1e-3) / 1e12,
        }
        res["mfma_frac"] = res["attn_TFLOPs"] / MFMA_F32_PEAK_TFLOPS
        res["mfma_frac_back_to_back"] = flops / (attn_back_to_back * 1e-3) / 1e12 / MFMA_F32_PEAK_TFLOPS
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
    def call():
        tl_gated_delta_rule_decode(pool, *ins, st, pt, out=out)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ms_step, back_to_back = timed_steps(None, call, steps)
    attn = flushed_calls(call, steps)  # the 168 MB state pool would otherwise stay in the MALL
    ms = attn["median_ms"]
    live = int(np.count_nonzero(slots >= 0))
    fresh = int(np.count_nonzero((slots >= 0) & (pos == 0)))
    D, H = wl.head_dim, wl.num_heads
    # state read (not for fresh rows) and written, q k v read and o written, g and beta, slots, positions
    nbytes = (live * 2 - fresh) * H * D * D * 4 + wl.batch * H * (4 * D * 4 + 8) + wl.batch * 8
    return wl, {"kind": "gdn", "workload": wl.name, "attn_ms": ms, "attn_ms_min": attn["min_ms"],
                "attn_ms_back_to_back": back_to_back, "attn_bytes": nbytes,
                "attn_GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "hbm_frac_back_to_back": nbytes / (back_to_back * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "ms_per_step": ms_step}


def history_write_rate(wl, pool, reps: int = 10, warmup: int = 2):
    """KV_CACHE_WRITE throughput on the workload's first history chunk (up to 64K tokens):
    the same rows rewritten to the same slots, timed with HIP events."""
    import torch
    from paged_kv_attention_cache_amd import accounting as A
    from paged_kv_attention_cache_amd import runner as R
    from paged_kv_attention_cache_amd import tl_kv_cache_write
    k, v, slots = next(wl.history_batches())
    dk, dv, ds = R._t(k, "cuda"), R._t(v, "cuda"), R._t(slots, "cuda")

    def call():
        tl_kv_cache_write(pool, dk, dv, ds)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t = flushed_calls(call, reps)
    ms = t["median_ms"]
    nbytes = A.write_bytes(slots, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    return {"hist_write_tokens": int(len(slots)), "hist_write_bytes": nbytes, "hist_write_ms": ms,
            "hist_write_ms_min": t["min_ms"], "hist_write_GBps": nbytes / (ms * 1e-3) / 1e9,
            "hist_write_hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}


_CPU_WL = None


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    global _CPU_LIMIT
    _CPU_LIMIT = threadpool_limits(1)  # one BLAS thread per worker process


def _cpu_sequence_step(b: int):
    """One sequence-step of the headline decode workload on the oracle: the sequence's
    pool write, then its decode attention.  The sequence's own pages form the pool (in
    the workload's shuffled order); its inputs are drawn before the clock starts."""
    import oracle
    from paged_kv_attention_cache_amd import accounting as A
    from paged_kv_attention_cache_amd import workloads as W
    global _CPU_WL
    if _CPU_WL is None:
        _CPU_WL = W.make("c2")
    wl = _CPU_WL
    L, S = int(wl.seq_lens[b]), wl.page_size
    n = -(-L // S)
    local = np.argsort(np.argsort(wl.block_tables[b, :n])).astype(np.int32)  # page ranks: the same shuffle
    table = np.full((1, wl.max_blocks), -1, np.int32)
    table[0, :n] = local
    slots = (local[np.arange(L) // S] * S + np.arange(L) % S).astype(np.int32)
    k, v = wl.seq_kv(b)
    q = wl.decode_q(b)[None]
    pool = oracle.KVPool(n, S, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    t0 = time.perf_counter()
    pool.write(k, v, slots)
    oracle.decode(pool, q, table, wl.seq_lens[b:b + 1], 0, wl.scale)
    dt = time.perf_counter() - t0
    nbytes = A.decode_bytes(wl.seq_lens[b:b + 1], wl.num_q_heads, wl.num_kv_heads, wl.head_dim, S, wl.kv_dtype)
    return os.getpid(), dt, nbytes, L


def cpu_baseline(target_s: float = 12.0, cap_s: float = 60.0):
    """The oracle on a time-bounded sample of the headline decode workload, on this host's
    cores: one worker process per core this process may use (at most 16, the host share
    of one GPU), each with one BLAS thread, taking sequence-steps in order (passes over
    the batch repeat) until the busiest worker has spent about target_s seconds.  The rate
    is the sample's algorithmic bytes (as for the GPU figure) over that busiest worker's
    compute time, i.e. the time of a run in which all workers start together."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    batch = 64
    busy, nbytes, done, positions = {}, 0, 0, 0
    t_start = time.perf_counter()
    with ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn"), initializer=_cpu_worker_init) as ex:
        while (not busy or max(busy.values()) < target_s) and time.perf_counter() - t_start < cap_s:
            futs = [ex.submit(_cpu_sequence_step, (done + i) % batch) for i in range(2 * cores)]
            for f in futs:
                pid, dt, nb, L = f.result()
                busy[pid] = busy.get(pid, 0.0) + dt
                nbytes += nb
                positions += L
            done += len(futs)
    t = max(busy.values())
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": len(busy), "kind": "oracle",
            "sample": f"{done} sequence-steps of the headline decode workload (sequences in order, passes "
                      f"repeating; {positions} positions): each one's pool write then its decode attention, "
                      f"numpy f64, on {len(busy)} worker processes of one BLAS thread each; busiest worker "
                      f"{t:.1f} s of compute (inputs drawn outside the clock)",
            "seconds": t}


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


def write_bench(configs: str, steps: int = 20, warmup: int = 2):
    """KV_CACHE_WRITE alone on each workload's first history chunk (up to 64K tokens; the
    same rows to the same slots every call), so that a rocprofv3 run sees only identical
    write_kernel dispatches (besides the cache-evicting reads between calls)."""
    import torch
    from paged_kv_attention_cache_amd import runner as R
    from paged_kv_attention_cache_amd import workloads as W
    out = {}
    for name in [c.strip() for c in configs.split(",") if c.strip()]:
        wl = W.make(name)
        pool = R.make_pool(wl, fill_byte=None)
        r = history_write_rate(wl, pool, reps=steps, warmup=warmup)
        r["kv_dtype"] = wl.kv_dtype
        out[name] = r
        log(f"[bench] write {name}: {r['hist_write_GBps']:.0f} GB/s ({r['hist_write_hbm_frac']:.3f} of peak)")
        del pool
        torch.cuda.empty_cache()
    print(json.dumps({"kv_cache_write": out}), flush=True)


def hbm_ceiling(gib: int = 4, reps: int = 20):
    """Streaming-read ceiling of this GPU's HBM: a 4 GiB buffer read once per call with
    plain and with nontemporal 16-byte loads (libtl_stream.so), at several grid sizes,
    each call after FLUSH_BYTES of scratch traffic, timed with HIP events; median GB/s.
    Context for the roofline fractions, whose denominator stays the published 8 TB/s."""
    import ctypes
    import torch
    from paged_kv_attention_cache_amd import _build
    L = ctypes.CDLL(_build.STREAM_LIB)
    L.tl_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    n = gib << 30
    buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for nt in (0, 1):
        for wg in (1024, 2048, 4096, 8192, 32768, 65536):
            def call():
                rc = L.tl_stream_read(buf.data_ptr(), n, sink.data_ptr(), nt, wg, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"tl_stream_read: HIP error {rc}")
            call()
            t = flushed_calls(call, reps)
            key = f"{'nontemporal' if nt else 'plain'}_wg{wg}"
            res[key] = {"median_GBps": n / (t["median_ms"] * 1e-3) / 1e9, "max_GBps": n / (t["min_ms"] * 1e-3) / 1e9,
                        "median_ms": t["median_ms"]}
            log(f"[bench] stream read {key}: {res[key]['median_GBps']:.0f} GB/s median")
    # The decode kernels' access pattern: 4 KiB spans (one (page, head) of K or V at
    # pages of 16 bf16 tokens) in a shuffled order, nontemporal loads.
    L.tl_block_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_void_p]
    nblk = n // 4096
    order = torch.from_numpy(np.random.default_rng(11).permutation(nblk).astype(np.int32)).cuda()
    gather = {}
    for wg in (2048, 8192, 32768):
        def gcall():
            rc = L.tl_block_read(buf.data_ptr(), order.data_ptr(), nblk, sink.data_ptr(), 1, wg, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"tl_block_read: HIP error {rc}")
        gcall()
        t = flushed_calls(gcall, reps)
        gather[f"nontemporal_wg{wg}"] = {"median_GBps": n / (t["median_ms"] * 1e-3) / 1e9,
                                         "max_GBps": n / (t["min_ms"] * 1e-3) / 1e9, "median_ms": t["median_ms"]}
        log(f"[bench] shuffled 4 KiB blocks wg{wg}: {gather[f'nontemporal_wg{wg}']['median_GBps']:.0f} GB/s median")
    # Bytes in flight: the same shuffled blocks on a persistent grid of 2 workgroups of
    # 4 waves per CU (the decode kernels' shape; 60 KiB of dynamic LDS each caps it),
    # with 4 .. 32 loads of 16 bytes per thread issued before any is used.
    L.tl_block_read_depth.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    depth = {}
    for u in (4, 8, 16, 32):
        wgs = 2 * cus
        read = (nblk // (wgs * u)) * wgs * u * 4096  # whole trips only

        def dcall():
            rc = L.tl_block_read_depth(buf.data_ptr(), order.data_ptr(), nblk, sink.data_ptr(), u, wgs, 61440,
                                       stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"tl_block_read_depth: error {rc}")
        dcall()
        t = flushed_calls(dcall, reps)
        depth[f"kib_in_flight_per_cu_{8 * u}"] = {"median_GBps": read / (t["median_ms"] * 1e-3) / 1e9,
                                                  "max_GBps": read / (t["min_ms"] * 1e-3) / 1e9,
                                                  "median_ms": t["median_ms"], "bytes": read}
        log(f"[bench] in flight {8 * u} KiB per CU: {depth[f'kib_in_flight_per_cu_{8 * u}']['median_GBps']:.0f} GB/s")
    # Reads and writes mixed: R bytes read per byte written (1 a copy; 2 and 4 as a KV
    # write into bf16 or 1-byte pools), every byte counted once, after the same
    # evicting read.
    L.tl_stream_rw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    mixed = {}
    for ratio in (1, 2, 4):
        out = (n // (ratio + 1)) // 4096 * 4096
        for ntl, nts in ((0, 0), (1, 0), (0, 1)):
            for wg in (2048, 8192):
                def rcall():
                    rc = L.tl_stream_rw(buf.data_ptr(), buf.data_ptr() + ratio * out, out, ratio, ntl, nts, wg,
                                        stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"tl_stream_rw: error {rc}")
                rcall()
                t = flushed_calls(rcall, reps)
                key = f"read{ratio}_write1_{'nt' if ntl else 'plain'}loads_{'nt' if nts else 'plain'}stores_wg{wg}"
                mixed[key] = {"median_GBps": (ratio + 1) * out / (t["median_ms"] * 1e-3) / 1e9,
                              "max_GBps": (ratio + 1) * out / (t["min_ms"] * 1e-3) / 1e9, "median_ms": t["median_ms"]}
                log(f"[bench] {key}: {mixed[key]['median_GBps']:.0f} GB/s median")
    best = max(res.items(), key=lambda kv: kv[1]["median_GBps"])
    print(json.dumps({"hbm_stream_read": res, "best": best[0], "best_median_GBps": best[1]["median_GBps"],
                      "shuffled_4k_blocks": gather, "in_flight_per_cu": depth, "read_write": mixed,
                      "bytes_per_call": n, "calls": reps, "peak_GBps": HBM_PEAK_GBPS}),
          flush=True)


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


def _dispatches(d: str, suffix: str):
    """Rows of one rocprofv3 CSV in dispatch order."""
    import csv
    return sorted(csv.DictReader(open(_find_csv(d, suffix))), key=lambda r: int(r["Start_Timestamp"]))


def _counters_by_dispatch(d: str):
    """{dispatch id: (kernel name, duration ns, {counter: value summed over instances})}, in order."""
    out = {}
    for r in _dispatches(d, "counter_collection.csv"):
        k = r["Dispatch_Id"]
        if k not in out:
            out[k] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), {})
        c = out[k][2]
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _copy_factors(copy_fetch_dir: str, copy_write_dir: str):
    cf = max(v[0] for v in _counter_means(copy_fetch_dir, "FETCH_SIZE").values()) * 1024
    cw = max(v[0] for v in _counter_means(copy_write_dir, "WRITE_SIZE").values()) * 1024
    return (1 << 30) / cf, (1 << 30) / cw, cf, cw


def write_summary(trace_dir: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                  configs: str, warmup: str, steps: str, command: str):
    """KV_CACHE_WRITE (write_kernel) from `bench.py --write-bench`: per workload, the
    flushed calls' durations from the kernel trace, and HBM bytes per dispatch from
    FETCH_SIZE / WRITE_SIZE scaled by the 1 GiB copy calibration, against the
    algorithmic bytes of one call."""
    from paged_kv_attention_cache_amd import accounting as A
    from paged_kv_attention_cache_amd import workloads as W
    w, k = int(warmup), int(steps)
    f_fetch, f_write, cf, cw = _copy_factors(copy_fetch_dir, copy_write_dir)
    trace = [r for r in _dispatches(trace_dir, "kernel_trace.csv") if "write_kernel" in r["Kernel_Name"]]
    fetch = [v for v in _counters_by_dispatch(fetch_dir).values() if "write_kernel" in v[0]]
    write = [v for v in _counters_by_dispatch(write_dir).values() if "write_kernel" in v[0]]
    print(f"command: {command}\n")
    print(f"calibration: a 1 GiB device copy reads {cf / 1024:.0f} KiB (FETCH_SIZE x {f_fetch:.3f}) and writes "
          f"{cw / 1024:.0f} KiB (WRITE_SIZE x {f_write:.3f}) per dispatch\n")
    print(f"Per workload: {w} warm-up calls, then {k} calls each after a 512 MiB cache-evicting read; durations "
          f"are of those {k}, traffic the mean over all {w + k} dispatches.\n")
    print("| workload | kv dtype | tokens | algorithmic bytes | median us | algorithmic GB/s | of 8 TB/s | read (scaled) | "
          "written (scaled) | traffic / algorithmic |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    n = w + k
    for ci, cfg in enumerate(configs.split(",")):
        wl = W.make(cfg)
        _, _, slots = next(wl.history_batches())
        alg = A.write_bytes(slots, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace[ci * n + w:(ci + 1) * n]]
        rd = np.mean([v[2]["FETCH_SIZE"] for v in fetch[ci * n:(ci + 1) * n]]) * 1024 * f_fetch
        wr = np.mean([v[2]["WRITE_SIZE"] for v in write[ci * n:(ci + 1) * n]]) * 1024 * f_write
        med = float(np.median(durs))
        print(f"| {cfg} | {wl.kv_dtype} | {len(slots)} | {alg / 1e6:.1f} MB | {med:.1f} | {alg / med / 1e3:.0f} | "
              f"{alg / med / 1e3 / HBM_PEAK_GBPS:.3f} | {rd / 1e6:.1f} MB | {wr / 1e6:.1f} MB | {(rd + wr) / alg:.3f} |")


def mfma_summary(d: str, configs: str, warmup: str, steps: str, command: str):
    """Prefill MFMA counters per workload: f32 MFMA flops counted by the hardware
    (SQ_INSTS_VALU_MFMA_MOPS_F32 x 512) against the algorithmic flops (visible pairs
    only), the MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs;
    GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's count is an eighth) and the
    effective clock."""
    from paged_kv_attention_cache_amd import accounting as A
    from paged_kv_attention_cache_amd import workloads as W
    per = [v for v in _counters_by_dispatch(d).values() if "prefill_kernel" in v[0]]
    n = int(warmup) + 2 * int(steps)
    print(f"command: {command}\n")
    print("| workload | dispatches | algorithmic TFLOP | MFMA f32 TFLOP counted | counted / algorithmic | "
          "duration us | algorithmic TFLOP/s | of 157.3 | MFMA busy | clock GHz |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for ci, cfg in enumerate(configs.split(",")):
        wl = W.make(cfg)
        alg = A.prefill_flops(wl.row_positions(), wl.num_q_heads, wl.head_dim, wl.window)
        rows = per[ci * n:(ci + 1) * n]
        if not rows:
            break
        mops = np.mean([r[2]["SQ_INSTS_VALU_MFMA_MOPS_F32"] for r in rows]) * 512
        busy = np.mean([r[2]["SQ_VALU_MFMA_BUSY_CYCLES"] for r in rows])
        gui = np.mean([r[2]["GRBM_GUI_ACTIVE"] for r in rows])
        dur = np.mean([r[1] for r in rows])
        xcd_cycles = gui / 8
        simds = 256 * 4
        print(f"| {cfg} | {len(rows)} | {alg / 1e12:.4f} | {mops / 1e12:.4f} | {mops / alg:.3f} | {dur / 1e3:.1f} | "
              f"{alg / dur / 1e3:.1f} | {alg / dur / 1e3 / MFMA_F32_PEAK_TFLOPS:.3f} | "
              f"{busy / (xcd_cycles * simds):.3f} | {xcd_cycles / dur:.2f} |")


def hbm_summary(result_json: str, trace_dir: str, command: str):
    """The streaming-read ceiling: `bench.py --hbm-ceiling`'s event-timed medians beside
    the kernel trace of the same mode (stream_read_kernel dispatches of 4 GiB; the
    512 MiB cache-evicting reads between them are listed apart)."""
    res = json.loads(open(result_json).read().strip().splitlines()[-1])
    rows = [r for r in _dispatches(trace_dir, "kernel_trace.csv") if "stream_read_kernel" in r["Kernel_Name"]]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    big = [x for x in durs if x > 300.0]  # 4 GiB reads; the 512 MiB evicting reads take about 100 us
    print(f"command: {command}\n")
    print("| loads, workgroups of 256 | median GB/s (HIP events) | best GB/s | of 8 TB/s |")
    print("|---|---|---|---|")
    for k, v in res["hbm_stream_read"].items():
        print(f"| {k} | {v['median_GBps']:.0f} | {v['max_GBps']:.0f} | {v['median_GBps'] / HBM_PEAK_GBPS:.3f} |")
    for k, v in res.get("shuffled_4k_blocks", {}).items():
        print(f"| shuffled 4 KiB blocks, {k} | {v['median_GBps']:.0f} | {v['max_GBps']:.0f} | "
              f"{v['median_GBps'] / HBM_PEAK_GBPS:.3f} |")
    for k, v in res.get("read_write", {}).items():
        print(f"| {k.replace('_', ' ')} | {v['median_GBps']:.0f} | {v['max_GBps']:.0f} | "
              f"{v['median_GBps'] / HBM_PEAK_GBPS:.3f} |")
    for k, v in res.get("in_flight_per_cu", {}).items():
        kib = k.rsplit("_", 1)[1]
        print(f"| shuffled 4 KiB blocks, 2 workgroups per CU, {kib} KiB in flight per CU | {v['median_GBps']:.0f} | "
              f"{v['max_GBps']:.0f} | {v['median_GBps'] / HBM_PEAK_GBPS:.3f} |")
    if big:
        print(f"\nKernel trace: {len(big)} dispatches of 4 GiB, {np.mean(big):.1f} us average, "
              f"{min(big):.1f} us min ({(4 << 30) / min(big) / 1e3:.0f} GB/s at the fastest).")


def clock_summary(d: str, kernels: str, command: str):
    """Effective clock per dispatch (GRBM_GUI_ACTIVE summed over the 8 XCDs, divided by
    8 and by the dispatch's duration) for the named kernels, in launch order."""
    per = list(_counters_by_dispatch(d).values())
    print(f"command: {command}\n")
    print("| kernel | dispatches | duration us, in order | clock GHz, in order |")
    print("|---|---|---|---|")
    for name in kernels.split(","):
        rows = [r for r in per if name in r[0]]
        durs = " ".join(f"{r[1] / 1e3:.0f}" for r in rows)
        ghz = " ".join(f"{r[2]['GRBM_GUI_ACTIVE'] / 8 / r[1]:.2f}" for r in rows)
        print(f"| {_short_name(rows[0][0])} | {len(rows)} | {durs} | {ghz} |")


def stats_summary(d: str, configs: str, warmup: str, steps: str, command: str):
    """Per-kernel durations from rocprofv3 --kernel-trace of one bench run, per workload.

    The run executes the workloads in the order given.  A prefill or GDN workload makes
    `warmup` attention calls, then `steps` back-to-back calls (the contract loop), then
    `steps` calls each after a cache-evicting read (the calls the roofline is taken
    from).  A decode workload makes `warmup` eager steps and `steps` timed eager steps,
    one eager step and one replay to check the captured graph, `warmup` replays, the
    `steps` replayed steps of the contract loop, then the `steps` flushed calls.
    Dispatches of the attention kernels are assigned to the workloads and phases in that
    order; the contract loop is listed as back to back."""
    import csv
    from paged_kv_attention_cache_amd import workloads as W
    rows = sorted(csv.DictReader(open(_find_csv(d, "kernel_trace.csv"))), key=lambda r: int(r["Start_Timestamp"]))
    w, k = int(warmup), int(steps)
    att = [r for r in rows if any(x in r["Kernel_Name"] for x in ATTN_KERNELS)]
    mains = [i for i, r in enumerate(att) if any(x in r["Kernel_Name"] for x in
                                                 ("decode_split_kernel", "prefill_kernel", "gdn_decode_kernel"))]
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # noqa: E731
    print(f"command: {command}\n")
    print(f"Durations from the kernel trace, grouped by workload.  Per workload: {w} warm-up calls, the "
          f"{k} back-to-back calls of the contract loop (for decode, {k} replays of the captured step, after "
          f"{w} eager and {k} timed eager steps, a check and {w} warm-up replays), then {k} calls each after a "
          f"512 MiB cache-evicting read (the roofline's calls).\n")
    print("| workload | kernel | flushed calls: average us | median us | min us | back-to-back average us |")
    print("|---|---|---|---|---|---|")
    lists = []
    pos = 0
    for cfg in configs.split(","):
        decode = getattr(W.make(cfg), "kind", "gdn") == "decode"
        n = 2 * w + 3 * k + 2 if decode else w + 2 * k
        blk = mains[pos:pos + n]
        if len(blk) < n:
            break
        hi = mains[pos + n] if pos + n < len(mains) else len(att)
        b0 = 2 * w + k + 2 if decode else w  # first back-to-back call of the contract loop
        phase_start = [blk[b0], blk[b0 + k], hi]
        pos += n
        per = {}
        for ph in (0, 1):
            for r in att[phase_start[ph]:phase_start[ph + 1]]:
                per.setdefault(_short_name(r["Kernel_Name"]), ([], []))[ph].append(dur(r))
        tot_f = tot_b = 0.0
        for name, (b2b, fl) in per.items():
            tot_f += float(np.mean(fl))
            tot_b += float(np.mean(b2b))
            print(f"| {cfg} | {name} | {np.mean(fl):.1f} | {np.median(fl):.1f} | {min(fl):.1f} | {np.mean(b2b):.1f} |")
            lists.append((cfg, name, b2b, fl))
        print(f"| {cfg} | whole attention call (sum of averages) | {tot_f:.1f} | | | {tot_b:.1f} |")
    print("\nPer-call durations (us), back-to-back calls then flushed calls:\n")
    print("| workload | kernel | back-to-back | flushed |")
    print("|---|---|---|---|")
    for cfg, name, b2b, fl in lists:
        print(f"| {cfg} | {name} | {' '.join(f'{x:.0f}' for x in b2b)} | {' '.join(f'{x:.0f}' for x in fl)} |")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-summary":
        traffic_summary(*sys.argv[2:8])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--stats-summary":
        stats_summary(*sys.argv[2:7])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--write-summary":
        write_summary(*sys.argv[2:11])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--mfma-summary":
        mfma_summary(*sys.argv[2:7])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--hbm-summary":
        hbm_summary(*sys.argv[2:5])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--clock-summary":
        clock_summary(*sys.argv[2:5])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--copy-calibration":
        copy_calibration()
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--hbm-ceiling":
        hbm_ceiling()
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--write-bench":
        write_bench(sys.argv[2] if len(sys.argv) > 2 else "c2,c5,c2i")
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
    roof["timing"] = (f"median of {args.steps} calls, each after {FLUSH_BYTES >> 20} MiB of cache-evicting "
                      f"traffic, HIP events on the launch stream")
    roof["avg_launch_ms"] = head["attn_ms"]
    if "hbm_frac_back_to_back" in head:
        roof["frac_back_to_back"] = head["hbm_frac_back_to_back"]
    elif "mfma_frac_back_to_back" in head:
        roof["frac_back_to_back"] = head["mfma_frac_back_to_back"]

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "step": ("one captured HIP graph per step: the step's KV write, then its decode call"
                 if head.get("step_mode") == "graph" else "the step's KV write, then its attention call, launched eagerly"),
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
