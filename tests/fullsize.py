"""Oracle references for the full-size parity checks, computed in worker processes.

Every output row of the full-size workloads is compared with the oracle.  The oracle
side regenerates each sequence's K/V from its seeded stream, encodes it (bytes the
GPU pool must hold, compared through a digest) and attends over the contiguous
stored history with ``oracle.paged.attend_history``.  That is seconds to minutes of
single-threaded numpy per workload, so sequences are spread over a pool of worker
processes started with "spawn" (fresh interpreters that never touch the GPU), each
with one BLAS thread.  No attention arithmetic lives here: only task plumbing.
"""
from __future__ import annotations

import functools
import hashlib
import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np


def workers() -> int:
    """Worker processes: the host's cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _init():
    from threadpoolctl import threadpool_limits
    global _LIMIT
    _LIMIT = threadpool_limits(1)


def pool() -> ProcessPoolExecutor:
    return ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"), initializer=_init)


@functools.lru_cache(maxsize=4)
def _wl(cfg: str):
    from paged_kv_attention_cache_amd import workloads as W
    return W.make(cfg)


def _stored(wl, b):
    from oracle import encode as E
    k, v = wl.seq_kv(b)
    kr, ks = E.encode_kv(k, wl.kv_dtype)
    vr, vs = E.encode_kv(v, wl.kv_dtype)
    return (kr, ks, vr, vs), E.kv_values(kr, ks, wl.kv_dtype), E.kv_values(vr, vs, wl.kv_dtype)


def digest(*arrays) -> str:
    """sha256 over the raw bytes of the given arrays (None skipped), in order."""
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
    return h.hexdigest()


def decode_row(cfg: str, b: int):
    """Reference output [H_q, D] of decode sequence b and the digest of its stored rows
    (positions 0..L-1 in logical order: K codes, V codes, then scales)."""
    import oracle
    wl = _wl(cfg)
    L = int(wl.seq_lens[b])
    (kr, ks, vr, vs), Kv, Vv = _stored(wl, b)
    ref = oracle.paged.attend_history(wl.decode_q(b)[None], Kv, Vv, np.array([L - 1]), wl.window, wl.scale)
    return b, digest(kr, vr, ks, vs), ref[0]


def prefill_rows(cfg: str, b: int, ts):
    """Reference outputs [len(ts), H_q, D] of prefill row b at tokens ts, and the digest
    of the row's stored history (positions 0..context-1)."""
    import oracle
    wl = _wl(cfg)
    ts = np.asarray(ts, dtype=np.int64)
    (kr, ks, vr, vs), Kv, Vv = _stored(wl, b)
    q = wl.prefill_rows(b)[0]
    pos = wl.row_positions()[b]
    ref = oracle.paged.attend_history(q[ts], Kv, Vv, pos[ts], wl.window, wl.scale)
    return b, ts, digest(kr, vr, ks, vs), ref
