"""Drive the library on a seeded workload: upload inputs, write history, run a step.

Plumbing only (torch device memory and the ctypes binding); no attention
arithmetic lives here.
"""
from __future__ import annotations

import numpy as np

from . import KVPool, tl_kv_cache_write, tl_paged_attn_decode, tl_paged_attn_decode_ring, \
    tl_paged_attn_decode_ring_workspace_size, tl_paged_attn_decode_workspace_size, tl_paged_attn_prefill
from .workloads import Workload

SENTINEL = 0xA5


def _t(x, device, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def make_pool(wl: Workload, device="cuda", fill_byte: int | None = SENTINEL) -> KVPool:
    return KVPool.allocate(wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, device,
                           fill_byte=fill_byte)


def write_history(pool: KVPool, wl: Workload, device="cuda") -> int:
    """Write every history position of the workload (chunked); returns tokens written."""
    n = 0
    for k, v, s in wl.history_batches():
        tl_kv_cache_write(pool, _t(k, device), _t(v, device), _t(s, device))
        n += len(s)
    return n


class DecodeStep:
    """Device inputs of one decode step: the step write and the decode call."""

    def __init__(self, wl: Workload, pool: KVPool, device="cuda"):
        import torch
        assert wl.kind == "decode"
        self.wl, self.pool = wl, pool
        k, v, s = wl.decode_step_rows()
        self.k_new, self.v_new, self.slots = _t(k, device), _t(v, device), _t(s, device)
        self.q = _t(wl.decode_q(), device)
        self.tables = _t(wl.block_tables, device)
        self.seq_lens = _t(wl.seq_lens, device)
        self.out = torch.empty_like(self.q)
        if wl.ring_pages > 0:
            nb = tl_paged_attn_decode_ring_workspace_size(pool, wl.batch, wl.num_q_heads, wl.ring_pages, wl.window)
        else:
            nb = tl_paged_attn_decode_workspace_size(pool, wl.batch, wl.num_q_heads, wl.max_blocks)
        self.workspace = torch.zeros(max(nb, 16), dtype=torch.uint8, device=device)

    def write(self, stream=None):
        tl_kv_cache_write(self.pool, self.k_new, self.v_new, self.slots, stream=stream)

    def attend(self, stream=None):
        if self.wl.ring_pages > 0:
            return tl_paged_attn_decode_ring(self.pool, self.q, self.tables, self.seq_lens, self.wl.window,
                                             self.wl.scale, out=self.out, workspace=self.workspace, stream=stream)
        return tl_paged_attn_decode(self.pool, self.q, self.tables, self.seq_lens, self.wl.window, self.wl.scale,
                                    out=self.out, workspace=self.workspace, stream=stream)

    def run(self, stream=None):
        self.write(stream)
        return self.attend(stream)


class PrefillStep:
    """Device inputs of one prefill call: the chunk's write and the prefill attention."""

    def __init__(self, wl: Workload, pool: KVPool, device="cuda"):
        import torch
        assert wl.kind == "prefill"
        self.wl, self.pool = wl, pool
        q, k, v, s, pos = wl.prefill_inputs()
        H, D = wl.num_kv_heads, wl.head_dim
        self.q = _t(q, device)
        self.k_new = _t(k.reshape(-1, H, D), device)
        self.v_new = _t(v.reshape(-1, H, D), device)
        self.slots = _t(s.reshape(-1), device)
        self.positions = _t(pos, device)
        self.tables = _t(wl.block_tables, device)
        self.out = torch.empty_like(self.q)

    def write(self, stream=None):
        tl_kv_cache_write(self.pool, self.k_new, self.v_new, self.slots, stream=stream)

    def attend(self, stream=None, window: int | None = None):
        w = self.wl.window if window is None else window
        return tl_paged_attn_prefill(self.pool, self.q, self.tables, self.positions, w, self.wl.scale,
                                     out=self.out, stream=stream)

    def run(self, stream=None):
        self.write(stream)
        return self.attend(stream)


def pool_logical(pool: KVPool):
    """Pool contents as numpy raw arrays in logical [P, H, S, D] order (+ scales)."""
    import torch
    k = pool.k.permute(0, 1, 3, 2, 4).reshape(pool.num_pages, pool.num_kv_heads, pool.page_size, pool.head_dim)
    raw = {"f32": torch.int32, "bf16": torch.int16, "fp8": torch.uint8, "fp8u": torch.uint8,
           "int8": torch.int8}[pool.kv_dtype]
    npdt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "fp8u": np.uint8, "int8": np.int8}[pool.kv_dtype]
    kk = k.contiguous().view(raw).cpu().numpy().view(npdt)
    vv = pool.v.contiguous().view(raw).cpu().numpy().view(npdt)
    ks = vs = None
    if pool.k_scale is not None:
        ks, vs = pool.k_scale.cpu().numpy(), pool.v_scale.cpu().numpy()
    return kk, vv, ks, vs
