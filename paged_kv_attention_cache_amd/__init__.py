"""Paged KV-cache write and paged attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libtl.so`` (C ABI in ``include/tl.h``).  It only
marshals arguments: every step of the path runs in the HIP kernels.  torch is
used for device memory and streams.  The binding has no fallback: if the
library is missing or its call fails, it raises.

Names follow the C ABI: ``tl_kv_cache_write``, ``tl_slot_mapping``,
``tl_paged_attn_decode``, ``tl_paged_attn_prefill``, their ring forms
``tl_paged_attn_decode_ring`` and ``tl_paged_attn_prefill_ring``, ``tl_kv_gather``
and the workspace-size queries.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtl.so")

# fp8 and int8: one f32 scale per (token, kv head); fp8u: the unscaled fp8 pool
KV_DTYPES = {"f32": 0, "bf16": 1, "fp8": 2, "fp8u": 3, "int8": 4}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "fp8u": 1, "int8": 1}
SCALED = ("fp8", "int8")

TL_OK, TL_ERR_INVALID, TL_ERR_UNSUPPORTED, TL_ERR_WORKSPACE, TL_ERR_HIP, TL_ERR_NO_PAGES = 0, -1, -2, -3, -4, -5


class TLError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


class _Pool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtl.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(_Pool)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.tl_kv_cache_write.argtypes = [P, vp, vp, vp, i64, vp]
        L.tl_paged_attn_decode_workspace_size.argtypes = [P, i32, i32, i32]
        L.tl_paged_attn_decode_workspace_size.restype = sz
        L.tl_paged_attn_decode.argtypes = [P, vp, i32, vp, i32, vp, i32, i32, f32, vp, vp, sz, vp]
        L.tl_paged_attn_prefill_workspace_size.argtypes = [P, i32, i32, i32, i32]
        L.tl_paged_attn_prefill_workspace_size.restype = sz
        L.tl_paged_attn_prefill.argtypes = [P, vp, i32, vp, i32, vp, i32, i32, i32, f32, vp, vp, sz, vp]
        L.tl_paged_attn_decode_ring_workspace_size.argtypes = [P, i32, i32, i32, i32]
        L.tl_paged_attn_decode_ring_workspace_size.restype = sz
        L.tl_paged_attn_decode_ring.argtypes = [P, vp, i32, vp, i32, vp, i32, i32, f32, vp, vp, sz, vp]
        L.tl_paged_attn_prefill_ring.argtypes = [P, vp, i32, vp, i32, vp, i32, i32, i32, f32, vp, vp, sz, vp]
        L.tl_kv_gather.argtypes = [P, vp, i32, vp, vp, vp, vp, vp]
        L.tl_slot_mapping.argtypes = [vp, i32, i32, vp, i32, i32, i32, i32, vp, vp]
        L.tl_paged_attn_decode_static.argtypes = [P, vp, i32, vp, i32, vp, i32, i32, f32, vp, vp]
        L.tl_paged_attn_decode_static.restype = ctypes.c_int
        L.tl_gated_delta_rule_decode.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
        f64 = ctypes.c_double
        L.tl_alloc_create.argtypes = [i32, i32, f64]
        L.tl_alloc_create.restype = vp
        L.tl_alloc_destroy.argtypes = [vp]
        L.tl_alloc_destroy.restype = None
        L.tl_alloc_free_pages.argtypes = [vp]
        L.tl_alloc_free_pages.restype = i32
        L.tl_alloc_start.argtypes = [vp, i64, f64]
        L.tl_alloc_end.argtypes = [vp, i64]
        L.tl_alloc_fork.argtypes = [vp, i64, i64, i64, f64]
        L.tl_alloc_append.argtypes = [vp, i64, i32, f64, vp, vp, vp, vp]
        L.tl_alloc_tables.argtypes = [vp, vp, i32, i32, vp, vp]
        L.tl_kv_copy_pages.argtypes = [P, vp, vp, i32, vp]
        for fn in ("tl_alloc_start", "tl_alloc_end", "tl_alloc_fork", "tl_alloc_append", "tl_alloc_tables",
                   "tl_kv_copy_pages"):
            getattr(L, fn).restype = ctypes.c_int
        L.tl_last_error.restype = ctypes.c_char_p
        L.tl_abi_version.restype = ctypes.c_int
        for fn in ("tl_kv_cache_write", "tl_paged_attn_decode", "tl_paged_attn_prefill", "tl_kv_gather", "tl_slot_mapping",
                   "tl_paged_attn_decode_ring", "tl_paged_attn_prefill_ring", "tl_gated_delta_rule_decode"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != TL_OK:
        raise TLError(rc, lib().tl_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# --------------------------------------------------------------------- pool
@dataclass
class KVPool:
    """One layer's K/V page pool in device memory (layouts of include/tl.h)."""

    k: "object"
    v: "object"
    k_scale: "object"
    v_scale: "object"
    kv_dtype: str
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim: int

    @property
    def chunk(self) -> int:
        """Elements per 16-byte chunk of the K layout."""
        return 16 // ELEM_BYTES[self.kv_dtype]

    @staticmethod
    def allocate(num_pages: int, page_size: int, num_kv_heads: int, head_dim: int, kv_dtype: str,
                 device="cuda", fill_byte: int | None = None) -> "KVPool":
        import torch
        x = 16 // ELEM_BYTES[kv_dtype]
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8, "fp8u": torch.uint8,
               "int8": torch.int8}[kv_dtype]
        kshape = (num_pages, num_kv_heads, head_dim // x, page_size, x)
        vshape = (num_pages, num_kv_heads, page_size, head_dim)
        mk = (lambda s, dt: torch.empty(s, dtype=dt, device=device))
        k, v = mk(kshape, tdt), mk(vshape, tdt)
        ks = vs = None
        if kv_dtype in SCALED:
            ks = mk((num_pages, num_kv_heads, page_size), torch.float32)
            vs = mk((num_pages, num_kv_heads, page_size), torch.float32)
        pool = KVPool(k, v, ks, vs, kv_dtype, num_pages, page_size, num_kv_heads, head_dim)
        if fill_byte is not None:
            for t in pool.tensors():
                t.view(torch.uint8).fill_(fill_byte)
        return pool

    def tensors(self):
        return [t for t in (self.k, self.v, self.k_scale, self.v_scale) if t is not None]

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors())

    def c_struct(self) -> _Pool:
        return _Pool(self.k.data_ptr(), self.v.data_ptr(), _ptr(self.k_scale), _ptr(self.v_scale),
                     KV_DTYPES[self.kv_dtype], self.num_pages, self.page_size, self.num_kv_heads, self.head_dim)


# --------------------------------------------------------------- entry points
def tl_kv_cache_write(pool: KVPool, k_new, v_new, slots, stream=None) -> None:
    """KV_CACHE_WRITE: k_new/v_new f32 [n, H_kv, D], slots int32 [n] (-1 = skip)."""
    n = int(slots.numel())
    ps = pool.c_struct()
    _check(lib().tl_kv_cache_write(ctypes.byref(ps), k_new.data_ptr(), v_new.data_ptr(), slots.data_ptr(), n,
                                   _stream(stream)))


def tl_paged_attn_decode_workspace_size(pool: KVPool, batch: int, num_q_heads: int, max_blocks: int) -> int:
    ps = pool.c_struct()
    return int(lib().tl_paged_attn_decode_workspace_size(ctypes.byref(ps), batch, num_q_heads, max_blocks))


def tl_paged_attn_prefill_workspace_size(pool: KVPool, batch: int, tokens_per_row: int, num_q_heads: int,
                                         max_blocks: int) -> int:
    ps = pool.c_struct()
    return int(lib().tl_paged_attn_prefill_workspace_size(ctypes.byref(ps), batch, tokens_per_row, num_q_heads,
                                                          max_blocks))


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def tl_paged_attn_decode(pool: KVPool, q, block_tables, seq_lens, window: int = 0, scale: float | None = None,
                         out=None, workspace=None, stream=None):
    """PAGED_ATTENTION decode: q f32 [B, H_q, D]; block_tables int32 [B, max_blocks]; seq_lens int32 [B]."""
    import torch
    B, Hq, D = q.shape
    max_blocks = int(block_tables.shape[1])
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = tl_paged_attn_decode_workspace_size(pool, B, Hq, max_blocks)
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=q.device)  # zero before first use
    ps = pool.c_struct()
    sc = default_scale(D) if scale is None else scale
    _check(lib().tl_paged_attn_decode(ctypes.byref(ps), q.data_ptr(), Hq, block_tables.data_ptr(), max_blocks,
                                      seq_lens.data_ptr(), B, window, sc, out.data_ptr(), workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def tl_paged_attn_decode_static(pool: KVPool, q, block_tables, seq_lens, window: int = 0,
                                scale: float | None = None, out=None, stream=None):
    """PAGED_ATTENTION decode with the library's static scratch (no workspace argument;
    the call allocates nothing): same arguments and results as tl_paged_attn_decode."""
    import torch
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    ps = pool.c_struct()
    sc = default_scale(D) if scale is None else scale
    _check(lib().tl_paged_attn_decode_static(ctypes.byref(ps), q.data_ptr(), Hq, block_tables.data_ptr(),
                                             int(block_tables.shape[1]), seq_lens.data_ptr(), B, window, sc,
                                             out.data_ptr(), _stream(stream)))
    return out


def tl_paged_attn_prefill(pool: KVPool, q, block_tables, positions, window: int = 0, scale: float | None = None,
                          out=None, workspace=None, stream=None):
    """PAGED_ATTENTION prefill: q f32 [B, T, H_q, D]; positions int32 [B, T] (-1 = pad)."""
    import torch
    B, T, Hq, D = q.shape
    max_blocks = int(block_tables.shape[1])
    if out is None:
        out = torch.empty_like(q)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    ps = pool.c_struct()
    sc = default_scale(D) if scale is None else scale
    _check(lib().tl_paged_attn_prefill(ctypes.byref(ps), q.data_ptr(), Hq, block_tables.data_ptr(), max_blocks,
                                       positions.data_ptr(), B, T, window, sc, out.data_ptr(), ws_ptr, ws_bytes,
                                       _stream(stream)))
    return out


def tl_paged_attn_decode_ring_workspace_size(pool: KVPool, batch: int, num_q_heads: int, ring_pages: int,
                                             window: int) -> int:
    ps = pool.c_struct()
    return int(lib().tl_paged_attn_decode_ring_workspace_size(ctypes.byref(ps), batch, num_q_heads, ring_pages,
                                                              window))


def tl_paged_attn_decode_ring(pool: KVPool, q, ring_tables, seq_lens, window: int = 0, scale: float | None = None,
                              out=None, workspace=None, stream=None):
    """PAGED_ATTENTION decode over ring tables: ring_tables int32 [B, ring_pages]."""
    import torch
    B, Hq, D = q.shape
    R = int(ring_tables.shape[1])
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = tl_paged_attn_decode_ring_workspace_size(pool, B, Hq, R, window)
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=q.device)  # zero before first use
    ps = pool.c_struct()
    sc = default_scale(D) if scale is None else scale
    _check(lib().tl_paged_attn_decode_ring(ctypes.byref(ps), q.data_ptr(), Hq, ring_tables.data_ptr(), R,
                                           seq_lens.data_ptr(), B, window, sc, out.data_ptr(), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def tl_paged_attn_prefill_ring(pool: KVPool, q, ring_tables, positions, window: int = 0, scale: float | None = None,
                               out=None, stream=None):
    """PAGED_ATTENTION prefill over ring tables: q f32 [B, T, H_q, D]; positions int32 [B, T]."""
    import torch
    B, T, Hq, D = q.shape
    R = int(ring_tables.shape[1])
    if out is None:
        out = torch.empty_like(q)
    ps = pool.c_struct()
    sc = default_scale(D) if scale is None else scale
    _check(lib().tl_paged_attn_prefill_ring(ctypes.byref(ps), q.data_ptr(), Hq, ring_tables.data_ptr(), R,
                                            positions.data_ptr(), B, T, window, sc, out.data_ptr(), None, 0,
                                            _stream(stream)))
    return out


def tl_slot_mapping(tables, positions, page_size: int, num_pages: int, ring_pages: int = 0, out=None,
                    stream=None):
    """SLOT_MAPPING (ring_pages = 0) or WINDOW_SLOT_MAPPING (ring_pages = R): slots int32
    [B, T] of positions [B, T] through tables [B, width] (device int32 tensors)."""
    import torch
    if positions.dim() == 1:
        positions = positions.reshape(1, -1)
    if tables.dim() == 1:
        tables = tables.reshape(1, -1)
    B, T = positions.shape
    if out is None:
        out = torch.empty((B, T), dtype=torch.int32, device=positions.device)
    _check(lib().tl_slot_mapping(tables.data_ptr(), int(tables.shape[1]), ring_pages, positions.data_ptr(), B, T,
                                 page_size, num_pages, out.data_ptr(), _stream(stream)))
    return out


def tl_gated_delta_rule_decode(state_pool, q, k, v, g, beta, state_slots, positions, out=None, stream=None):
    """GATED_DELTA_RULE decode step: state_pool f32 [num_slots, H, 128, 128] (updated in
    place); q, k, v f32 [B, H, 128]; g, beta f32 [B, H]; state_slots, positions int32 [B]."""
    import torch
    B, H, D = q.shape
    if out is None:
        out = torch.empty_like(v)
    _check(lib().tl_gated_delta_rule_decode(state_pool.data_ptr(), int(state_pool.shape[0]), H, D, q.data_ptr(),
                                            k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                                            state_slots.data_ptr(), positions.data_ptr(), B, out.data_ptr(),
                                            _stream(stream)))
    return out


class PageAllocator:
    """The library's host page allocator (include/tl.h: tl_alloc_*), marshalled with
    ctypes: per-sequence pages, refusal by name (TLError with code TL_ERR_NO_PAGES),
    least-recently-active reclaim of idle sequences, and prefix sharing with
    copy-on-write."""

    def __init__(self, num_pages: int, page_size: int, idle_timeout: float):
        self._h = lib().tl_alloc_create(num_pages, page_size, idle_timeout)
        if not self._h:
            raise TLError(TL_ERR_INVALID, lib().tl_last_error().decode())
        self.page_size = page_size

    def close(self) -> None:
        if self._h:
            lib().tl_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def free_pages(self) -> int:
        return int(lib().tl_alloc_free_pages(self._h))

    def start(self, seq: int, now: float) -> None:
        _check(lib().tl_alloc_start(self._h, seq, now))

    def end(self, seq: int) -> None:
        _check(lib().tl_alloc_end(self._h, seq))

    def fork(self, parent: int, child: int, n_tokens: int, now: float) -> None:
        _check(lib().tl_alloc_fork(self._h, parent, child, n_tokens, now))

    def append(self, seq: int, n_tokens: int, now: float):
        """Slots of the next n_tokens positions and the page copies [(src, dst)] to run first."""
        slots = (ctypes.c_int32 * max(n_tokens, 1))()
        src, dst, nc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().tl_alloc_append(self._h, seq, n_tokens, now, slots, ctypes.byref(src), ctypes.byref(dst),
                                     ctypes.byref(nc)))
        return list(slots)[:n_tokens], [(src.value, dst.value)] if nc.value else []

    def tables(self, seqs, max_blocks: int):
        """Block tables [len(seqs)][max_blocks] (-1 unused) and lengths, as Python lists."""
        n = len(seqs)
        ids = (ctypes.c_int64 * max(n, 1))(*seqs)
        tab = (ctypes.c_int32 * max(n * max_blocks, 1))()
        lens = (ctypes.c_int32 * max(n, 1))()
        _check(lib().tl_alloc_tables(self._h, ids, n, max_blocks, tab, lens))
        flat = list(tab)
        return [flat[i * max_blocks:(i + 1) * max_blocks] for i in range(n)], list(lens)[:n]


def tl_kv_copy_pages(pool: KVPool, src_pages, dst_pages, stream=None) -> None:
    """Device copy of whole pages src_pages[i] -> dst_pages[i] (int32 device tensors)."""
    ps = pool.c_struct()
    _check(lib().tl_kv_copy_pages(ctypes.byref(ps), src_pages.data_ptr(), dst_pages.data_ptr(), int(src_pages.numel()),
                                  _stream(stream)))


def tl_kv_gather(pool: KVPool, block_table_row, length: int, stream=None):
    """Stored rows of positions 0..length-1 in logical order: k, v [L, H_kv, D] (+ scales [L, H_kv])."""
    import torch
    dev = pool.k.device
    shp = (length, pool.num_kv_heads, pool.head_dim)
    k = torch.empty(shp, dtype=pool.k.dtype, device=dev)
    v = torch.empty(shp, dtype=pool.v.dtype, device=dev)
    ks = vs = None
    if pool.kv_dtype in SCALED:
        ks = torch.empty((length, pool.num_kv_heads), dtype=torch.float32, device=dev)
        vs = torch.empty((length, pool.num_kv_heads), dtype=torch.float32, device=dev)
    ps = pool.c_struct()
    _check(lib().tl_kv_gather(ctypes.byref(ps), block_table_row.data_ptr(), length, k.data_ptr(), v.data_ptr(),
                              _ptr(ks), _ptr(vs), _stream(stream)))
    return k, v, ks, vs


def tl_last_error() -> str:
    return lib().tl_last_error().decode()


def tl_abi_version() -> int:
    return int(lib().tl_abi_version())


__all__ = ["KVPool", "TLError", "tl_kv_cache_write", "tl_paged_attn_decode", "tl_paged_attn_prefill",
           "tl_kv_gather", "tl_slot_mapping", "tl_paged_attn_decode_workspace_size", "tl_paged_attn_prefill_workspace_size",
           "tl_last_error", "tl_abi_version", "lib"]
