"""The C ABI library: loads on a machine without a GPU, exports every symbol that
include/tl.h declares, and rejects bad arguments on the host by name (no GPU call
is made on any of these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

import paged_kv_attention_cache_amd as tl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tl.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tl_[a-z0-9_]+)\s*\(", src)))


def test_library_exists_and_loads():
    assert os.path.exists(tl.LIB_PATH), "libtl.so not built"
    assert tl.tl_abi_version() == 1


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"tl_kv_cache_write", "tl_paged_attn_decode", "tl_paged_attn_prefill"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", tl.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (tl_[a-z0-9_]+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, f"not exported: {missing}"
    L = tl.lib()
    for n in names:
        assert getattr(L, n) is not None


def _pool(**kw):
    base = dict(k=0x1000, v=0x2000, k_scale=0x3000, v_scale=0x4000, dtype=1, num_pages=4, page_size=16,
                num_kv_heads=2, head_dim=128)
    base.update(kw)
    return tl._Pool(**base)


def _write(pool, n=4, k=0x5000, v=0x6000, slots=0x7000):
    return tl.lib().tl_kv_cache_write(ctypes.byref(pool) if pool is not None else None, k, v, slots, n, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(head_dim=96), tl.TL_ERR_UNSUPPORTED, "head_dim"),
    (dict(page_size=12), tl.TL_ERR_UNSUPPORTED, "page_size"),
    (dict(page_size=4), tl.TL_ERR_UNSUPPORTED, "page_size"),
    (dict(dtype=7), tl.TL_ERR_UNSUPPORTED, "dtype"),
    (dict(k=0), tl.TL_ERR_INVALID, "pool->k"),
    (dict(v=0x2004), tl.TL_ERR_INVALID, "pool->v"),
    (dict(num_pages=0), tl.TL_ERR_INVALID, "num_pages"),
    (dict(num_kv_heads=0), tl.TL_ERR_INVALID, "num_kv_heads"),
    (dict(dtype=2, k_scale=0), tl.TL_ERR_INVALID, "k_scale"),
    (dict(num_pages=1 << 27, page_size=16), tl.TL_ERR_UNSUPPORTED, "2^31"),
])
def test_write_rejects_bad_pool(kw, code, needle):
    rc = _write(_pool(**kw))
    assert rc == code
    assert needle in tl.tl_last_error()


def test_write_rejects_null_and_misaligned():
    assert _write(None) == tl.TL_ERR_INVALID and "pool is NULL" in tl.tl_last_error()
    assert _write(_pool(), k=0) == tl.TL_ERR_INVALID and "k_new" in tl.tl_last_error()
    assert _write(_pool(), v=0x6004) == tl.TL_ERR_INVALID and "v_new" in tl.tl_last_error()
    assert _write(_pool(), slots=0) == tl.TL_ERR_INVALID and "slots" in tl.tl_last_error()
    assert _write(_pool(), n=-1) == tl.TL_ERR_INVALID and "n_tokens" in tl.tl_last_error()
    assert _write(_pool(), n=0) == tl.TL_OK  # nothing to do, nothing enqueued


def _decode(pool, Hq=8, batch=2, max_blocks=4, ws=0x9000, ws_bytes=1 << 30, q=0x8000):
    return tl.lib().tl_paged_attn_decode(ctypes.byref(pool), q, Hq, 0xA000, max_blocks, 0xB000, batch, 0,
                                         ctypes.c_float(0.1), 0xC000, ws, ws_bytes, None)


def test_decode_rejects_bad_arguments():
    p = _pool()
    assert _decode(p, Hq=7) == tl.TL_ERR_INVALID and "num_q_heads" in tl.tl_last_error()
    assert _decode(p, Hq=32) == tl.TL_ERR_UNSUPPORTED and "1, 2, 4 or 8" in tl.tl_last_error()
    assert _decode(p, batch=-1) == tl.TL_ERR_INVALID and "batch" in tl.tl_last_error()
    assert _decode(p, max_blocks=0) == tl.TL_ERR_INVALID and "max_blocks" in tl.tl_last_error()
    assert _decode(p, ws=0) == tl.TL_ERR_WORKSPACE and "workspace" in tl.tl_last_error()
    assert _decode(p, ws_bytes=16) == tl.TL_ERR_WORKSPACE
    assert _decode(p, q=0x8004) == tl.TL_ERR_INVALID and "q is not" in tl.tl_last_error()
    assert _decode(p, batch=0) == tl.TL_OK


# control words, then one arrival counter per (sequence of a 2048-sequence launch, head
# group of up to 64), at the same place for every shape
WS_HEADER = 16 + 2048 * 64 * 4


def test_decode_workspace_size_formula():
    p = _pool(dtype=1, page_size=16, head_dim=128)
    # bf16 at G = 4 and D = 128 (the exact-split tile): splits of 1,024 keys (64 pages of
    # 16): 128 blocks of 16 = 2048 keys -> 2 splits
    n = tl.lib().tl_paged_attn_decode_workspace_size(ctypes.byref(p), 3, 8, 128)
    assert n == 3 * 8 * 2 * (128 + 2) * 4 + WS_HEADER  # partial states (acc + m, l) after the header
    # bf16 at G = 2 (the register tile): splits of 512 keys -> 4 splits
    n2 = tl.lib().tl_paged_attn_decode_workspace_size(ctypes.byref(p), 3, 4, 128)
    assert n2 == 3 * 4 * 4 * (128 + 2) * 4 + WS_HEADER
    p8 = _pool(dtype=2, page_size=64, head_dim=128)
    n8 = tl.lib().tl_paged_attn_decode_workspace_size(ctypes.byref(p8), 2, 16, 512)  # 32768 keys / 4096
    assert n8 == 2 * 16 * 8 * 130 * 4 + WS_HEADER
    assert tl.lib().tl_paged_attn_decode_workspace_size(ctypes.byref(p), 3, 7, 64) == 0


def test_prefill_rejects_bad_arguments():
    p = _pool()
    L = tl.lib()
    f = ctypes.c_float(0.1)
    assert L.tl_paged_attn_prefill(ctypes.byref(p), 0x8000, 8, 0xA000, 4, 0, 2, 16, 0, f, 0xC000, None, 0, None) \
        == tl.TL_ERR_INVALID and "positions" in tl.tl_last_error()
    assert L.tl_paged_attn_prefill(ctypes.byref(p), 0x8000, 8, 0xA000, 4, 0xB000, 2, -3, 0, f, 0xC000, None, 0,
                                   None) == tl.TL_ERR_INVALID and "tokens_per_row" in tl.tl_last_error()
    assert L.tl_paged_attn_prefill(ctypes.byref(p), 0x8000, 6, 0xA000, 4, 0xB000, 2, 16, 0, f, 0xC000, None, 0,
                                   None) == tl.TL_ERR_UNSUPPORTED
    assert L.tl_paged_attn_prefill(ctypes.byref(p), 0x8000, 8, 0xA000, 4, 0xB000, 0, 16, 0, f, 0xC000, None, 0,
                                   None) == tl.TL_OK
    assert tl.lib().tl_paged_attn_prefill_workspace_size(ctypes.byref(p), 2, 16, 8, 4) == 0


def test_gather_rejects_bad_arguments():
    p = _pool(dtype=2)
    L = tl.lib()
    assert L.tl_kv_gather(ctypes.byref(p), 0xA000, 5, 0xC000, 0xD000, None, None, None) == tl.TL_ERR_INVALID
    assert "scale" in tl.tl_last_error()
    assert L.tl_kv_gather(ctypes.byref(p), 0xA000, -1, 0xC000, 0xD000, None, None, None) == tl.TL_ERR_INVALID
    assert L.tl_kv_gather(ctypes.byref(p), 0xA000, 0, 0xC000, 0xD000, None, None, None) == tl.TL_OK


def test_last_error_is_cleared_by_a_successful_call():
    _write(None)
    assert tl.tl_last_error() != ""
    assert _write(_pool(), n=0) == tl.TL_OK
    assert tl.tl_last_error() == ""


def test_ring_entries_reject_bad_arguments_and_size_their_workspace():
    p = _pool(dtype=1, page_size=16, head_dim=128)
    L = tl.lib()
    f = ctypes.c_float(0.1)
    rc = L.tl_paged_attn_decode_ring(ctypes.byref(p), 0x8000, 8, 0xA000, 0, 0xB000, 2, 64, f, 0xC000, 0x9000, 1 << 30,
                                     None)
    assert rc == tl.TL_ERR_INVALID and "ring_pages" in tl.tl_last_error()
    rc = L.tl_paged_attn_prefill_ring(ctypes.byref(p), 0x8000, 8, 0xA000, -2, 0xB000, 2, 16, 64, f, 0xC000, None, 0,
                                      None)
    assert rc == tl.TL_ERR_INVALID and "ring_pages" in tl.tl_last_error()
    rc = L.tl_paged_attn_decode_ring(ctypes.byref(p), 0x8000, 8, 0, 4, 0xB000, 2, 64, f, 0xC000, 0x9000, 1 << 30, None)
    assert rc == tl.TL_ERR_INVALID and "ring_tables" in tl.tl_last_error()
    # bf16 at G = 4, D = 128: splits of 1,024 keys.  A ring of 8 pages of 16 = 128 slots;
    # window 100 spans at most 99 // 1024 + 2 = 2 splits
    n = L.tl_paged_attn_decode_ring_workspace_size(ctypes.byref(p), 3, 8, 8, 100)
    assert n == WS_HEADER + 3 * 8 * 2 * (128 + 2) * 4
    # no window: the ring's 128 slots
    assert L.tl_paged_attn_decode_ring_workspace_size(ctypes.byref(p), 3, 8, 8, 0) == n
    # a window wider than a large ring is cut to the ring: 4096 slots -> 4095 // 1024 + 2 = 5 splits
    assert L.tl_paged_attn_decode_ring_workspace_size(ctypes.byref(p), 1, 8, 256, 10 ** 6) == WS_HEADER + 8 * 5 * 130 * 4
    # at G = 2 (the register tile, 512-key splits): 4095 // 512 + 2 = 9 splits
    assert L.tl_paged_attn_decode_ring_workspace_size(ctypes.byref(p), 1, 4, 256, 10 ** 6) == WS_HEADER + 4 * 9 * 130 * 4
    rc = L.tl_paged_attn_decode_ring(ctypes.byref(p), 0x8000, 8, 0xA000, 8, 0xB000, 3, 100, f, 0xC000, 0x9000, n - 1,
                                     None)
    assert rc == tl.TL_ERR_WORKSPACE
