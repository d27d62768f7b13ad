"""GPU edge cases through the C ABI, against the oracle.

- SLOT_MAPPING / WINDOW_SLOT_MAPPING ("How serving works in Tlaloc", section 3):
  tl_slot_mapping against oracle.slot_mapping, bit for bit, with pads, positions past
  the table and entries outside the pool;
- TL_VALIDATE=1: a bad slot, a duplicate slot, a bad table entry, a length past the
  table, a bad position and a duplicate state slot are each refused on the host with
  TL_ERR_INVALID naming the argument, and nothing is enqueued (outputs and pools keep
  their bytes);
- calls with no live position (section 2, blockwise bullet: a row of length 0 comes
  out 0): prefill rows that are all pads and decode batches whose lengths are all 0
  give exactly 0, and leave the decode workspace header at zero;
- pools whose unwritten bytes are NaN in every dtype (0xFF): windowed prefill, ring
  prefill and windowed decode read only keys some token can see, so outputs match the
  oracle (whose pool holds zeros there) and are finite.
"""
import numpy as np
import pytest

import oracle
from paged_kv_attention_cache_amd import workloads as W
from paged_kv_attention_cache_amd import runner as R
from tests.helpers import row_rel_err
from tests.test_gpu_parity import TOL, torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu

HEADER = 524304  # decode workspace header bytes (control words and arrival counters)


def _t(torch, x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t if dtype is None else t.to(dtype)).cuda()


# ---------------------------------------------------------------- slot mapping
@pytest.mark.parametrize("ring_pages", [0, 1, 3, 7])
def test_slot_mapping_matches_the_oracle(torch_cuda, ring_pages):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    rng = np.random.default_rng([40, ring_pages])
    B, T, S, P, width = 5, 300, 16, 50, 9
    tables = rng.integers(-2, P + 3, size=(B, width)).astype(np.int32)  # some -1, -2 and >= P entries
    pos = rng.integers(-3, 20 * S, size=(B, T)).astype(np.int32)         # pads, past-the-table blocks
    pos[0, :S * 3] = np.arange(S * 3)
    got = tl.tl_slot_mapping(_t(torch, tables), _t(torch, pos), S, P, ring_pages=ring_pages).cpu().numpy()
    want = oracle.slot_mapping(tables, pos, S, P, ring_pages)
    assert np.array_equal(got, want)
    assert np.any(want == -1) and np.any(want >= 0)


def test_slot_mapping_feeds_the_write_like_the_workload_slots(torch_cuda):
    """The slots tl_slot_mapping gives for a prefill call are those the oracle writes at."""
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    wl = W.custom_prefill(41, [30, 0, 17], [5, 0, 40], 32, 8, 2, 64, 16, "bf16", spare_pages=2)
    pos = wl.row_positions()
    got = tl.tl_slot_mapping(_t(torch, wl.block_tables), _t(torch, pos), wl.page_size, wl.num_pages).cpu().numpy()
    assert np.array_equal(got, oracle.slot_mapping(wl.block_tables, pos, wl.page_size, wl.num_pages))


# ------------------------------------------------------------------ TL_VALIDATE
def _expect_invalid(tl, fn, needle):
    with pytest.raises(tl.TLError) as e:
        fn()
    assert e.value.code == tl.TL_ERR_INVALID, e.value.message
    assert needle in e.value.message and "TL_VALIDATE" in e.value.message, e.value.message


def test_validate_mode_refuses_bad_indices_before_launch(torch_cuda, monkeypatch):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    monkeypatch.setenv("TL_VALIDATE", "1")
    P, S, H, D = 6, 16, 2, 64
    gp = tl.KVPool.allocate(P, S, H, D, "bf16", fill_byte=0xA5)
    k = _t(torch, np.ones((4, H, D), np.float32))
    snap = [t.clone() for t in gp.tensors()]

    _expect_invalid(tl, lambda: tl.tl_kv_cache_write(gp, k, k, _t(torch, np.array([0, 1, P * S + 5, 2], np.int32))),
                    "slots[2]")
    _expect_invalid(tl, lambda: tl.tl_kv_cache_write(gp, k, k, _t(torch, np.array([3, -1, 7, 3], np.int32))),
                    "slot 3 appears twice")
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(snap, gp.tensors())), "a refused write changed the pool"

    q = _t(torch, np.ones((2, 4, D), np.float32))
    tables = np.array([[0, 1], [2, 999]], np.int32)
    out = torch.full((2, 4, D), 7.0, device="cuda")
    _expect_invalid(tl, lambda: tl.tl_paged_attn_decode(gp, q, _t(torch, tables), _t(torch, np.array([20, 30], np.int32)),
                                                       out=out), "block_tables[1][1] = 999")
    _expect_invalid(tl, lambda: tl.tl_paged_attn_decode(gp, q, _t(torch, tables), _t(torch, np.array([40, 3], np.int32)),
                                                       out=out), "seq_lens[0] = 40")
    qp = _t(torch, np.ones((1, 3, 4, D), np.float32))
    outp = torch.full((1, 3, 4, D), 7.0, device="cuda")
    _expect_invalid(tl, lambda: tl.tl_paged_attn_prefill(gp, qp, _t(torch, tables[:1]), _t(torch, np.array([[-1, -2, 0]], np.int32)),
                                                        out=outp), "positions[0][1] = -2")
    _expect_invalid(tl, lambda: tl.tl_slot_mapping(_t(torch, tables), _t(torch, np.array([[0, 40], [0, 1]], np.int32)), S, P),
                    "positions[0][1] = 40")
    _expect_invalid(tl, lambda: tl.tl_slot_mapping(_t(torch, tables), _t(torch, np.array([[0, 1], [0, 20]], np.int32)), S, P),
                    "tables[1][1] = 999")
    st = torch.zeros((3, 2, 128, 128), device="cuda")
    x = torch.zeros((2, 2, 128), device="cuda")
    gb = torch.zeros((2, 2), device="cuda")
    _expect_invalid(tl, lambda: tl.tl_gated_delta_rule_decode(st, x, x, x, gb, gb, _t(torch, np.array([1, 1], np.int32)),
                                                             _t(torch, np.array([3, 4], np.int32))), "state slot 1 appears twice")
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(outp == 7.0), "a refused call wrote its output"
    # the same calls with valid indices go through
    tl.tl_kv_cache_write(gp, k, k, _t(torch, np.array([0, 1, 2, 3], np.int32)))
    tl.tl_paged_attn_decode(gp, q, _t(torch, np.array([[0, 1], [2, 3]], np.int32)), _t(torch, np.array([4, 1], np.int32)),
                            out=out)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))


# ----------------------------------------------------------- no live position
@pytest.mark.parametrize("kv_dtype,hq", [("bf16", 8), ("fp8", 16), ("f32", 2)])
def test_prefill_call_with_no_live_position_is_all_zero(torch_cuda, kv_dtype, hq):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    P, S, H, D, B, T = 4, 16, 2, 128, 3, 70
    gp = tl.KVPool.allocate(P, S, H, D, kv_dtype, fill_byte=0xFF)
    q = torch.randn((B, T, hq, D), device="cuda")
    out = torch.full((B, T, hq, D), float("nan"), device="cuda")
    tables = _t(torch, np.zeros((B, 2), np.int32))
    pos = _t(torch, np.full((B, T), -1, np.int32))
    for win in (0, 33):
        out.fill_(float("nan"))
        tl.tl_paged_attn_prefill(gp, q, tables, pos, win, out=out)
        torch.cuda.synchronize()
        assert torch.all(out == 0), f"window {win}"


@pytest.mark.parametrize("kv_dtype,hq", [("bf16", 8), ("fp8", 16), ("int8", 4), ("fp8", 8)])
def test_decode_with_all_lengths_zero_is_all_zero_and_leaves_the_header_clear(torch_cuda, kv_dtype, hq):
    """fp8 at G = 8 runs the exact-split kernel (splits merged in place), the others the
    register-tile kernel and the merge kernel."""
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    P, S, H, D, B = 8, 16, 2, 128, 37
    gp = tl.KVPool.allocate(P, S, H, D, kv_dtype, fill_byte=0xFF)
    q = torch.randn((B, hq, D), device="cuda")
    tables = _t(torch, np.zeros((B, 4), np.int32))
    nb = tl.tl_paged_attn_decode_workspace_size(gp, B, hq, 4)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    out = torch.full((B, hq, D), float("nan"), device="cuda")
    for win in (0, 5):
        out.fill_(float("nan"))
        tl.tl_paged_attn_decode(gp, q, tables, _t(torch, np.zeros(B, np.int32)), win, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(out == 0), f"window {win}"
        assert not torch.any(ws[:HEADER]), "workspace header not zero after the call"


# --------------------------------------------------------------- NaN-filled pools
def _pools_written_from(tl, torch, wl, first):
    """GPU pool of 0xFF bytes (NaN in every dtype's values or scales) and an oracle pool
    of zeros, both holding sequence 0's K/V at positions first .. context-1 only."""
    H, D = wl.num_kv_heads, wl.head_dim
    gp = tl.KVPool.allocate(wl.num_pages, wl.page_size, H, D, wl.kv_dtype, fill_byte=0xFF)
    op = oracle.KVPool(wl.num_pages, wl.page_size, H, D, wl.kv_dtype, sentinel=0)
    k, v = wl.seq_kv(0)
    p = np.arange(first, wl.context_len(0))
    slots = wl.slots_for(0, p)
    tl.tl_kv_cache_write(gp, _t(torch, k[p]), _t(torch, v[p]), _t(torch, slots))
    op.write(k[p], v[p], slots)
    return gp, op


@pytest.mark.parametrize("kv_dtype,hq", [("bf16", 8), ("fp8", 16), ("f32", 4), ("int8", 8), ("fp8", 8)])
def test_windowed_prefill_and_decode_ignore_unwritten_nan_rows(torch_cuda, kv_dtype, hq):
    """The window starts mid-page and mid-tile, so the first key tile and page hold rows
    before it that were never written."""
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    win, chunk, start = 100, 45, 333
    wl = W.custom_prefill(60 + hq, [chunk], [start], chunk, hq, 2, 128, 16, kv_dtype, window=win, spare_pages=2)
    gp, op = _pools_written_from(tl, torch, wl, start - win + 1)  # the chunk's first visible key
    q = wl.prefill_rows(0)[0][None]
    pos = wl.row_positions()
    out = tl.tl_paged_attn_prefill(gp, _t(torch, q), _t(torch, wl.block_tables), _t(torch, pos), win, wl.scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)), "prefill read an unwritten row into its sums"
    assert row_rel_err(got, oracle.prefill(op, q, wl.block_tables, pos, win, wl.scale)) <= TOL[kv_dtype]
    # decode of the last position, on a pool written only inside its own window (fp8 at
    # G = 8 and bf16 and int8 at G = 4 take the exact-split tiles, the others the
    # register tile)
    L = np.array([start + chunk], np.int32)
    gp, op = _pools_written_from(tl, torch, wl, int(L[0]) - win)
    qd = np.ascontiguousarray(q[:, -1])
    od = tl.tl_paged_attn_decode(gp, _t(torch, qd), _t(torch, wl.block_tables), _t(torch, L), win, wl.scale)
    torch.cuda.synchronize()
    gd = od.cpu().numpy()
    assert np.all(np.isfinite(gd)), "decode read an unwritten row into its sums"
    assert row_rel_err(gd, oracle.decode(op, qd, wl.block_tables, L, win, wl.scale)) <= TOL[kv_dtype]


def test_ring_prefill_ignores_unwritten_nan_slots(torch_cuda):
    """A ring whose slots were never all written: position 0 and two ring pages hold NaN
    bytes; the tokens (positions 40..56, window 40) see from position 1, so the first key
    tile starts on the unwritten position 0, which must not be read into the sums."""
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    S, H, D, hq, win, Rp = 16, 2, 128, 8, 40, 6
    P = 9
    ring = np.array([[7, 2, 5, 0, 8, 3]], np.int32)
    rng = np.random.default_rng(3)
    n = 57  # positions 1..56 written: position 0 and ring pages 4, 5 never
    k = rng.standard_normal((n - 1, H, D)).astype(np.float32)
    v = rng.standard_normal((n - 1, H, D)).astype(np.float32)
    gp = tl.KVPool.allocate(P, S, H, D, "bf16", fill_byte=0xFF)
    op = oracle.KVPool(P, S, H, D, "bf16", sentinel=0)
    p = np.arange(1, n, dtype=np.int32)
    slots = tl.tl_slot_mapping(_t(torch, ring), _t(torch, p[None]), S, P, ring_pages=Rp).cpu().numpy().reshape(-1)
    assert np.array_equal(slots, oracle.ring_slots(ring[0], p, S))
    tl.tl_kv_cache_write(gp, _t(torch, k), _t(torch, v), _t(torch, slots))
    op.write(k, v, slots)
    T = 20
    pos = np.full((1, T), -1, np.int32)
    pos[0, 3:] = np.arange(n - (T - 3), n)
    q = rng.standard_normal((1, T, hq, D)).astype(np.float32)
    out = tl.tl_paged_attn_prefill_ring(gp, _t(torch, q), _t(torch, ring), _t(torch, pos), win, 0.088388346)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(got[0, :3] == 0)
    assert row_rel_err(got, oracle.prefill_ring(op, q, ring, pos, win, 0.088388346)) <= 2e-5
