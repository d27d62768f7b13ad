"""GPU parity of the ring (windowed KV pool) entry points through the C ABI.

Page "How serving works in Tlaloc", section 3 (windowed KV pool) and section 2
(ring bullet).  The HIP path is compared with the ring oracle (age-masked ring
slots, f64) at the same tolerances as the full-table entries, and with the
HIP full-table entries on a pool holding the same K/V: a ring that holds the
window gives the same bits.  Ring pools are written by tl_kv_cache_write at the
windowed slot mapping, one call per N positions (slots of a call are distinct).
"""
import numpy as np
import pytest

import oracle
from paged_kv_attention_cache_amd import runner as R
from tests.helpers import row_rel_err
from tests.test_gpu_parity import TOL, assert_pool_equal, torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu


def ring_slots_gpu(ring_row, p, S, num_pages):
    """WINDOW_SLOT_MAPPING through the library (tl_slot_mapping on the device), checked
    against the oracle's ring_slots for the same positions."""
    import torch
    import paged_kv_attention_cache_amd as tl
    ring_row = np.asarray(ring_row, dtype=np.int32)
    got = tl.tl_slot_mapping(torch.from_numpy(ring_row).cuda(), torch.from_numpy(np.asarray(p, np.int32)).cuda(), S,
                             num_pages, ring_pages=len(ring_row)).cpu().numpy().reshape(-1)
    assert np.array_equal(got, oracle.ring_slots(ring_row, p, S)), "ring slot mapping differs from the oracle"
    return got


def kv_rows(rng, n, Hkv, D):
    k = (rng.standard_normal((n, Hkv, D)) * rng.uniform(0.5, 2.0, (n, Hkv, 1))).astype(np.float32)
    v = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    return k, v


class RingCase:
    """B sequences, each with its own ring of R pages in one pool (pages shuffled)."""

    def __init__(self, seed, lens, Hq, Hkv, D, S, dt, R_pages):
        self.rng = np.random.default_rng([7, seed])
        self.lens = np.asarray(lens, dtype=np.int32)
        self.B, self.Hq, self.Hkv, self.D, self.S, self.dt, self.R = len(lens), Hq, Hkv, D, S, dt, R_pages
        self.N = R_pages * S
        self.P = self.B * R_pages + 3
        self.ring = self.rng.permutation(self.P)[:self.B * R_pages].reshape(self.B, R_pages).astype(np.int32)
        self.kv = [kv_rows(self.rng, int(L), Hkv, D) for L in lens]

    def write(self, gpu_pool, oracle_pool, upto=None):
        """Write every sequence's positions 0..L-1 in calls of N positions (oldest first)."""
        import torch
        import paged_kv_attention_cache_amd as tl
        upto = self.lens if upto is None else upto
        for p0 in range(0, int(max(upto)) if len(upto) else 0, self.N):
            ks, vs, ss_gpu, ss_orc = [], [], [], []
            for b in range(self.B):
                p = np.arange(p0, min(int(upto[b]), p0 + self.N))
                if p.size == 0:
                    continue
                ks.append(self.kv[b][0][p]); vs.append(self.kv[b][1][p])
                ss_gpu.append(ring_slots_gpu(self.ring[b], p, self.S, self.P))
                ss_orc.append(oracle.ring_slots(self.ring[b], p, self.S))
            k, v = np.concatenate(ks), np.concatenate(vs)
            tl.tl_kv_cache_write(gpu_pool, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                                 torch.from_numpy(np.concatenate(ss_gpu)).cuda())
            if oracle_pool is not None:
                oracle_pool.write(k, v, np.concatenate(ss_orc))


def pools(c):
    import paged_kv_attention_cache_amd as tl
    gp = tl.KVPool.allocate(c.P, c.S, c.Hkv, c.D, c.dt, fill_byte=R.SENTINEL)
    op = oracle.KVPool(c.P, c.S, c.Hkv, c.D, c.dt, sentinel=R.SENTINEL)
    return gp, op


RING_DECODE_CASES = [
    # (name, lens, Hq, Hkv, D, S, dtype, ring_pages, window)
    ("bf16_g4_wrapped", [5, 64, 200, 1000, 4099], 8, 2, 128, 16, "bf16", 5, 64),
    ("f32_g2_d64_no_window", [3, 40, 300], 4, 2, 64, 16, "f32", 3, 0),
    ("fp8_g8_exact_split", [10, 700, 5000], 16, 2, 128, 16, "fp8", 40, 600),
    ("fp8_g4_page64", [100, 9000], 8, 2, 128, 64, "fp8", 9, 520),
    ("bf16_ring_shorter_than_window", [100, 333], 8, 2, 128, 16, "bf16", 2, 50),
    ("bf16_g8_window_one", [1, 77], 16, 2, 128, 16, "bf16", 1, 1),
    ("bf16_wide_ring_many_splits", [2500, 7000], 8, 2, 128, 16, "bf16", 120, 1800),
    ("fp8u_g8_exact_split", [10, 700, 5000], 16, 2, 128, 16, "fp8u", 40, 600),
    ("int8_g4", [30, 2000], 8, 2, 128, 16, "int8", 10, 150),
]


@pytest.mark.parametrize("case", RING_DECODE_CASES, ids=[c[0] for c in RING_DECODE_CASES])
def test_ring_decode_parity(torch_cuda, case):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    name, lens, Hq, Hkv, D, S, dt, Rp, win = case
    c = RingCase(500 + RING_DECODE_CASES.index(case), lens, Hq, Hkv, D, S, dt, Rp)
    gp, op = pools(c)
    c.write(gp, op)
    q = c.rng.standard_normal((c.B, Hq, D)).astype(np.float32)
    scale = 1.0 / np.sqrt(D)
    out = tl.tl_paged_attn_decode_ring(gp, torch.from_numpy(q).cuda(), torch.from_numpy(c.ring).cuda(),
                                       torch.from_numpy(c.lens).cuda(), win, scale)
    torch.cuda.synchronize()
    assert_pool_equal(gp, op)
    ref = oracle.decode_ring(op, q, c.ring, c.lens, win, scale)
    err = row_rel_err(out.cpu().numpy(), ref)
    assert err <= TOL[dt], f"{name}: max row error {err:.3e}"


def full_table_pool(c, upto=None):
    """The same sequences in a full-history pool: block j of sequence b on its own page."""
    import torch
    import paged_kv_attention_cache_amd as tl
    upto = c.lens if upto is None else upto
    blocks = [(int(L) + c.S - 1) // c.S for L in c.lens]
    P = sum(blocks) + 2
    perm = np.random.default_rng([8, int(c.lens.sum())]).permutation(P)
    maxb = max(blocks)
    tables = np.full((c.B, maxb), -1, np.int32)
    at = 0
    for b, n in enumerate(blocks):
        tables[b, :n] = perm[at:at + n]
        at += n
    gp = tl.KVPool.allocate(P, c.S, c.Hkv, c.D, c.dt, fill_byte=R.SENTINEL)
    for b in range(c.B):
        p = np.arange(int(upto[b]))
        if p.size == 0:
            continue
        slots = (tables[b, p // c.S] * c.S + p % c.S).astype(np.int32)
        tl.tl_kv_cache_write(gp, torch.from_numpy(c.kv[b][0][p]).cuda(), torch.from_numpy(c.kv[b][1][p]).cuda(),
                             torch.from_numpy(slots).cuda())
    return gp, tables


@pytest.mark.parametrize("dt,Hq,S,Rp,win,lens", [
    ("bf16", 8, 16, 45, 700, [1500, 64, 3000, 701]),
    ("fp8", 16, 16, 40, 600, [10, 700, 5000]),
    ("f32", 4, 8, 10, 77, [78, 500]),
])
def test_ring_decode_equals_full_table_window_bit_for_bit(torch_cuda, dt, Hq, S, Rp, win, lens):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    c = RingCase(600 + Rp, lens, Hq, 2, 128, S, dt, Rp)
    assert c.N >= win
    gp, _ = pools(c)
    c.write(gp, None)
    fp, tables = full_table_pool(c)
    q = torch.from_numpy(c.rng.standard_normal((c.B, Hq, 128)).astype(np.float32)).cuda()
    lens_t = torch.from_numpy(c.lens).cuda()
    ring_out = tl.tl_paged_attn_decode_ring(gp, q, torch.from_numpy(c.ring).cuda(), lens_t, win, 0.088388346)
    full_out = tl.tl_paged_attn_decode(fp, q, torch.from_numpy(tables).cuda(), lens_t, win, 0.088388346)
    torch.cuda.synchronize()
    assert torch.equal(ring_out, full_out)


@pytest.mark.parametrize("dt,Hq,Hkv,D,S,win,chunk,extra", [
    ("bf16", 8, 2, 128, 16, 100, 40, 0),     # ring sized for the chunk
    ("f32", 4, 2, 64, 16, 50, 16, 0),
    ("fp8", 16, 2, 128, 16, 64, 24, 0),
    ("bf16", 8, 2, 128, 16, 100, 40, 1),     # one page more than needed
])
def test_chunked_ring_prefill_parity_and_equals_full_table(torch_cuda, dt, Hq, Hkv, D, S, win, chunk, extra):
    """Rows of two sequences prefilled in calls of `chunk` tokens through their rings:
    each call's output matches the ring oracle and, bit for bit, the full-table entry
    with the same window on a full-history pool."""
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    total = 7 * chunk + 5
    Rp = -(-(win - 1 + chunk) // S) + extra  # ceil((W - 1 + n) / S) pages
    c = RingCase(700 + win + chunk, [total, total - 9], Hq, Hkv, D, S, dt, Rp)
    gp, op = pools(c)
    fp, tables = full_table_pool(c, upto=np.zeros(c.B, np.int64))
    qs = [c.rng.standard_normal((int(L), Hq, D)).astype(np.float32) for L in c.lens]
    scale = 1.0 / np.sqrt(D)
    ring_t, tab_t = torch.from_numpy(c.ring).cuda(), torch.from_numpy(tables).cuda()
    worst = 0.0
    for p0 in range(0, total, chunk):
        # right-aligned rows of `chunk` tokens: pads (position -1) first where a row has fewer
        pos = np.full((c.B, chunk), -1, np.int32)
        q = np.zeros((c.B, chunk, Hq, D), np.float32)
        for b in range(c.B):
            p = np.arange(p0, min(int(c.lens[b]), p0 + chunk))
            if p.size:
                pos[b, chunk - p.size:] = p
                q[b, chunk - p.size:] = qs[b][p]
        ks, vs, rs, os_, fs = [], [], [], [], []
        for b in range(c.B):
            p = pos[b][pos[b] >= 0]
            if p.size == 0:
                continue
            ks.append(c.kv[b][0][p]); vs.append(c.kv[b][1][p])
            rs.append(ring_slots_gpu(c.ring[b], p, S, c.P))
            os_.append(oracle.ring_slots(c.ring[b], p, S))
            fs.append((tables[b, p // S] * S + p % S).astype(np.int32))
        k, v = np.concatenate(ks), np.concatenate(vs)
        kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        tl.tl_kv_cache_write(gp, kt, vt, torch.from_numpy(np.concatenate(rs)).cuda())
        tl.tl_kv_cache_write(fp, kt, vt, torch.from_numpy(np.concatenate(fs)).cuda())
        op.write(k, v, np.concatenate(os_))
        qt, pt = torch.from_numpy(q).cuda(), torch.from_numpy(pos).cuda()
        ring_out = tl.tl_paged_attn_prefill_ring(gp, qt, ring_t, pt, win, scale)
        full_out = tl.tl_paged_attn_prefill(fp, qt, tab_t, pt, win, scale)
        torch.cuda.synchronize()
        assert torch.equal(ring_out, full_out), f"call at {p0}: ring differs from the full table"
        ref = oracle.prefill_ring(op, q, c.ring, pos, win, scale)
        got = ring_out.cpu().numpy()
        worst = max(worst, row_rel_err(got, ref))
        assert np.all(got[pos < 0] == 0)
    assert_pool_equal(gp, op)
    assert worst <= TOL[dt], f"max row error {worst:.3e}"


def test_prefill_chunk_too_long_for_the_ring_follows_the_age_mask(torch_cuda):
    """A call that writes more than the ring can hold past the window: the kernel still
    scores each slot by its age, as stored (the oracle's reading), and the result then
    differs from the full-history model."""
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    S, win, chunk_ok = 16, 60, 20
    Rp = -(-(win - 1 + chunk_ok) // S)
    chunk = Rp * S - (win - 1) + 1  # one token more than fits once p0 >= W - 1
    total = 6 * chunk  # calls from p0 = 3 * chunk on start past W - 1
    c = RingCase(800, [total], 8, 2, 128, S, "f32", Rp)
    gp, op = pools(c)
    fp, tables = full_table_pool(c, upto=np.zeros(1, np.int64))
    qs = c.rng.standard_normal((total, 8, 128)).astype(np.float32)
    scale = 0.088388346
    differs = False
    for p0 in range(0, total, chunk):
        p = np.arange(p0, min(total, p0 + chunk))
        k, v = c.kv[0][0][p], c.kv[0][1][p]
        kt, vt = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        tl.tl_kv_cache_write(gp, kt, vt, torch.from_numpy(ring_slots_gpu(c.ring[0], p, S, c.P)).cuda())
        tl.tl_kv_cache_write(fp, kt, vt, torch.from_numpy((tables[0, p // S] * S + p % S).astype(np.int32)).cuda())
        op.write(k, v, oracle.ring_slots(c.ring[0], p, S))
        pos = p[None].astype(np.int32)
        qt, pt = torch.from_numpy(qs[p][None].copy()).cuda(), torch.from_numpy(pos).cuda()
        ring_out = tl.tl_paged_attn_prefill_ring(gp, qt, torch.from_numpy(c.ring).cuda(), pt, win, scale)
        full_out = tl.tl_paged_attn_prefill(fp, qt, torch.from_numpy(tables).cuda(), pt, win, scale)
        torch.cuda.synchronize()
        ref = oracle.prefill_ring(op, qs[p][None], c.ring, pos, win, scale)
        assert row_rel_err(ring_out.cpu().numpy(), ref) <= 2e-5
        differs |= not torch.equal(ring_out, full_out)
    assert differs
