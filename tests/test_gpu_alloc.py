"""Prefix sharing on the GPU against the oracle, and against unshared histories.

- A seeded stream of start / append / fork / end operations is replayed on the
  library (tl_alloc_* for the decisions, tl_kv_copy_pages for copy-on-write,
  tl_kv_cache_write for the tokens) and on the oracle (oracle.alloc.PageAllocator,
  KVPool.copy_pages, KVPool.write).  The two allocators must make the same decisions,
  the whole GPU pool (values and scales, untouched pages included) must equal the
  oracle's byte for byte after every few operations, and the decode outputs of the
  live sequences must match oracle.decode ("How serving works in Tlaloc", section 3
  backend bullets; the KV-cache management page, "Reuse identical causal prefixes").
- A forked sequence that appends through copy-on-write decodes to exactly the bits of
  the same history written without sharing.
"""
import random

import numpy as np
import pytest

import oracle
from oracle.alloc import PageAllocator as RefAlloc, Refused
from tests.helpers import row_rel_err
from tests.test_gpu_parity import TOL, assert_pool_equal, torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_dtype,hq", [("bf16", 8), ("fp8", 16), ("int8", 8)])
def test_allocator_replay_on_the_gpu_pool_matches_the_oracle(torch_cuda, kv_dtype, hq):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    P, S, H, D, timeout = 24, 16, 2, 64, 6.0  # small enough that the stream meets reclaims and refusals
    rng = random.Random(1000 + hq)
    nrng = np.random.default_rng(1000 + hq)
    a, r = tl.PageAllocator(P, S, timeout), RefAlloc(P, S, timeout)
    gp = tl.KVPool.allocate(P, S, H, D, kv_dtype, fill_byte=0xA5)
    op = oracle.KVPool(P, S, H, D, kv_dtype, sentinel=0xA5)
    live, now, nid, copies, refusals, reclaims, decodes = [], 0.0, 0, 0, 0, 0, 0
    for step in range(200):
        now += rng.random()
        x = rng.random()
        if x < 0.15 or not live:
            a.start(nid, now); r.start(nid, now); live.append(nid); nid += 1
        elif x < 0.7:
            i, n = rng.choice(live), rng.randint(1, 2 * S + 3)
            try:
                want_slots, want_cp = r.append(i, n, now)
            except Refused:
                with pytest.raises(tl.TLError) as e:
                    a.append(i, n, now)
                assert e.value.code == tl.TL_ERR_NO_PAGES
                refusals += 1
            else:
                slots, cp = a.append(i, n, now)
                assert (slots, cp) == (want_slots, want_cp), step
                if cp:  # copy-on-write before the write, on both sides
                    tl.tl_kv_copy_pages(gp, torch.tensor([c[0] for c in cp], dtype=torch.int32).cuda(),
                                        torch.tensor([c[1] for c in cp], dtype=torch.int32).cuda())
                    op.copy_pages([c[0] for c in cp], [c[1] for c in cp])
                    copies += len(cp)
                k = (nrng.standard_normal((n, H, D)) * nrng.uniform(0.1, 4.0, (n, H, 1))).astype(np.float32)
                v = nrng.standard_normal((n, H, D)).astype(np.float32)
                tl.tl_kv_cache_write(gp, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                                     torch.tensor(slots, dtype=torch.int32).cuda())
                op.write(k, v, np.array(slots, np.int32))
        elif x < 0.82:
            i = rng.choice(live)
            kk = rng.randint(0, r.seqs[i]["len"])
            a.fork(i, nid, kk, now); r.fork(i, nid, kk, now); live.append(nid); nid += 1
        else:
            i = rng.choice(live)
            a.end(i); r.end(i); live.remove(i)
        n_live = len(live)
        live = [i for i in live if i in r.seqs]  # reclaimed sequences are gone on both sides
        reclaims += n_live - len(live)
        assert a.free_pages() == r.free_count(), step
        if step % 25 == 24 and live:
            torch.cuda.synchronize()
            assert_pool_equal(gp, op)
            mb = max(1, max(len(r.seqs[i]["pages"]) for i in live))
            tabs, lens = a.tables(live, mb)
            assert (tabs, lens) == tuple(r.table(live, mb))
            q = nrng.standard_normal((len(live), hq, D)).astype(np.float32)
            tab_np, len_np = np.array(tabs, np.int32), np.array(lens, np.int32)
            out = tl.tl_paged_attn_decode(gp, torch.from_numpy(q).cuda(), torch.from_numpy(tab_np).cuda(),
                                          torch.from_numpy(len_np).cuda(), 0, 0.125)
            torch.cuda.synchronize()
            ref = oracle.decode(op, q, tab_np, len_np, 0, 0.125)
            assert row_rel_err(out.cpu().numpy(), ref) <= TOL[kv_dtype], step
            decodes += 1
    torch.cuda.synchronize()
    assert_pool_equal(gp, op)
    assert copies > 0 and refusals > 0 and reclaims > 0 and decodes >= 5, (copies, refusals, reclaims, decodes)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_fork_copy_on_write_equals_unshared_histories(torch_cuda, kv_dtype):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    S, H, D, Hq, P = 16, 2, 128, 8, 24
    rng = np.random.default_rng(91)
    kv = {s: (rng.standard_normal((50, H, D)).astype(np.float32), rng.standard_normal((50, H, D)).astype(np.float32))
          for s in (1, 2)}
    kv[2][0][:37] = kv[1][0][:37]  # the shared prefix
    kv[2][1][:37] = kv[1][1][:37]
    lens = {1: 40, 2: 42}

    def write(pool, slots, s, p):
        k, v = kv[s]
        tl.tl_kv_cache_write(pool, torch.from_numpy(k[p]).cuda(), torch.from_numpy(v[p]).cuda(),
                             torch.tensor(slots, dtype=torch.int32).cuda())

    # shared: parent writes 37 tokens, child forks at 37 and appends 5, parent appends 3
    a = tl.PageAllocator(P, S, 1e9)
    gp = tl.KVPool.allocate(P, S, H, D, kv_dtype, fill_byte=0xA5)
    a.start(1, 0.0)
    slots, cp = a.append(1, 37, 0.0)
    assert cp == []
    write(gp, slots, 1, np.arange(37))
    a.fork(1, 2, 37, 1.0)
    slots, cp = a.append(2, 5, 2.0)
    assert len(cp) == 1  # position 37 goes into the shared page 2 (5 of 16 used): copy first
    tl.tl_kv_copy_pages(gp, torch.tensor([cp[0][0]], dtype=torch.int32).cuda(),
                        torch.tensor([cp[0][1]], dtype=torch.int32).cuda())
    write(gp, slots, 2, np.arange(37, 42))
    slots, cp = a.append(1, 3, 3.0)
    assert cp == []      # the parent's page 2 is its own again
    write(gp, slots, 1, np.arange(37, 40))
    tabs, ls = a.tables([1, 2], 4)
    assert ls == [40, 42] and tabs[0][:2] == tabs[1][:2] and tabs[0][2] != tabs[1][2]

    # unshared: each history written on its own pages
    b = tl.PageAllocator(P, S, 1e9)
    up = tl.KVPool.allocate(P, S, H, D, kv_dtype, fill_byte=0xA5)
    for s in (1, 2):
        b.start(s, 0.0)
        slots, _ = b.append(s, lens[s], 0.0)
        write(up, slots, s, np.arange(lens[s]))
    utabs, _ = b.tables([1, 2], 4)

    q = torch.from_numpy(rng.standard_normal((2, Hq, D)).astype(np.float32)).cuda()
    lens_t = torch.tensor([40, 42], dtype=torch.int32).cuda()
    o1 = tl.tl_paged_attn_decode(gp, q, torch.tensor(tabs, dtype=torch.int32).cuda(), lens_t, 0, 0.088388346)
    o2 = tl.tl_paged_attn_decode(up, q, torch.tensor(utabs, dtype=torch.int32).cuda(), lens_t, 0, 0.088388346)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for i, s in enumerate((1, 2)):
        g1 = tl.tl_kv_gather(gp, torch.tensor(tabs[i], dtype=torch.int32).cuda(), lens[s])
        g2 = tl.tl_kv_gather(up, torch.tensor(utabs[i], dtype=torch.int32).cuda(), lens[s])
        torch.cuda.synchronize()
        for x, y in zip(g1, g2):
            if x is not None:
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
