"""Prefix sharing on the GPU: a forked sequence shares its parent's pages, the
allocator's copy-on-write copy runs with tl_kv_copy_pages before the child writes
into the shared partly filled page, and both sequences then gather and decode the same
bits as the same histories written without sharing."""
import numpy as np
import pytest

from tests.test_gpu_parity import torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu


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
