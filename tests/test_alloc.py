"""The library's host page allocator (tl_alloc_*, C++) against the reference model in
oracle/alloc.py, decision by decision on random operation sequences: the same slots,
the same page copies, the same refusals (with the same message naming the holders),
the same reclaims (visible in the tables) and the same free-page counts.  Host code
only: no GPU call is made."""
import random

import pytest

import paged_kv_attention_cache_amd as tl
from oracle.alloc import PageAllocator as Ref, Refused


@pytest.mark.parametrize("seed,pages,S,timeout", [(1, 30, 4, 5.0), (2, 12, 16, 2.0), (3, 64, 8, 1e9)])
def test_allocator_matches_the_reference_model(seed, pages, S, timeout):
    rng = random.Random(seed)
    a, r = tl.PageAllocator(pages, S, timeout), Ref(pages, S, timeout)
    live, now, nid = [], 0.0, 0
    for step in range(2500):
        now += rng.random()
        op = rng.random()
        if op < 0.15 or not live:
            a.start(nid, now); r.start(nid, now); live.append(nid); nid += 1
        elif op < 0.7:
            i, n = rng.choice(live), rng.randint(0, 2 * S + 1)
            try:
                want = r.append(i, n, now)
            except Refused as e:
                with pytest.raises(tl.TLError) as ge:
                    a.append(i, n, now)
                assert ge.value.code == tl.TL_ERR_NO_PAGES
                assert ge.value.message == "tl_alloc_append: " + str(e), step
            else:
                assert a.append(i, n, now) == (want[0], want[1]), step
        elif op < 0.8:
            i = rng.choice(live)
            k = rng.randint(0, r.seqs[i]["len"])
            a.fork(i, nid, k, now); r.fork(i, nid, k, now); live.append(nid); nid += 1
        else:
            i = rng.choice(live)
            a.end(i); r.end(i); live.remove(i)
        live = [i for i in live if i in r.seqs]
        assert a.free_pages() == r.free_count(), step
        if step % 50 == 0 and live:
            mb = max(1, max(len(r.seqs[i]["pages"]) for i in live))
            assert a.tables(live, mb) == r.table(live, mb)


def test_allocator_errors_name_the_argument():
    a = tl.PageAllocator(4, 4, 1.0)
    a.start(7, 0.0)
    with pytest.raises(tl.TLError, match="sequence 7 is already started"):
        a.start(7, 0.0)
    with pytest.raises(tl.TLError, match="sequence 8 is not started"):
        a.append(8, 1, 0.0)
    with pytest.raises(tl.TLError, match="prefix of 3 tokens is outside sequence 7"):
        a.fork(7, 9, 3, 0.0)
    a.append(7, 16, 0.0)
    with pytest.raises(tl.TLError) as e:
        a.append(7, 1, 0.5)
    assert e.value.code == tl.TL_ERR_NO_PAGES and "held by: 7 (4 pages)" in e.value.message
