"""Pins of the reference page allocator against the pages' stated rules (see
oracle/alloc.py): ownership and reference counts stay consistent under random
operations, a refusal changes nothing but the refused sequence's activity time and
names the holders, reclaim takes idle sequences least recently active first and only
as many as needed, and copy-on-write gives a forked sequence its own copy of a shared
partly filled page before writing into it."""
import random

import pytest

from oracle.alloc import PageAllocator, Refused


def check_invariants(a: PageAllocator):
    count = [0] * len(a.ref)
    for s in a.seqs.values():
        assert len(s["pages"]) == (s["len"] + a.S - 1) // a.S
        for p in s["pages"]:
            count[p] += 1
    assert count == a.ref


def test_random_operations_keep_ownership_consistent():
    rng = random.Random(3)
    a = PageAllocator(40, 4, idle_timeout=5.0)
    live, now, next_id = [], 0.0, 0
    for _ in range(3000):
        now += rng.random()
        op = rng.random()
        try:
            if op < 0.15 or not live:
                a.start(next_id, now); live.append(next_id); next_id += 1
            elif op < 0.65:
                i = rng.choice(live)
                L = a.seqs[i]["len"]
                slots, copies = a.append(i, rng.randint(1, 9), now)
                pages = a.seqs[i]["pages"]
                assert slots == [pages[p // 4] * 4 + p % 4 for p in range(L, a.seqs[i]["len"])]
                for src, dst in copies:
                    assert a.ref[dst] == 1 and dst == pages[L // 4]
            elif op < 0.75:
                i = rng.choice(live)
                a.fork(i, next_id, rng.randint(0, a.seqs[i]["len"]), now); live.append(next_id); next_id += 1
            else:
                i = rng.choice(live)
                a.end(i); live.remove(i)
        except Refused:
            pass
        live = [i for i in live if i in a.seqs]  # reclaimed sequences are gone
        check_invariants(a)


def test_refusal_by_name_keeps_everything():
    a = PageAllocator(4, 4, idle_timeout=100.0)
    a.start(1, 0.0); a.append(1, 8, 0.0)    # 2 pages
    a.start(2, 0.0); a.append(2, 5, 0.0)    # 2 pages: pool full
    before = ([list(s["pages"]) for s in a.seqs.values()], list(a.ref))
    with pytest.raises(Refused) as e:
        a.append(2, 4, 10.0)                 # needs a third page: nobody is idle for 100
    assert "sequence 2 needs 1 pages, 0 free" in str(e.value)
    assert "1 (2 pages)" in str(e.value) and "2 (2 pages)" in str(e.value)
    assert ([list(s["pages"]) for s in a.seqs.values()], list(a.ref)) == before
    assert a.seqs[2]["last"] == 10.0 and a.seqs[2]["len"] == 5


def test_reclaim_least_recently_active_only_as_many_as_needed():
    a = PageAllocator(6, 4, idle_timeout=10.0)
    for i, t in ((1, 0.0), (2, 1.0), (3, 2.0)):
        a.start(i, t); a.append(i, 8, t)      # 2 pages each: pool full
    a.start(4, 50.0)
    a.append(4, 4, 50.0)                      # one page needed: reclaims sequence 1 only
    assert 1 not in a.seqs and 2 in a.seqs and 3 in a.seqs
    a.append(4, 8, 51.0)                      # two more: one free, then sequence 2
    assert 2 not in a.seqs and 3 in a.seqs
    a2 = PageAllocator(2, 4, idle_timeout=10.0)
    a2.start(1, 0.0); a2.append(1, 4, 0.0)
    a2.start(2, 9.0); a2.append(2, 4, 9.0)
    a2.start(3, 12.0)
    with pytest.raises(Refused):
        a2.append(3, 8, 12.0)                 # needs 2, only sequence 1 is idle (1 page)
    assert 1 in a2.seqs                       # nothing reclaimed on a refusal


def test_fork_shares_full_pages_and_copies_the_partial_one_on_write():
    a = PageAllocator(16, 4, idle_timeout=1e9)
    a.start(1, 0.0); a.append(1, 10, 0.0)    # pages for 0..3, 4..7, 8..9 (partial)
    p = list(a.seqs[1]["pages"])
    a.fork(1, 2, 10, 1.0)
    assert a.seqs[2]["pages"] == p and a.ref[p[2]] == 2 and a.ref[p[0]] == 2
    slots, copies = a.append(2, 1, 2.0)      # writes position 10 into the shared page
    new = a.seqs[2]["pages"][2]
    assert copies == [(p[2], new)] and new not in p and a.ref[p[2]] == 1
    assert slots == [new * 4 + 2] and a.seqs[2]["pages"][:2] == p[:2]
    slots, copies = a.append(1, 1, 3.0)      # the parent's last page is its own again
    assert copies == [] and slots == [p[2] * 4 + 2]
    a.fork(1, 3, 8, 4.0)                      # a page-aligned prefix: nothing to copy later
    slots, copies = a.append(3, 2, 5.0)
    assert copies == [] and a.seqs[3]["pages"][:2] == p[:2] and a.seqs[3]["pages"][2] not in p
    a.end(1)
    assert a.ref[p[0]] == 2 and a.ref[p[2]] == 0  # still held by 2 and 3; page 2 freed
