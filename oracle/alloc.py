"""Reference model of the host page allocator (per-sequence pages, refusal by name,
least-recently-active reclaim, prefix sharing with reference counts and copy-on-write).

TEST INFRASTRUCTURE ONLY: plain Python; the library's allocator (C++) is checked
against it decision by decision.  It shares no code with the library.

What it follows:
- page "How serving works in Tlaloc", the runtime comparison table and the backend
  bullets of section 3: pages are allocated per sequence and freed when it ends;
  when pages run short they are reclaimed only from sequences idle past the timeout,
  least recently active first and only as many as needed; otherwise the request is
  refused by name, listing the sequences that hold pages, and the refused sequence
  keeps its pages and KV (a refused request still counts as activity); a live
  sequence is never preempted;
- the page on KV-cache management ("Reuse identical causal prefixes" and the
  paragraph before it): shared prefixes need reference counts, a mutable suffix needs
  private storage or copy-on-write, and a page is freed only when no holder is left.

Readings (listed in the design notes): a free page is always the lowest-numbered
one; "idle past the timeout" is last activity < now - idle_timeout; reclaim happens
only when the reclaimable sequences can cover the whole shortage (else the request
is refused and nothing is reclaimed); a sequence sharing a partly filled last page
copies it (one new page) before its next token is written there.
"""
from __future__ import annotations


class Refused(Exception):
    """A request refused by name (no pages left)."""


class PageAllocator:
    def __init__(self, num_pages: int, page_size: int, idle_timeout: float):
        self.S = page_size
        self.timeout = idle_timeout
        self.ref = [0] * num_pages
        self.seqs: dict[int, dict] = {}  # id -> {"len", "pages", "last"}

    # ------------------------------------------------------------------ helpers
    def free_count(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def _take(self) -> int:
        p = self.ref.index(0)  # the lowest free page
        self.ref[p] = 1
        return p

    def _release(self, seq: int) -> None:
        for p in self.seqs[seq]["pages"]:
            self.ref[p] -= 1
        del self.seqs[seq]

    # --------------------------------------------------------------- operations
    def start(self, seq: int, now: float) -> None:
        if seq in self.seqs:
            raise ValueError(f"sequence {seq} is already started")
        self.seqs[seq] = {"len": 0, "pages": [], "last": now}

    def end(self, seq: int) -> None:
        if seq not in self.seqs:
            raise ValueError(f"sequence {seq} is not started")
        self._release(seq)

    def fork(self, parent: int, child: int, n_tokens: int, now: float) -> None:
        if parent not in self.seqs:
            raise ValueError(f"sequence {parent} is not started")
        if child in self.seqs:
            raise ValueError(f"sequence {child} is already started")
        par = self.seqs[parent]
        if not 0 <= n_tokens <= par["len"]:
            raise ValueError(f"prefix of {n_tokens} tokens is outside sequence {parent}")
        pages = par["pages"][: (n_tokens + self.S - 1) // self.S]
        for p in pages:
            self.ref[p] += 1
        self.seqs[child] = {"len": n_tokens, "pages": list(pages), "last": now}
        par["last"] = now

    def append(self, seq: int, n_tokens: int, now: float):
        """Room for n_tokens more positions: returns (slots, copies [(src, dst) pages])."""
        if seq not in self.seqs:
            raise ValueError(f"sequence {seq} is not started")
        s = self.seqs[seq]
        S, L = self.S, s["len"]
        new_pages = (L + n_tokens + S - 1) // S - len(s["pages"])
        cow = n_tokens > 0 and L % S != 0 and self.ref[s["pages"][-1]] > 1
        need = new_pages + int(cow)
        free = self.free_count()
        if need > free:
            idle = sorted((o["last"], i) for i, o in self.seqs.items()
                          if i != seq and o["last"] < now - self.timeout)
            # pages each reclaim would free, in order, counting shared pages once
            ref = list(self.ref)
            gain, take = 0, []
            for _, i in idle:
                if free + gain >= need:
                    break
                for p in self.seqs[i]["pages"]:
                    ref[p] -= 1
                    gain += ref[p] == 0
                take.append(i)
            if free + gain < need:
                s["last"] = now
                held = ", ".join(f"{i} ({len(o['pages'])} pages)" for i, o in sorted(self.seqs.items())
                                 if o["pages"])
                raise Refused(f"sequence {seq} needs {need} pages, {free} free; held by: {held}")
            for i in take:
                self._release(i)
        copies = []
        if cow:
            old = s["pages"][-1]
            new = self._take()
            self.ref[old] -= 1
            s["pages"][-1] = new
            copies.append((old, new))
        for _ in range(new_pages):
            s["pages"].append(self._take())
        slots = [s["pages"][p // S] * S + p % S for p in range(L, L + n_tokens)]
        s["len"] = L + n_tokens
        s["last"] = now
        return slots, copies

    def table(self, seqs: list[int], max_blocks: int):
        """Block tables [len(seqs)][max_blocks] (-1 unused) and lengths of the sequences."""
        rows, lens = [], []
        for i in seqs:
            p = self.seqs[i]["pages"]
            if len(p) > max_blocks:
                raise ValueError(f"sequence {i} holds {len(p)} pages, more than {max_blocks}")
            rows.append(p + [-1] * (max_blocks - len(p)))
            lens.append(self.seqs[i]["len"])
        return rows, lens
