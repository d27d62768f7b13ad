"""CPU oracle for the paged KV write and paged attention path.

TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct numpy (f64)
implementation of what the HIP path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it; the library and its Python binding never do, and it shares no code with
them (the seeded input generator in ``paged_kv_attention_cache_amd.workloads``
is the only module both sides read, and it holds none of the method's
arithmetic).

Parity pins: every function here is pinned in ``tests/test_oracle_*.py`` to
something other than itself (format definitions, closed forms, brute force,
invariants the pages state, and the pages' printed byte counts).
"""
from . import alloc, encode, gdn, paged  # noqa: F401
from .paged import (KVPool, KEY_BLOCK, attend_rows, attend_rows_blockwise, decode, decode_ring,  # noqa: F401
                    prefill, prefill_ring, ring_slots, slot_mapping)
