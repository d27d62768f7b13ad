"""Host logic: byte accounting against the pages' printed numbers, and the seeded generator."""
import json
import os

import numpy as np
import pytest

from paged_kv_attention_cache_amd import accounting as A
from paged_kv_attention_cache_amd import workloads as W

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_llama3_kv_bytes_per_token_and_sequence():
    g = G["llama3_8b_bf16"]
    per_tok = A.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
    assert per_tok == g["bytes_per_token"]
    assert per_tok * g["seq_positions"] == g["bytes_per_seq"]
    wrong = A.kv_bytes_per_token(g["layers"], g["q_heads"], g["head_dim"], g["elem_bytes"])
    assert wrong * g["seq_positions"] == g["bytes_per_seq_with_q_heads"]


def test_muse_glimmer_full_and_windowed_table():
    g = G["muse_glimmer_f32_pages"]
    assert A.page_bytes(g["page_size"], g["kv_heads"], g["head_dim"], g["elem_bytes"]) == g["page_bytes_per_layer"]
    assert A.ring_pages_default(g["window"], g["page_size"]) == g["ring_pages"]
    full_layers = g["layers"] - g["window_layers"]
    for row in g["rows"]:
        full = A.full_history_bytes(row["positions"], g["layers"], g["page_size"], g["kv_heads"],
                                    g["head_dim"], g["elem_bytes"])
        win = A.windowed_bytes(row["positions"], full_layers, g["window_layers"], g["ring_pages"],
                               g["page_size"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
        assert round(A.mib(full)) == row["full_mib"]
        assert round(A.mib(win)) == row["windowed_mib"]
        assert round(full / win, 2) == row["ratio"]
    # the ratio approaches layers / full layers
    far = 1 << 24
    full = A.full_history_bytes(far, g["layers"], g["page_size"], g["kv_heads"], g["head_dim"], 4)
    win = A.windowed_bytes(far, full_layers, g["window_layers"], g["ring_pages"], g["page_size"],
                           g["kv_heads"], g["head_dim"], 4)
    assert abs(full / win - g["ratio_limit"]) < 1e-2
    four = 4 * A.full_history_bytes(32768, g["layers"], g["page_size"], g["kv_heads"], g["head_dim"], 4)
    assert A.mib(four) == g["four_seqs_full_history_mib"]


def test_ring_sizes_and_call_limit():
    g = G["ring_for_chunk"]
    assert A.ring_pages_for_chunk(g["window"], g["chunk"], g["page_size"]) == g["ring_pages"]
    assert g["ring_pages"] * g["page_size"] == g["ring_positions"]
    assert A.ring_pages_default(g["window"], g["page_size"]) == g["default_ring_pages"]
    c = G["ring_call_limit"]
    ring = A.ring_pages_default(c["window"], c["page_size"])
    worst = min(A.ring_call_limit(ring, c["page_size"], p0, c["window"]) for p0 in range(0, 5000, 7))
    assert worst == c["min_tokens_with_spare_page"]


def test_gather_and_score_sizes():
    g = G["per_token_gather"]
    assert A.per_token_gather_bytes(g["tokens"], g["context"], g["kv_heads"], g["head_dim"], g["elem_bytes"]) == g["bytes"]
    g = G["score_tensor"]
    assert A.score_tensor_bytes(g["kv_heads"], g["rows"], g["keys"]) == g["bytes"]
    g = G["score_block"]
    assert A.score_tensor_bytes(g["heads"], g["tokens"], g["keys"]) == g["bytes"]
    g = G["call_scores_64x"]
    assert g["context"] // g["call_tokens"] == g["factor"]


def test_algorithmic_counts_small():
    # two sequences of lengths 3 and 5, 1 kv head of 4, 2 q heads, f32, pages of 2
    b = A.decode_bytes([3, 5], 2, 1, 4, 2, "f32")
    kv = (3 + 5) * 1 * 4 * 2 * 4
    qo = 2 * 2 * 2 * 4 * 4
    tables = (2 + 3) * 4
    assert b == kv + qo + tables + 2 * 4
    assert A.decode_bytes([3, 5], 2, 1, 4, 2, "fp8") == (3 + 5) * 4 * 2 + (3 + 5) * 2 * 4 + qo + tables + 8
    assert A.write_bytes([0, -1, 5], 2, 4, "bf16") == 2 * 2 * 4 * 2 * (4 + 2) + 12
    pos = np.array([[-1, 0, 1, 2]])
    assert A.prefill_flops(pos, 2, 4) == (0 + 1 + 2 + 3) * 4 * 4 * 2
    assert A.prefill_flops(pos, 2, 4, window=2) == (0 + 1 + 2 + 2) * 4 * 4 * 2


def test_config_shapes_match_their_descriptions():
    c1 = W.make("c1")
    assert list(c1.seq_lens) == [5, 37] and c1.num_pages == 8 and len(c1.spare_pages) == 4
    assert (c1.num_q_heads, c1.num_kv_heads, c1.head_dim, c1.page_size, c1.kv_dtype) == (4, 2, 64, 16, "f32")
    c2 = W.make("c2")
    assert c2.batch == 64 and c2.seq_lens.min() >= 512 and c2.seq_lens.max() <= 8192
    assert c2.num_pages == sum((int(L) + 15) // 16 for L in c2.seq_lens)
    c3 = W.make("c3")
    assert c3.tokens_per_row == 2048 and c3.row_lens.min() >= 64 and c3.row_lens.max() <= 2048
    pos = c3.row_positions()
    for b in range(c3.batch):
        n = int(c3.row_lens[b])
        assert np.all(pos[b, :2048 - n] == -1) and list(pos[b, 2048 - n:]) == list(range(n))
    c4 = W.make("c4")
    assert c4.num_pages == 4096 and list(c4.start_pos) == [30720, 30720]
    assert W.make("c4w").window == 4096
    c5 = W.make("c5")
    assert c5.batch == 128 and c5.seq_lens.min() >= 1024 and c5.seq_lens.max() <= 32768
    assert (c5.num_q_heads, c5.page_size, c5.kv_dtype) == (64, 64, "fp8")


def test_streams_are_per_sequence_and_deterministic():
    a, b = W.make("c2"), W.make("c2")
    assert np.array_equal(a.seq_lens, b.seq_lens) and np.array_equal(a.block_tables, b.block_tables)
    ka, _ = a.seq_kv(3)
    kb, _ = b.seq_kv(3)
    assert np.array_equal(ka, kb) and ka.dtype == np.float32
    # every page is used at most once across sequences
    t = a.block_tables[a.block_tables >= 0]
    assert len(np.unique(t)) == len(t)


def test_slots_follow_the_tables():
    wl = W.make("c1")
    s = wl.slots_for(1, np.arange(37))
    for j in range(37):
        assert s[j] == wl.block_tables[1][j // 16] * 16 + j % 16
    assert wl.slots_for(0, np.array([-1]))[0] == -1
    with pytest.raises(ValueError):
        wl.slots_for(0, np.array([16]))  # sequence 0 has one page


def test_history_batches_chunking_covers_every_history_token_once():
    wl = W.custom_decode(120, [70, 3, 129], 2, 1, 4, 8, "f32")
    wl.history_chunk_tokens = 50
    seen = []
    for k, v, s in wl.history_batches():
        assert len(s) <= 50
        seen += s.tolist()
    want = []
    for b in range(3):
        want += wl.slots_for(b, np.arange(int(wl.seq_lens[b]) - 1)).tolist()
    assert sorted(seen) == sorted(want)


def test_ring_workload_writes_what_the_ring_holds_once():
    """c2r: each sequence's ring of 129 pages receives its last 129*16 positions (the
    history's tail, then the step token), each ring slot once, at the windowed slot
    mapping (block j on ring entry j % 129)."""
    wl = W.make("c2r")
    R, S = wl.ring_pages, wl.page_size
    assert R == 129 and wl.window == 2048 and wl.block_tables.shape == (wl.batch, R)
    assert len(np.unique(wl.block_tables)) == wl.batch * R  # rings do not share pages
    seen = {}
    for k, v, s in wl.history_batches():
        assert len(np.unique(s)) == len(s)
        for x in s.tolist():
            seen[x] = seen.get(x, 0) + 1
    ks, vs, ss = wl.decode_step_rows()
    for x in ss.tolist():
        seen[x] = seen.get(x, 0) + 1
    assert max(seen.values()) == 1
    for b in (0, 7, wl.batch - 1):
        L = int(wl.seq_lens[b])
        p = np.arange(max(0, L - R * S), L)
        want = wl.block_tables[b][(p // S) % R] * S + p % S
        assert np.array_equal(wl.slots_for(b, p), want)
        assert all(int(x) in seen for x in want)
    assert len(seen) == sum(min(int(L), R * S) for L in wl.seq_lens)
