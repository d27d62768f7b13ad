"""Pins of the ring (windowed KV pool) oracle against things other than itself.

Page "How serving works in Tlaloc", section 3 (windowed KV pool) and section 2
(ring bullet), and the verification table's windowed-pool rows:
- the slot mapping: logical block b on ring page b % R, so N consecutive
  positions fill the ring's N slots once each and position p + N reuses p's slot;
- a ring that holds the window gives exactly the attention of the full-history
  windowed model (the pages report bit-identical results for the two layouts in
  their interpreter): compared bit for bit against attention over the window's
  slice of a full-history pool holding the same K/V;
- a ring one page short, or a prefill chunk one token too long for the ring,
  changes the result (the pages' negative controls);
- closed form: a window of 1 returns the value stored at the last position.
"""
import numpy as np
import pytest

from oracle import encode as E
from oracle.paged import KVPool, attend_rows, decode_ring, prefill_ring, ring_live_slots, ring_slots

S, H, G, D = 4, 2, 2, 16
SCALE = 0.25


def seq_kv(n, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, H, D)).astype(np.float32)
    v = rng.standard_normal((n, H, D)).astype(np.float32)
    return k, v


def full_pool(k, v, kv_dtype, seed=1):
    """A full-history pool holding positions 0..n-1 on shuffled pages, and its table."""
    n = k.shape[0]
    pages = (n + S - 1) // S
    table = np.random.default_rng(seed).permutation(pages + 3)[:pages].astype(np.int32)
    pool = KVPool(pages + 3, S, H, D, kv_dtype)
    j = np.arange(n)
    pool.write(k, v, (table[j // S] * S + j % S).astype(np.int32))
    return pool, table


def ring_pool(R, kv_dtype, seed=2):
    ring = np.random.default_rng(seed).permutation(R + 5)[:R].astype(np.int32)
    return KVPool(R + 5, S, H, D, kv_dtype), ring


def window_reference(pool, table, q, p, window):
    """Attention of the query at position p over the window slice of the full history."""
    lo = 0 if window <= 0 else max(0, p - window + 1)
    K, V = pool.gather_values(table, p + 1)
    out = np.zeros((H * G, D), np.float32)
    for h in range(H):
        o = attend_rows(q[h * G:(h + 1) * G], K[lo:, h], V[lo:, h], np.full(G, p - lo), 0, SCALE)
        out[h * G:(h + 1) * G] = o.astype(np.float32)
    return out


def test_ring_slots_cover_the_ring_once_and_repeat_with_period_n():
    R = 5
    ring = np.array([7, 2, 9, 0, 4], np.int32)
    N = R * S
    for p0 in (0, 3, 17, 1000):
        s = ring_slots(ring, np.arange(p0, p0 + N), S)
        want = sorted(int(pg) * S + o for pg in ring for o in range(S))
        assert sorted(s.tolist()) == want
        assert np.array_equal(ring_slots(ring, np.arange(p0, p0 + N) + N, S), s)
    assert ring_slots(ring, np.array([-1, 5]), S)[0] == -1
    # position p sits on the ring page of its logical block, at offset p % S
    p = np.arange(200)
    assert np.array_equal(ring_slots(ring, p, S), ring[(p // S) % R] * S + p % S)


def test_live_slots_are_the_last_positions_in_position_order():
    N = 12
    for L in (1, 5, 12, 13, 40):
        for W in (0, 1, 5, 12, 30):
            live = ring_live_slots(L, W, N)
            n = min(L, N) if W <= 0 else min(L, W, N)
            want = [p % N for p in range(L - n, L)]  # the last n positions, oldest first
            assert live == want, (L, W)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("W,R,L", [
    (8, 2, 5),      # ring not yet full
    (8, 2, 8),      # exactly one window
    (8, 3, 8),      # the default spare page
    (8, 3, 41),     # wrapped several times
    (7, 2, 30),     # window not a page multiple
    (1, 1, 19),     # window of one
    (0, 4, 16),     # no window, ring holds the whole history
])
def test_ring_decode_equals_full_history_window_bit_for_bit(kv_dtype, W, R, L):
    k, v = seq_kv(L, seed=10 + L)
    fp, table = full_pool(k, v, kv_dtype)
    rp, ring = ring_pool(R, kv_dtype)
    rp.write(k, v, ring_slots(ring, np.arange(L), S))  # in position order: later ones overwrite
    q = np.random.default_rng(3).standard_normal((1, H * G, D)).astype(np.float32)
    got = decode_ring(rp, q, ring[None], np.array([L]), W, SCALE)[0]
    want = window_reference(fp, table, q[0], L - 1, W)
    assert np.array_equal(got, want)


def test_window_of_one_returns_the_last_value():
    L, R = 23, 2
    k, v = seq_kv(L, seed=5)
    rp, ring = ring_pool(R, "f32")
    rp.write(k, v, ring_slots(ring, np.arange(L), S))
    q = np.random.default_rng(4).standard_normal((1, H * G, D)).astype(np.float32)
    got = decode_ring(rp, q, ring[None], np.array([L]), 1, SCALE)[0]
    for h in range(H):
        assert np.array_equal(got[h * G:(h + 1) * G], np.repeat(v[L - 1, h][None], G, axis=0))


def test_negative_control_ring_one_page_short_changes_decode():
    W, L = 8, 30
    k, v = seq_kv(L, seed=6)
    fp, table = full_pool(k, v, "f32")
    q = np.random.default_rng(7).standard_normal((1, H * G, D)).astype(np.float32)
    want = window_reference(fp, table, q[0], L - 1, W)
    R_short = (W + S - 1) // S - 1  # one page less than a window needs
    rp, ring = ring_pool(R_short, "f32")
    rp.write(k, v, ring_slots(ring, np.arange(L), S))
    got = decode_ring(rp, q, ring[None], np.array([L]), W, SCALE)[0]
    assert np.abs(got - want).max() > 1e-3


def chunked_ring_prefill(k, v, q, W, R, chunk, kv_dtype="f32"):
    """Write and attend the sequence through a ring in calls of `chunk` tokens."""
    n = k.shape[0]
    rp, ring = ring_pool(R, kv_dtype)
    out = np.zeros((n, H * G, D), np.float32)
    for p0 in range(0, n, chunk):
        p = np.arange(p0, min(n, p0 + chunk))
        rp.write(k[p], v[p], ring_slots(ring, p, S))
        out[p] = prefill_ring(rp, q[p][None], ring[None], p[None], W, SCALE)[0]
    return out


@pytest.mark.parametrize("W,chunk", [(8, 3), (8, 5), (6, 4), (5, 1)])
def test_chunked_prefill_through_a_sized_ring_equals_full_history(W, chunk):
    n = 37
    k, v = seq_kv(n, seed=20 + W)
    q = np.random.default_rng(21).standard_normal((n, H * G, D)).astype(np.float32)
    fp, table = full_pool(k, v, "f32")
    R = -(-(W - 1 + chunk) // S)  # ceil((W - 1 + N) / S): a call of `chunk` tokens fits past the window
    got = chunked_ring_prefill(k, v, q, W, R, chunk)
    for p in range(n):
        assert np.array_equal(got[p], window_reference(fp, table, q[p], p, W)), p


def test_negative_control_chunk_one_token_too_long_changes_prefill():
    n, W, chunk = 37, 8, 5
    k, v = seq_kv(n, seed=30)
    q = np.random.default_rng(31).standard_normal((n, H * G, D)).astype(np.float32)
    R = -(-(W - 1 + chunk) // S)
    N = R * S
    too_long = N - (W - 1) + 1  # min(p0, W - 1) + n = N + 1 once p0 >= W - 1
    fp, table = full_pool(k, v, "f32")
    got = chunked_ring_prefill(k, v, q, W, R, too_long)
    diffs = [np.abs(got[p] - window_reference(fp, table, q[p], p, W)).max() for p in range(n)]
    assert max(diffs) > 1e-3
