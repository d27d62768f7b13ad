"""CPU oracle of the paged KV write and paged attention (decode and prefill).

TEST INFRASTRUCTURE ONLY.  This is a plain, slow, f64 numpy reference.  Nothing
in the product path imports it: only tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` do.  It shares no code with the HIP kernels.

What it follows (page "How serving works in Tlaloc"):
- section 1: KV_CACHE_WRITE stores each token's K and V into the pool, then
  PAGED_ATTENTION reads them; a decode entry has one new token per sequence, a
  prefill entry right-aligns each sequence in its own row with pads first
  (slot -1, never written), and a token's causal length is its position + 1;
- section 2, PAGED_ATTENTION bullet: gather the pages the block table names,
  score with a dot product, masked softmax, weighted sum of the values;
- section 2, blockwise bullet: a loop over 2,048-key blocks keeping a running
  max, a running sum and a running P.V, from the first block any row of the
  call can see to the block holding the call's last position; a row of
  length 0 comes out 0;
- section 2, KV_CACHE_WRITE bullet: a scatter into the pool at the token's slot;
- section 3, sliding-window paragraph: with window W the token at p reads only
  positions p-W+1 .. p;
- section 3, manifest bullets: a K pool and a V pool of numBlocks pages of
  blockSize tokens each.
Grouped-query attention (page "Serving Models", "Change the cache at the
architectural level"): H_q query heads share H_kv key/value heads; query head
h reads KV head h // (H_q / H_kv).

Readings where the pages are silent (each is listed in the design notes):
- pool layout [pages, H_kv, page_size, D] per K and V; fp8 scales [pages, H_kv, page_size];
- slot = page * page_size + offset; slot -1 skips; any other out-of-range slot is an error;
- the scale multiplies the finished dot product; exp is the natural exponential;
- a decode sequence of length L has its new token at position L-1;
- a pad has position -1 and an empty visible set, so its output row is 0.

Arithmetic: stored K/V are widened exactly to f64, Q (f32) is widened to f64,
scores, exponentials and sums are f64, and outputs are rounded to f32 once.
``dtype=np.float32`` runs the same steps in f32; it exists only to pin the
blockwise-vs-one-shot agreement that the pages state for f32.
"""
from __future__ import annotations

import numpy as np

from . import encode as enc

KEY_BLOCK = 2048  # the pages' key-block width for blockwise attention


# ===================================================================== pool
class KVPool:
    """One layer's K and V pools of ``num_pages`` pages of ``page_size`` tokens."""

    def __init__(self, num_pages: int, page_size: int, num_kv_heads: int, head_dim: int,
                 kv_dtype: str, sentinel: int = 0xA5):
        self.num_pages, self.page_size = num_pages, page_size
        self.num_kv_heads, self.head_dim, self.kv_dtype = num_kv_heads, head_dim, kv_dtype
        shp = (num_pages, num_kv_heads, page_size, head_dim)
        raw = enc.RAW_DTYPE[kv_dtype]
        nbytes = int(np.prod(shp)) * np.dtype(raw).itemsize
        self.k = np.frombuffer(bytearray([sentinel]) * nbytes, dtype=raw).reshape(shp).copy()
        self.v = self.k.copy()
        if kv_dtype in enc.SCALED:
            sshp = (num_pages, num_kv_heads, page_size)
            sb = bytearray([sentinel]) * (int(np.prod(sshp)) * 4)
            self.k_scale = np.frombuffer(sb, dtype=np.float32).reshape(sshp).copy()
            self.v_scale = self.k_scale.copy()
        else:
            self.k_scale = self.v_scale = None

    # ------------------------------------------------------------- write
    def write(self, k_new: np.ndarray, v_new: np.ndarray, slots: np.ndarray) -> None:
        """KV_CACHE_WRITE: for each token i in order, store enc(k_new[i]) at slots[i].

        k_new, v_new: f32 [n, H_kv, D]; slots: int [n].  Slot -1 writes nothing.
        """
        k_new = np.asarray(k_new, dtype=np.float32)
        v_new = np.asarray(v_new, dtype=np.float32)
        slots = np.asarray(slots).reshape(-1)
        n = slots.shape[0]
        if k_new.shape != (n, self.num_kv_heads, self.head_dim) or v_new.shape != k_new.shape:
            raise ValueError("write: k_new/v_new must be [n, H_kv, D]")
        limit = self.num_pages * self.page_size
        for i in range(n):
            s = int(slots[i])
            if s == -1:
                continue
            if s < 0 or s >= limit:
                raise ValueError(f"write: slot {s} of token {i} is outside the pool")
        live = np.nonzero(slots != -1)[0]
        if live.size == 0:
            return
        kr, ks = enc.encode_kv(k_new[live], self.kv_dtype)
        vr, vs = enc.encode_kv(v_new[live], self.kv_dtype)
        for j, i in enumerate(live):  # token order: a repeated slot keeps the last token
            page, off = divmod(int(slots[i]), self.page_size)
            self.k[page, :, off, :] = kr[j]
            self.v[page, :, off, :] = vr[j]
            if ks is not None:
                self.k_scale[page, :, off] = ks[j]
                self.v_scale[page, :, off] = vs[j]

    # ------------------------------------------------------------ gather
    def gather_raw(self, table_row: np.ndarray, length: int):
        """Stored rows of positions 0..length-1 in logical order.

        Position j lives on page table_row[j // S] at offset j % S.
        Returns (k_raw [L, H_kv, D], v_raw, k_scale [L, H_kv] or None, v_scale).
        """
        S = self.page_size
        j = np.arange(length)
        pages = np.asarray(table_row)[j // S].astype(np.int64)
        if length and (pages.min() < 0 or pages.max() >= self.num_pages):
            raise ValueError("gather: block table names a page outside the pool")
        off = j % S
        k = self.k[pages, :, off, :]
        v = self.v[pages, :, off, :]
        if self.kv_dtype in enc.SCALED:
            return k, v, self.k_scale[pages, :, off], self.v_scale[pages, :, off]
        return k, v, None, None

    def gather_values(self, table_row: np.ndarray, length: int):
        """Gathered K and V widened exactly to f64: [L, H_kv, D] each."""
        k, v, ks, vs = self.gather_raw(table_row, length)
        return (enc.kv_values(k, ks, self.kv_dtype), enc.kv_values(v, vs, self.kv_dtype))

    def copy_pages(self, src, dst) -> None:
        """Copy whole pages src[i] -> dst[i] (K, V and scales), in order."""
        for a, b in zip(src, dst):
            self.k[b] = self.k[a]
            self.v[b] = self.v[a]
            if self.k_scale is not None:
                self.k_scale[b] = self.k_scale[a]
                self.v_scale[b] = self.v_scale[a]

    def pool_bytes(self) -> bytes:
        """The whole pool (K, V, then scales) as bytes, for byte-exact comparison."""
        parts = [self.k.tobytes(), self.v.tobytes()]
        if self.k_scale is not None:
            parts += [self.k_scale.tobytes(), self.v_scale.tobytes()]
        return b"".join(parts)


# ======================================================= visible key ranges
def visible_range(pos: np.ndarray, window: int) -> tuple[np.ndarray, np.ndarray]:
    """Visible keys of a query at position p: lo..hi inclusive (empty when hi < lo).

    Causal: j <= p.  Window W > 0: j >= p - W + 1.  A pad (p < 0) sees nothing.
    """
    pos = np.asarray(pos, dtype=np.int64)
    hi = pos.copy()
    lo = np.zeros_like(pos) if window <= 0 else np.maximum(pos - window + 1, 0)
    lo = np.where(pos < 0, 0, lo)
    hi = np.where(pos < 0, -1, hi)
    return lo, hi


# ================================================================ one-shot
def attend_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray, window: int,
                scale: float, dtype=np.float64, max_elems: int = 1 << 24) -> np.ndarray:
    """Softmax attention of R query rows over one head's contiguous history.

    q [R, D] f32, K/V [L, D] (stored values), pos [R].  Each row attends over its
    visible keys with s_j = (q . k_j) * scale, w = exp(s - max s),
    o = sum w_j v_j / sum w_j; an empty visible set gives o = 0.
    Returns [R, D] in ``dtype`` (f64 by default).
    """
    q = np.asarray(q, dtype=np.float32).astype(dtype)
    K = np.asarray(K).astype(dtype)
    V = np.asarray(V).astype(dtype)
    R, L = q.shape[0], K.shape[0]
    lo, hi = visible_range(pos, window)
    if np.any(hi >= L):
        raise ValueError("attend_rows: a query position is beyond the gathered history")
    out = np.zeros((R, q.shape[1]), dtype=dtype)
    sc = dtype(np.float32(scale))
    step = max(1, max_elems // max(L, 1))
    j = np.arange(L)
    for a in range(0, R, step):
        c = min(R, a + step)
        s = (q[a:c] @ K.T) * sc
        vis = (j[None, :] >= lo[a:c, None]) & (j[None, :] <= hi[a:c, None])
        s = np.where(vis, s, -np.inf)
        any_vis = vis.any(axis=1)
        m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0).astype(dtype)
        w = np.where(vis, np.exp(s - m[:, None]), 0).astype(dtype)
        den = w.sum(axis=1)
        num = w @ V
        out[a:c] = np.where(any_vis[:, None], num / np.where(any_vis, den, 1)[:, None], 0)
    return out


# =============================================================== blockwise
def attend_rows_blockwise(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray,
                          window: int, scale: float, dtype=np.float64, block: int = KEY_BLOCK,
                          first_block: int | None = None, last_block: int | None = None) -> np.ndarray:
    """The same attention as ``attend_rows`` by the online softmax over key blocks.

    Blocks are absolute positions [block*c, block*c + block - 1].  c runs from the
    first block any row can see to the block holding the last position (or the
    given bounds).  Per block, for each row that sees at least one key of it:
        m' = max(m, max_j s_j)
        a  = exp(m - m')
        l  = l * a + sum_j exp(s_j - m')
        acc = acc * a + sum_j exp(s_j - m') v_j
    A row that sees no key of a block skips it.  Finally o = acc / l (0 if l == 0).
    """
    q = np.asarray(q, dtype=np.float32).astype(dtype)
    K = np.asarray(K).astype(dtype)
    V = np.asarray(V).astype(dtype)
    R, D = q.shape
    lo, hi = visible_range(pos, window)
    live = hi >= lo
    if not live.any():
        return np.zeros((R, D), dtype=dtype)
    if np.any(hi >= K.shape[0]):
        raise ValueError("attend_rows_blockwise: a query position is beyond the history")
    c0 = int(lo[live].min()) // block if first_block is None else first_block
    c1 = int(hi[live].max()) // block if last_block is None else last_block
    sc = dtype(np.float32(scale))
    m = np.full(R, -np.inf, dtype=dtype)
    l = np.zeros(R, dtype=dtype)
    acc = np.zeros((R, D), dtype=dtype)
    for c in range(c0, c1 + 1):
        a_, b_ = c * block, min((c + 1) * block, K.shape[0])
        if a_ >= b_:
            continue
        j = np.arange(a_, b_)
        vis = (j[None, :] >= lo[:, None]) & (j[None, :] <= hi[:, None])
        rows = vis.any(axis=1)
        if not rows.any():
            continue
        s = (q[rows] @ K[a_:b_].T) * sc
        vr = vis[rows]
        s = np.where(vr, s, -np.inf)
        m_new = np.maximum(m[rows], s.max(axis=1))
        alpha = np.exp(m[rows] - m_new).astype(dtype)  # m = -inf gives 0
        p = np.where(vr, np.exp(s - m_new[:, None]), 0).astype(dtype)
        l[rows] = l[rows] * alpha + p.sum(axis=1)
        acc[rows] = acc[rows] * alpha[:, None] + p @ V[a_:b_]
        m[rows] = m_new
    out = np.zeros((R, D), dtype=dtype)
    nz = l > 0
    out[nz] = acc[nz] / l[nz, None]
    return out


# ================================================================== decode
def decode(pool: KVPool, q: np.ndarray, block_tables: np.ndarray, seq_lens: np.ndarray,
           window: int, scale: float, seqs=None) -> np.ndarray:
    """PAGED_ATTENTION for a decode entry: the new token of sequence b is at seq_lens[b]-1.

    q [B, H_q, D] f32.  Returns f32 [B, H_q, D] (only rows of ``seqs`` filled if given).
    """
    q = np.asarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    G = Hq // pool.num_kv_heads
    out = np.zeros((B, Hq, D), dtype=np.float32)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K, V = pool.gather_values(block_tables[b], L)
        for h in range(pool.num_kv_heads):
            rows = slice(h * G, (h + 1) * G)
            o = attend_rows(q[b, rows], K[:, h], V[:, h], np.full(G, L - 1), window, scale)
            out[b, rows] = o.astype(np.float32)
    return out


# ================================================================= prefill
def prefill(pool: KVPool, q: np.ndarray, block_tables: np.ndarray, positions: np.ndarray,
            window: int, scale: float, blockwise: bool = False, dtype=np.float64,
            tokens=None) -> np.ndarray:
    """PAGED_ATTENTION for a prefill entry with right-aligned rows.

    q [B, T, H_q, D] f32, positions [B, T] (-1 = pad).  Each row's pages are
    gathered once (up to its last position) and every token of the row attends
    over them with its own causal length position + 1.  ``tokens`` optionally
    restricts the computed rows to a list of (b, t) pairs; other rows stay 0.
    Returns f32 [B, T, H_q, D].
    """
    q = np.asarray(q, dtype=np.float32)
    positions = np.asarray(positions)
    B, T, Hq, D = q.shape
    G = Hq // pool.num_kv_heads
    out = np.zeros((B, T, Hq, D), dtype=np.float32)
    want = {}
    if tokens is not None:
        for b, t in tokens:
            want.setdefault(int(b), []).append(int(t))
    first = last = None
    if blockwise:  # the call's block range: first block any row sees .. block of the last position
        lo, hi = visible_range(positions.reshape(-1), window)
        lv = hi >= lo
        if lv.any():
            first, last = int(lo[lv].min()) // KEY_BLOCK, int(hi[lv].max()) // KEY_BLOCK
    for b in range(B):
        ts = np.arange(T) if tokens is None else np.array(sorted(want.get(b, [])), dtype=np.int64)
        if ts.size == 0:
            continue
        pos = positions[b, ts].astype(np.int64)
        if pos.max() < 0:
            continue
        L = int(pos.max()) + 1
        K, V = pool.gather_values(block_tables[b], L)
        for h in range(pool.num_kv_heads):
            qh = q[b][ts][:, h * G:(h + 1) * G, :].reshape(-1, D)  # rows (t, g)
            ph = np.repeat(pos, G)
            if blockwise:
                o = attend_rows_blockwise(qh, K[:, h], V[:, h], ph, window, scale, dtype,
                                          first_block=first, last_block=last)
            else:
                o = attend_rows(qh, K[:, h], V[:, h], ph, window, scale, dtype)
            out[b, ts, h * G:(h + 1) * G, :] = o.reshape(len(ts), G, D).astype(np.float32)
    return out


# ====================================================== contiguous history
def attend_history(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray, window: int,
                   scale: float) -> np.ndarray:
    """Attention of one sequence's query rows over its history held contiguously.

    q [R, H_q, D] f32, K/V stored values [L, H_kv, D], pos [R].  Used for sampled
    checks at full size, where a sequence's stored history is rebuilt by
    encoding its K/V rows in logical order instead of paging a whole pool.
    Returns f32 [R, H_q, D].
    """
    q = np.asarray(q, dtype=np.float32)
    R, Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((R, Hq, D), dtype=np.float32)
    for h in range(Hkv):
        qh = q[:, h * G:(h + 1) * G, :].reshape(-1, D)
        o = attend_rows(qh, K[:, h], V[:, h], np.repeat(np.asarray(pos), G), window, scale)
        out[:, h * G:(h + 1) * G, :] = o.reshape(R, G, D).astype(np.float32)
    return out


# ============================================================= ring (windowed pool)
# Page "How serving works in Tlaloc", section 3 (windowed KV pool bullets) and
# section 2 (the ring bullet of PAGED_ATTENTION): a sliding-window layer keeps, per
# sequence, a ring of R pages.  Logical block b of the sequence lives on the ring's
# page b % R (the ring table's entry b % R), so position p overwrites position
# p - R*S.  Attention with ring = true scores the ring's N = R*S slots, masking
# each by its age: slot i (ring page i // S, offset i % S) holds the position
# (L - 1 - i) mod N behind the row's last one, and is live when that age is less
# than the window and less than L.
#
# Reading (the pages define the age from "the row's last" position): a decode row
# has L = seq_len; a prefill token at position p uses its own causal length
# L = p + 1 (section 1).  A slot is scored with whatever it holds; the pages size
# calls so that it holds the position its age names (min(p0, W - 1) + n <= N).
# W <= 0 (no window) leaves only the L bound.  Live slots are gathered oldest
# first, i.e. in the order of the positions they stand for.
def ring_slots(ring_row: np.ndarray, positions: np.ndarray, page_size: int) -> np.ndarray:
    """WINDOW_SLOT_MAPPING: slot of each position on the sequence's ring (-1 for p < 0)."""
    ring_row = np.asarray(ring_row, dtype=np.int64)
    R = ring_row.shape[0]
    p = np.asarray(positions, dtype=np.int64)
    blk = np.where(p < 0, 0, p) // page_size
    slot = ring_row[blk % R] * page_size + np.where(p < 0, 0, p) % page_size
    return np.where(p < 0, -1, slot).astype(np.int32)


def slot_mapping(tables: np.ndarray, positions: np.ndarray, page_size: int, num_pages: int,
                 ring_pages: int = 0) -> np.ndarray:
    """SLOT_MAPPING (ring_pages = 0) or WINDOW_SLOT_MAPPING (ring_pages = R) of a call.

    tables [B, width], positions [B, T].  Position p of row b is on the page of its
    block j = p // S (on a ring, j = (p // S) % R) at offset p % S, so its slot is
    tables[b][j] * S + p % S.  A pad (p < 0), a block past the table and an entry
    that is not a page of the pool give -1 (nothing is written there).
    """
    tables = np.asarray(tables, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    B, T = positions.shape
    width = tables.shape[1]
    out = np.full((B, T), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            p = int(positions[b, t])
            if p < 0:
                continue
            j = p // page_size
            if ring_pages > 0:
                j %= ring_pages
            if j >= width:
                continue
            page = int(tables[b, j])
            if 0 <= page < num_pages:
                out[b, t] = page * page_size + p % page_size
    return out


def ring_live_slots(L: int, window: int, n_slots: int) -> list[int]:
    """Ring slot indices live for a row of causal length L, oldest first."""
    live = []
    for i in range(n_slots):
        age = (L - 1 - i) % n_slots
        if age < L and (window <= 0 or age < window):
            live.append((age, i))
    live.sort(reverse=True)  # largest age (oldest position) first
    return [i for _, i in live]


def ring_values(pool: KVPool, ring_row: np.ndarray, slots_idx: list[int]):
    """Stored K and V of the given ring slot indices, widened exactly: [n, H_kv, D] each."""
    S = pool.page_size
    ring_row = np.asarray(ring_row, dtype=np.int64)
    idx = np.asarray(slots_idx, dtype=np.int64)
    pages = ring_row[idx // S]
    if idx.size and (pages.min() < 0 or pages.max() >= pool.num_pages):
        raise ValueError("ring: the ring table names a page outside the pool")
    off = idx % S
    k, v = pool.k[pages, :, off, :], pool.v[pages, :, off, :]
    ks = vs = None
    if pool.kv_dtype in enc.SCALED:
        ks, vs = pool.k_scale[pages, :, off], pool.v_scale[pages, :, off]
    return enc.kv_values(k, ks, pool.kv_dtype), enc.kv_values(v, vs, pool.kv_dtype)


def decode_ring(pool: KVPool, q: np.ndarray, ring_tables: np.ndarray, seq_lens: np.ndarray,
                window: int, scale: float) -> np.ndarray:
    """PAGED_ATTENTION decode with ring = true.  ring_tables [B, R]: sequence b's ring pages."""
    q = np.asarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    G = Hq // pool.num_kv_heads
    N = ring_tables.shape[1] * pool.page_size
    out = np.zeros((B, Hq, D), dtype=np.float32)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        live = ring_live_slots(L, window, N)
        K, V = ring_values(pool, ring_tables[b], live)
        n = len(live)
        for h in range(pool.num_kv_heads):
            rows = slice(h * G, (h + 1) * G)
            o = attend_rows(q[b, rows], K[:, h], V[:, h], np.full(G, n - 1), 0, scale)
            out[b, rows] = o.astype(np.float32)
    return out


def prefill_ring(pool: KVPool, q: np.ndarray, ring_tables: np.ndarray, positions: np.ndarray,
                 window: int, scale: float) -> np.ndarray:
    """PAGED_ATTENTION prefill with ring = true: each token masks the ring by its own age.

    q [B, T, H_q, D], positions [B, T] (-1 = pad, output 0).  Returns f32 [B, T, H_q, D].
    """
    q = np.asarray(q, dtype=np.float32)
    positions = np.asarray(positions)
    B, T, Hq, D = q.shape
    G = Hq // pool.num_kv_heads
    N = ring_tables.shape[1] * pool.page_size
    out = np.zeros((B, T, Hq, D), dtype=np.float32)
    for b in range(B):
        for t in range(T):
            p = int(positions[b, t])
            if p < 0:
                continue
            live = ring_live_slots(p + 1, window, N)
            K, V = ring_values(pool, ring_tables[b], live)
            n = len(live)
            for h in range(pool.num_kv_heads):
                rows = slice(h * G, (h + 1) * G)
                o = attend_rows(q[b, t, rows], K[:, h], V[:, h], np.full(G, n - 1), 0, scale)
                out[b, t, rows] = o.astype(np.float32)
    return out
