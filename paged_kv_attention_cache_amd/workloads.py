"""Seeded synthetic workloads for the paged KV write + paged attention path.

This module only *draws* inputs: sequence lengths, page permutations, block
tables, slot ids, positions and N(0, 1) f32 query/key/value rows.  It holds none
of the attention arithmetic and none of the KV encoders, so both the CPU oracle
(under ``oracle/``) and the GPU path can consume the same inputs without
sharing any of the method's code.

Shapes follow the pages' workloads ("How serving works in Tlaloc", sections 2-3:
block tables, slot mapping with -1 for pads, right-aligned prefill rows,
2,048-key blocks, chunked prefill at 32,768 positions; "Serving Models",
"Count KV heads and distinct stored tensors": Llama-3-8B geometry of 8 KV heads
of 128).

Random streams: every tensor of every sequence has its own PCG64 stream,
``numpy.random.default_rng([seed, cfg_id, tensor_id, b])``, so a single sequence
can be regenerated on its own (the oracle does this for sampled parity checks
at full size).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Iterator

import numpy as np

# tensor ids of the per-sequence random streams
T_LENGTHS, T_PERM, T_Q, T_K, T_V, T_PAD_K, T_PAD_V = 0, 1, 2, 3, 4, 5, 6
SEED = 0


@dataclass
class Workload:
    """One seeded configuration.

    kind == "decode": sequence b holds ``seq_lens[b]`` positions including the
    new token (position seq_lens[b]-1).  Its history (positions
    0..seq_lens[b]-2) is written first, then the step token of every sequence,
    then one decode call.

    kind == "prefill": row b of the token axis (width ``tokens_per_row``) holds
    ``row_lens[b]`` live tokens at positions ``start_pos[b] ..`` right-aligned
    (pads first, slot -1, position -1).  Positions ``0 .. start_pos[b]-1`` are
    history written before the call.
    """

    name: str
    cfg_id: int
    kind: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str  # "f32" | "bf16" | "fp8" (scaled) | "fp8u" (unscaled) | "int8" (scaled)
    window: int = 0  # <= 0: full attention
    seq_lens: np.ndarray | None = None  # decode: [B] int32, incl. the new token
    tokens_per_row: int = 0  # prefill: T
    row_lens: np.ndarray | None = None  # prefill: [B] live tokens per row
    start_pos: np.ndarray | None = None  # prefill: [B] first live position
    num_pages: int = 0
    block_tables: np.ndarray | None = None  # [B, max_blocks] int32, -1 unused
    spare_pages: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    history_chunk_tokens: int = 1 << 16
    seed: int = SEED
    ring_pages: int = 0  # > 0: block_tables are [B, ring_pages] rings (windowed pool)

    # ---------------------------------------------------------------- shapes
    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        """Softmax scale as an f32 value: f32(1/sqrt(D))."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def context_len(self, b: int) -> int:
        """Positions sequence b holds after this workload's writes."""
        if self.kind == "decode":
            return int(self.seq_lens[b])
        return int(self.start_pos[b] + self.row_lens[b])

    def history_len(self, b: int) -> int:
        if self.kind == "decode":
            return max(0, int(self.seq_lens[b]) - 1)
        return int(self.start_pos[b])

    def history_start(self, b: int) -> int:
        """First history position written: 0, or on a ring the oldest position it still
        holds once the step token is written (earlier ones would be overwritten)."""
        if self.ring_pages <= 0:
            return 0
        return max(0, self.context_len(b) - self.ring_pages * self.page_size)

    # --------------------------------------------------------------- streams
    def _rng(self, tensor_id: int, b: int) -> np.random.Generator:
        return np.random.default_rng([self.seed, self.cfg_id, tensor_id, b])

    def seq_kv(self, b: int) -> tuple[np.ndarray, np.ndarray]:
        """K and V rows of sequence b for positions 0..context_len-1, f32 [L, H_kv, D]."""
        L = self.context_len(b)
        shp = (L, self.num_kv_heads, self.head_dim)
        k = self._rng(T_K, b).standard_normal(shp, dtype=np.float32)
        v = self._rng(T_V, b).standard_normal(shp, dtype=np.float32)
        return k, v

    def slots_for(self, b: int, positions: np.ndarray) -> np.ndarray:
        """Slot ids (page * page_size + offset) of sequence b's positions; -1 for p < 0."""
        positions = np.asarray(positions, dtype=np.int64)
        S = self.page_size
        out = np.full(positions.shape, -1, dtype=np.int32)
        live = positions >= 0
        blk = positions[live] // S
        if self.ring_pages > 0:  # windowed pool: block j on the ring's entry j % R
            blk = blk % self.ring_pages
        pages = self.block_tables[b][blk].astype(np.int64)
        if np.any(pages < 0):
            raise ValueError(f"sequence {b}: block table has no page for a written position")
        out[live] = (pages * S + positions[live] % S).astype(np.int32)
        return out

    # ------------------------------------------------------ decode workloads
    def decode_q(self, b: int | None = None) -> np.ndarray:
        """Query rows of the step token: [B, H_q, D] (or [H_q, D] for one b)."""
        shp = (self.num_q_heads, self.head_dim)
        if b is not None:
            return self._rng(T_Q, b).standard_normal(shp, dtype=np.float32)
        return np.stack([self._rng(T_Q, i).standard_normal(shp, dtype=np.float32)
                         for i in range(self.batch)])

    def history_batches(self) -> Iterator[tuple[np.ndarray, np.ndarray, np.ndarray]]:
        """History writes in chunks of at most ``history_chunk_tokens`` tokens.

        Yields (k_new [n, H_kv, D] f32, v_new, slots [n] int32).
        """
        ks, vs, ss, n = [], [], [], 0
        for b in range(self.batch):
            h = self.history_len(b)
            if h == 0:
                continue
            k, v = self.seq_kv(b)
            pos = np.arange(h)
            for a in range(self.history_start(b), h, self.history_chunk_tokens):
                c = min(h, a + self.history_chunk_tokens)
                if n + (c - a) > self.history_chunk_tokens and n:
                    yield np.concatenate(ks), np.concatenate(vs), np.concatenate(ss)
                    ks, vs, ss, n = [], [], [], 0
                ks.append(k[a:c]); vs.append(v[a:c]); ss.append(self.slots_for(b, pos[a:c]))
                n += c - a
        if n:
            yield np.concatenate(ks), np.concatenate(vs), np.concatenate(ss)

    def decode_step_rows(self) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
        """The step write of a decode workload: one token per sequence, at L-1."""
        ks, vs, ss = [], [], []
        for b in range(self.batch):
            L = int(self.seq_lens[b])
            if L == 0:  # nothing to write: a pad row
                z = np.zeros((self.num_kv_heads, self.head_dim), np.float32)
                ks.append(z); vs.append(z); ss.append(-1)
                continue
            k, v = self.seq_kv(b)
            ks.append(k[L - 1]); vs.append(v[L - 1])
            ss.append(self.slots_for(b, np.array([L - 1]))[0])
        return np.stack(ks), np.stack(vs), np.array(ss, dtype=np.int32)

    # ----------------------------------------------------- prefill workloads
    def row_positions(self) -> np.ndarray:
        """[B, T] int32 positions, -1 for pads (right-aligned rows)."""
        T = self.tokens_per_row
        pos = np.full((self.batch, T), -1, dtype=np.int32)
        for b in range(self.batch):
            n = int(self.row_lens[b])
            pos[b, T - n:] = self.start_pos[b] + np.arange(n)
        return pos

    def prefill_rows(self, b: int) -> tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
        """Row b of a prefill call: q [T, H_q, D], k/v [T, H_kv, D], slots [T].

        Pad tokens carry random K/V from their own streams (so a write that
        does not skip slot -1 shows up) and slot -1.
        """
        T, n = self.tokens_per_row, int(self.row_lens[b])
        q = self._rng(T_Q, b).standard_normal((T, self.num_q_heads, self.head_dim), dtype=np.float32)
        shp = (T, self.num_kv_heads, self.head_dim)
        k = self._rng(T_PAD_K, b).standard_normal(shp, dtype=np.float32)
        v = self._rng(T_PAD_V, b).standard_normal(shp, dtype=np.float32)
        if n:
            ks, vs = self.seq_kv(b)
            p0 = int(self.start_pos[b])
            k[T - n:] = ks[p0:p0 + n]
            v[T - n:] = vs[p0:p0 + n]
        pos = self.row_positions()[b]
        return q, k, v, self.slots_for(b, pos)

    def prefill_inputs(self):
        """All rows stacked: q [B,T,H_q,D], k/v [B,T,H_kv,D], slots [B,T], positions [B,T]."""
        rows = [self.prefill_rows(b) for b in range(self.batch)]
        q = np.stack([r[0] for r in rows]); k = np.stack([r[1] for r in rows])
        v = np.stack([r[2] for r in rows]); s = np.stack([r[3] for r in rows])
        return q, k, v, s, self.row_positions()


# ------------------------------------------------------------------ builders
def _assign_pages(wl: Workload, ctx_lens: list[int], num_pages: int | None = None,
                  spare: int = 0) -> None:
    """Hand each sequence ceil(L/S) pages of a seeded permutation, in order."""
    S = wl.page_size
    need = [(L + S - 1) // S for L in ctx_lens]
    P = sum(need) + spare if num_pages is None else num_pages
    if sum(need) > P:
        raise ValueError("page budget too small")
    perm = np.random.default_rng([wl.seed, wl.cfg_id, T_PERM, 0]).permutation(P).astype(np.int32)
    max_blocks = max(1, max(need))
    tables = np.full((wl.batch, max_blocks), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[at:at + n]
        at += n
    wl.num_pages = P
    wl.block_tables = tables
    wl.spare_pages = perm[at:]


def _assign_rings(wl: Workload, ring_pages: int, spare: int = 0) -> None:
    """Hand each sequence a ring of ring_pages pages of a seeded permutation, in order."""
    P = wl.batch * ring_pages + spare
    perm = np.random.default_rng([wl.seed, wl.cfg_id, T_PERM, 0]).permutation(P).astype(np.int32)
    wl.num_pages = P
    wl.ring_pages = ring_pages
    wl.block_tables = perm[:wl.batch * ring_pages].reshape(wl.batch, ring_pages).copy()
    wl.spare_pages = perm[wl.batch * ring_pages:]


def tiny_decode() -> Workload:
    """Tiny decode step: B=2 at lengths 5 and 37, H_q=4, H_kv=2, D=64, S=16, f32 pool of 8 pages."""
    wl = Workload("c1_tiny_decode", 1, "decode", 2, 4, 2, 64, 16, "f32",
                  seq_lens=np.array([5, 37], dtype=np.int32))
    _assign_pages(wl, [5, 37], num_pages=8)
    return wl


def llama3_decode(batch: int = 64, lo: int = 512, hi: int = 8192) -> Workload:
    """Llama-3-8B-shaped decode layer: H_q=32, H_kv=8, D=128, S=16, bf16 KV, L ~ U[512, 8192]."""
    rng = np.random.default_rng([SEED, 2, T_LENGTHS, 0])
    lens = rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)
    wl = Workload("c2_llama3_decode_bf16", 2, "decode", batch, 32, 8, 128, 16, "bf16", seq_lens=lens)
    _assign_pages(wl, lens.tolist())
    return wl


def llama3_decode_int8(batch: int = 64, lo: int = 512, hi: int = 8192) -> Workload:
    """The c2 decode layer (same lengths) on an int8 KV pool with per-(token, head) scales."""
    rng = np.random.default_rng([SEED, 2, T_LENGTHS, 0])  # the same lengths as c2
    lens = rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)
    wl = Workload("c2i_llama3_decode_int8", 8, "decode", batch, 32, 8, 128, 16, "int8", seq_lens=lens)
    _assign_pages(wl, lens.tolist())
    return wl


def llama3_decode_ring(batch: int = 64, lo: int = 512, hi: int = 8192, window: int = 2048) -> Workload:
    """The c2 decode layer as a sliding-window layer on a windowed pool: window 2,048,
    rings of ceil(2048/16) + 1 = 129 pages (section 3's default of one spare page)."""
    rng = np.random.default_rng([SEED, 2, T_LENGTHS, 0])  # the same lengths as c2
    lens = rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)
    wl = Workload("c2r_llama3_decode_bf16_window2048_ring", 6, "decode", batch, 32, 8, 128, 16, "bf16",
                  window=window, seq_lens=lens)
    _assign_rings(wl, -(-window // 16) + 1)
    return wl


def batched_prefill(batch: int = 8, T: int = 2048, lo: int = 64, hi: int = 2048) -> Workload:
    """Right-aligned batched prefill: B rows of T tokens, prompt lengths ~ U[64, 2048], bf16 KV."""
    rng = np.random.default_rng([SEED, 3, T_LENGTHS, 0])
    lens = rng.integers(lo, min(hi, T), size=batch, endpoint=True).astype(np.int32)
    wl = Workload("c3_batched_prefill_bf16", 3, "prefill", batch, 32, 8, 128, 16, "bf16",
                  tokens_per_row=T, row_lens=lens, start_pos=np.zeros(batch, np.int32))
    _assign_pages(wl, lens.tolist())
    return wl


def long_prefill(window: int = 0, batch: int = 2, history: int = 30720, chunk: int = 2048) -> Workload:
    """Long-context chunked prefill: history positions 0..history-1, then a chunk; bf16 KV."""
    name = "c4_long_prefill_bf16" + (f"_window{window}" if window > 0 else "")
    wl = Workload(name, 4, "prefill", batch, 32, 8, 128, 16, "bf16", window=window,
                  tokens_per_row=chunk, row_lens=np.full(batch, chunk, np.int32),
                  start_pos=np.full(batch, history, np.int32))
    _assign_pages(wl, [history + chunk] * batch)
    return wl


def fp8_decode(batch: int = 128, lo: int = 1024, hi: int = 32768) -> Workload:
    """fp8 KV decode: H_q=64, H_kv=8, D=128, S=64, L log-uniform in [1024, 32768]."""
    rng = np.random.default_rng([SEED, 5, T_LENGTHS, 0])
    u = rng.uniform(math.log(lo), math.log(hi), size=batch)
    lens = np.clip(np.round(np.exp(u)), lo, hi).astype(np.int32)
    wl = Workload("c5_fp8_decode", 5, "decode", batch, 64, 8, 128, 64, "fp8", seq_lens=lens)
    _assign_pages(wl, lens.tolist())
    return wl


def fp8_unscaled_decode(batch: int = 128, lo: int = 1024, hi: int = 32768) -> Workload:
    """c5's lengths and shape on the pages' own unscaled fp8 pool (no scale arrays)."""
    rng = np.random.default_rng([SEED, 5, T_LENGTHS, 0])  # the same lengths as c5
    u = rng.uniform(math.log(lo), math.log(hi), size=batch)
    lens = np.clip(np.round(np.exp(u)), lo, hi).astype(np.int32)
    wl = Workload("c5u_fp8_unscaled_decode", 7, "decode", batch, 64, 8, 128, 64, "fp8u", seq_lens=lens)
    _assign_pages(wl, lens.tolist())
    return wl


@dataclass
class GdnWorkload:
    """Inputs of one GATED_DELTA_RULE decode step over a slot-indexed state pool
    ("How serving works in Tlaloc", "Linear-attention layers: the state pools").
    Row b holds slot ``slots[b]`` (-1 = pad) at position ``positions[b]`` (0 = fresh
    row, starts from zero state).  q and k are N(0, 1/128) (norm about 1), v N(0, 1),
    g (log decay) U(-1, -0.01), beta U(0.05, 0.95); the pool starts N(0, 0.1^2)."""

    name: str
    cfg_id: int
    batch: int
    num_heads: int
    num_slots: int
    head_dim: int = 128
    seed: int = SEED

    def _rng(self, tensor_id: int) -> np.random.Generator:
        return np.random.default_rng([self.seed, self.cfg_id, tensor_id, 0])

    def slots_positions(self) -> tuple[np.ndarray, np.ndarray]:
        rng = self._rng(T_PERM)
        slots = rng.permutation(self.num_slots)[:self.batch].astype(np.int32)
        positions = rng.integers(1, 32768, size=self.batch).astype(np.int32)
        positions[::9] = 0                     # fresh rows: zero state whatever the slot holds
        if self.batch > 3:
            slots[3] = -1                      # a pad row
        return slots, positions

    def step_inputs(self, step: int = 0):
        """q, k, v [B, H, D], g, beta [B, H] (f32) of decode step `step`."""
        rng = np.random.default_rng([self.seed, self.cfg_id, T_Q, step])
        shp = (self.batch, self.num_heads, self.head_dim)
        sd = np.float32(1.0 / math.sqrt(self.head_dim))
        q = (rng.standard_normal(shp, dtype=np.float32) * sd).astype(np.float32)
        k = (rng.standard_normal(shp, dtype=np.float32) * sd).astype(np.float32)
        v = rng.standard_normal(shp, dtype=np.float32)
        g = rng.uniform(-1.0, -0.01, (self.batch, self.num_heads)).astype(np.float32)
        beta = rng.uniform(0.05, 0.95, (self.batch, self.num_heads)).astype(np.float32)
        return q, k, v, g, beta

    def initial_pool(self) -> np.ndarray:
        shp = (self.num_slots, self.num_heads, self.head_dim, self.head_dim)
        return (self._rng(T_K).standard_normal(shp, dtype=np.float32) * np.float32(0.1)).astype(np.float32)


def gdn_decode_layer(batch: int = 128, heads: int = 16, slots: int = 160) -> GdnWorkload:
    """A Gated DeltaNet decode layer: 128 sequences, 16 heads of 128 x 128 f32 state,
    a pool of 160 slots (128 KiB read and written per sequence and head)."""
    return GdnWorkload("c6_gated_delta_rule_decode", 9, batch, heads, slots)


CONFIGS = {
    "c1": tiny_decode,
    "c2": llama3_decode,
    "c3": batched_prefill,
    "c4": long_prefill,
    "c4w": lambda: long_prefill(window=4096),
    "c5": fp8_decode,
    "c2r": llama3_decode_ring,
    "c5u": fp8_unscaled_decode,
    "c2i": llama3_decode_int8,
    "c6": gdn_decode_layer,
}


def make(name: str):
    return CONFIGS[name]()


def custom_decode(cfg_id: int, seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  page_size: int, kv_dtype: str, window: int = 0, spare_pages: int = 0,
                  seed: int = SEED) -> Workload:
    """A small decode workload with explicit lengths (tests)."""
    lens = np.asarray(seq_lens, dtype=np.int32)
    wl = Workload(f"decode_{cfg_id}", cfg_id, "decode", len(lens), num_q_heads, num_kv_heads,
                  head_dim, page_size, kv_dtype, window=window, seq_lens=lens, seed=seed)
    _assign_pages(wl, [max(int(x), 1) for x in lens], spare=spare_pages)
    return wl


def custom_prefill(cfg_id: int, row_lens, start_pos, tokens_per_row: int, num_q_heads: int,
                   num_kv_heads: int, head_dim: int, page_size: int, kv_dtype: str,
                   window: int = 0, spare_pages: int = 0, seed: int = SEED) -> Workload:
    """A small prefill workload with explicit row lengths and start positions (tests)."""
    rl = np.asarray(row_lens, dtype=np.int32)
    sp = np.asarray(start_pos, dtype=np.int32)
    wl = Workload(f"prefill_{cfg_id}", cfg_id, "prefill", len(rl), num_q_heads, num_kv_heads,
                  head_dim, page_size, kv_dtype, window=window, tokens_per_row=tokens_per_row,
                  row_lens=rl, start_pos=sp, seed=seed)
    _assign_pages(wl, [max(int(a + b), 1) for a, b in zip(sp, rl)], spare=spare_pages)
    return wl
