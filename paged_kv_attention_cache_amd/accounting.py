"""Byte and flop accounting for the paged KV path (host logic, no device work).

The formulas follow the pages:
- "Serving Models", "Count KV heads and distinct stored tensors": KV bytes per
  stored token = 2 * layers * H_kv * d_head * bytes-per-element (K and V);
  "The 1 GiB example" gives Llama-3-8B in bf16 as 128 KiB a token.
- "How serving works in Tlaloc", section 3 (windowed KV pool): bytes per page
  per layer, full-history vs ring pages, the ring sizes ceil(W/S) + 1 and
  ceil((W - 1 + N) / S), and the per-call token limit of a ring.
- same page, section 2: gathering pages once per token instead of once per
  sequence costs tokens x context keys and values per layer.
The algorithmic counts of one launch (what the bench divides by time) count
each byte the method must move once: stored K/V of the visible history,
fp8 scales, queries, outputs, block-table entries and lengths.
"""
from __future__ import annotations

import math

import numpy as np

BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "fp8u": 1, "int8": 1}  # fp8u: the unscaled fp8 pool
SCALED = ("fp8", "int8")  # one f32 scale per (token, kv head) for K and for V


# ----------------------------------------------------- page-level formulas
def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: float) -> float:
    return 2 * layers * kv_heads * head_dim * elem_bytes


def page_bytes(page_size: int, kv_heads: int, head_dim: int, elem_bytes: float) -> float:
    """K plus V bytes of one page of one layer."""
    return 2 * page_size * kv_heads * head_dim * elem_bytes


def pages_for(positions: int, page_size: int) -> int:
    return (positions + page_size - 1) // page_size


def full_history_bytes(positions: int, layers: int, page_size: int, kv_heads: int,
                       head_dim: int, elem_bytes: float) -> float:
    return pages_for(positions, page_size) * page_bytes(page_size, kv_heads, head_dim, elem_bytes) * layers


def ring_pages_default(window: int, page_size: int) -> int:
    """Pages of a ring that holds one window plus the spare page."""
    return pages_for(window, page_size) + 1


def ring_pages_for_chunk(window: int, chunk: int, page_size: int) -> int:
    """Pages a ring needs so that a call of ``chunk`` tokens fits past the window."""
    return pages_for(window - 1 + chunk, page_size)


def ring_call_limit(ring_pages: int, page_size: int, p0: int, window: int) -> int:
    """Most tokens one call starting at position p0 may write through a ring."""
    return ring_pages * page_size - min(p0, window - 1)


def windowed_bytes(positions: int, full_layers: int, window_layers: int, ring_pages: int,
                   page_size: int, kv_heads: int, head_dim: int, elem_bytes: float) -> float:
    """Full-history pages for the full layers plus at most a ring for the windowed ones."""
    pb = page_bytes(page_size, kv_heads, head_dim, elem_bytes)
    return (pages_for(positions, page_size) * full_layers
            + min(pages_for(positions, page_size), ring_pages) * window_layers) * pb


def per_token_gather_bytes(tokens: int, context: int, kv_heads: int, head_dim: int,
                           elem_bytes: float) -> float:
    """Per-layer bytes of gathering a context's K and V once for every token."""
    return tokens * context * 2 * kv_heads * head_dim * elem_bytes


def score_tensor_bytes(kv_heads: int, rows: int, keys: int, elem_bytes: int = 4) -> int:
    return kv_heads * rows * keys * elem_bytes


# ------------------------------------------------ per-launch algorithmic work
def visible_counts(positions: np.ndarray, window: int) -> np.ndarray:
    """Number of keys each query position sees (0 for pads)."""
    p = np.asarray(positions, dtype=np.int64)
    n = p + 1
    if window > 0:
        n = np.minimum(n, window)
    return np.where(p < 0, 0, n)


def decode_bytes(seq_lens, num_q_heads: int, kv_heads: int, head_dim: int, page_size: int,
                 kv_dtype: str, window: int = 0) -> int:
    """Bytes one decode launch must move: visible K/V (+ scales), Q, out, tables, lengths."""
    L = np.asarray(seq_lens, dtype=np.int64)
    vis = visible_counts(L - 1, window)
    kv = int(vis.sum()) * kv_heads * head_dim * 2 * BYTES[kv_dtype]
    if kv_dtype in SCALED:
        kv += int(vis.sum()) * kv_heads * 2 * 4
    B = len(L)
    qo = 2 * B * num_q_heads * head_dim * 4
    tables = int(sum(pages_for(int(x), page_size) for x in L)) * 4
    return kv + qo + tables + B * 4


def write_bytes(slots, kv_heads: int, head_dim: int, kv_dtype: str) -> int:
    """Bytes one write launch must move: live rows read in f32 and stored, scales, slots."""
    s = np.asarray(slots)
    live = int(np.count_nonzero(s != -1))
    b = live * kv_heads * head_dim * 2 * (4 + BYTES[kv_dtype])
    if kv_dtype in SCALED:
        b += live * kv_heads * 2 * 4
    return b + 4 * s.size


def prefill_flops(positions: np.ndarray, num_q_heads: int, head_dim: int, window: int = 0) -> int:
    """4 * D * H_q flop per visible (token, key) pair: 2D for q.k and 2D for p.v."""
    return int(visible_counts(positions, window).sum()) * 4 * head_dim * num_q_heads


def decode_flops(seq_lens, num_q_heads: int, head_dim: int, window: int = 0) -> int:
    L = np.asarray(seq_lens, dtype=np.int64)
    return int(visible_counts(L - 1, window).sum()) * 4 * head_dim * num_q_heads


def mib(x: float) -> float:
    return x / 2 ** 20


def gib(x: float) -> float:
    return x / 2 ** 30


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("math", "np", "annotations")]
