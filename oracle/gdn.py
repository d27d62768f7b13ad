"""CPU oracle of the Gated DeltaNet decode recurrence over a slot-indexed state pool.

TEST INFRASTRUCTURE ONLY.  Plain numpy in f64; nothing in the product path imports
it, and it shares no code with the HIP kernel.

What it follows (page "How serving works in Tlaloc", "Linear-attention layers: the
state pools"): a Gated DeltaNet layer keeps, per sequence, an f32 recurrent state of
[heads, 128, 128] in a pool indexed by the sequence's state slot; the
GATED_DELTA_RULE op runs, per token and head,
    S = S * exp(g);   S += k (outer) beta * (v - k^T S);   o = q^T S,
and returns its output and the updated pool; a decode step runs it once.  A row
whose first token is at position 0 starts from zero state, so a reused slot needs no
clearing.

Readings where the page is silent (listed in the design notes):
- S[i][j]: i runs over the key dimension, j over the value dimension, so k^T S and
  q^T S are vectors over j and the outer product is (k (outer) x)[i][j] = k_i x_j;
- o uses the state after this token's update;
- g (a log decay) and beta are one scalar per (token, head); q, k, v are used as
  given (any normalisation belongs to the layer before the op);
- a state slot of -1 is a pad: no state is read or written and the output row is 0.
"""
from __future__ import annotations

import numpy as np


def gated_delta_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, g: float,
                     beta: float) -> tuple[np.ndarray, np.ndarray]:
    """One token of one head: returns (new S [dk, dv], o [dv]) in f64."""
    S = np.asarray(S, dtype=np.float64) * np.exp(np.float64(g))
    k = np.asarray(k, dtype=np.float64)
    u = k @ S                                   # k^T S, over the value dimension
    S = S + np.outer(k, np.float64(beta) * (np.asarray(v, dtype=np.float64) - u))
    o = np.asarray(q, dtype=np.float64) @ S     # q^T S with the updated state
    return S, o


def gdn_decode(pool: np.ndarray, q, k, v, g, beta, slots, positions) -> np.ndarray:
    """A decode step over a batch: pool [num_slots, H, dk, dv] f32 is updated in place
    (rounded to f32 once per step); q, k [B, H, dk], v [B, H, dv], g, beta [B, H],
    slots, positions [B].  Returns o [B, H, dv] f32."""
    B, H = np.shape(g)
    dv = pool.shape[3]
    out = np.zeros((B, H, dv), dtype=np.float32)
    for b in range(B):
        s = int(slots[b])
        if s == -1:
            continue
        if s < 0 or s >= pool.shape[0]:
            raise ValueError(f"gdn_decode: state slot {s} of row {b} is outside the pool")
        for h in range(H):
            S0 = np.zeros(pool.shape[2:], np.float64) if int(positions[b]) == 0 else pool[s, h].astype(np.float64)
            S1, o = gated_delta_step(S0, q[b, h], k[b, h], v[b, h], float(g[b, h]), float(beta[b, h]))
            pool[s, h] = S1.astype(np.float32)
            out[b, h] = o.astype(np.float32)
    return out
