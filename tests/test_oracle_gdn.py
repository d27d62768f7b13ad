"""Pins of the Gated DeltaNet decode oracle against things other than itself.

- the delta rule's defining property: with beta = 1 and a unit-norm key, the updated
  state maps that key exactly to v (k^T S' = v), whatever S was;
- closed forms: beta = 0 and g = 0 leave S unchanged and give o = q^T S; a zero
  state gives S' = beta k v^T and o = beta (q . k) v; g scales the old state by e^g;
- element-wise brute force: plain Python loops over i and j;
- the pool: a row at position 0 ignores what its slot holds; slot -1 touches nothing
  and gives a zero row; two rows on different slots do not interact.
"""
import math

import numpy as np
import pytest

from oracle.gdn import gated_delta_step, gdn_decode

DK = DV = 16


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_delta_rule_writes_v_at_a_unit_key():
    S = rnd(1, DK, DV)
    k = rnd(2, DK)
    k /= np.linalg.norm(k)
    v = rnd(3, DV)
    S1, _ = gated_delta_step(S, rnd(4, DK), k, v, g=-0.3, beta=1.0)
    assert np.allclose(k @ S1, v, rtol=0, atol=1e-12)


def test_closed_forms():
    S, q, k, v = rnd(5, DK, DV), rnd(6, DK), rnd(7, DK), rnd(8, DV)
    S1, o = gated_delta_step(S, q, k, v, g=0.0, beta=0.0)
    assert np.array_equal(S1, S) and np.allclose(o, q @ S, atol=1e-12)
    S2, o2 = gated_delta_step(np.zeros((DK, DV)), q, k, v, g=-1.0, beta=0.25)
    assert np.allclose(S2, 0.25 * np.outer(k, v), atol=1e-14)
    assert np.allclose(o2, 0.25 * (q @ k) * v, atol=1e-12)
    S3, _ = gated_delta_step(S, q, np.zeros(DK), v, g=-0.7, beta=0.5)  # k = 0: decay only
    assert np.allclose(S3, S * math.exp(-0.7), atol=1e-14)


def test_matches_plain_python_loops():
    S, q, k, v = rnd(9, DK, DV), rnd(10, DK), rnd(11, DK), rnd(12, DV)
    g, beta = -0.2, 0.6
    d = math.exp(g)
    Sd = [[S[i][j] * d for j in range(DV)] for i in range(DK)]
    u = [math.fsum(k[i] * Sd[i][j] for i in range(DK)) for j in range(DV)]
    Sn = [[Sd[i][j] + k[i] * beta * (v[j] - u[j]) for j in range(DV)] for i in range(DK)]
    o = [math.fsum(q[i] * Sn[i][j] for i in range(DK)) for j in range(DV)]
    S1, o1 = gated_delta_step(S, q, k, v, g, beta)
    assert np.allclose(S1, np.array(Sn), atol=1e-12) and np.allclose(o1, np.array(o), atol=1e-12)


def test_pool_slots_positions_and_pads():
    H, slots_n = 2, 4
    pool = rnd(13, slots_n, H, DK, DV).astype(np.float32)
    before = pool.copy()
    B = 3
    q, k, v = rnd(14, B, H, DK), rnd(15, B, H, DK), rnd(16, B, H, DV)
    g, beta = -np.abs(rnd(17, B, H)), 1 / (1 + np.exp(-rnd(18, B, H)))
    slots = np.array([2, -1, 0])
    pos = np.array([0, 5, 7])  # row 0 starts from zero state whatever slot 2 holds
    out = gdn_decode(pool, q, k, v, g, beta, slots, pos)
    assert np.all(out[1] == 0)
    assert np.array_equal(pool[1], before[1]) and np.array_equal(pool[3], before[3])
    for h in range(H):
        S, o = gated_delta_step(np.zeros((DK, DV)), q[0, h], k[0, h], v[0, h], g[0, h], beta[0, h])
        assert np.array_equal(pool[2, h], S.astype(np.float32)) and np.array_equal(out[0, h], o.astype(np.float32))
        S, o = gated_delta_step(before[0, h], q[2, h], k[2, h], v[2, h], g[2, h], beta[2, h])
        assert np.array_equal(pool[0, h], S.astype(np.float32))
    with pytest.raises(ValueError):
        gdn_decode(pool, q, k, v, g, beta, np.array([9, 0, 1]), pos)
