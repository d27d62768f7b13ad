"""GPU parity of the Gated DeltaNet decode step (tl_gated_delta_rule_decode) against
the oracle of "Linear-attention layers: the state pools" ("How serving works in
Tlaloc"): outputs and the whole updated pool, per row max|x - ref| / max|ref| <= 2e-5
(f32 arithmetic against f64), over several consecutive steps; pads and slots no row
names stay bit-identical; fresh rows ignore their slot's old state."""
import numpy as np
import pytest

from oracle.gdn import gated_delta_step, gdn_decode
from paged_kv_attention_cache_amd import workloads as W
from tests.helpers import row_rel_err
from tests.test_gpu_parity import torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu


def run_steps(torch, wl, steps):
    import paged_kv_attention_cache_amd as tl
    pool = wl.initial_pool()
    opool = pool.copy()
    gpool = torch.from_numpy(pool).cuda()
    slots, pos = wl.slots_positions()
    st, pt = torch.from_numpy(slots).cuda(), torch.from_numpy(pos).cuda()
    worst_o = worst_s = 0.0
    for step in range(steps):
        q, k, v, g, beta = wl.step_inputs(step)
        dev = [torch.from_numpy(x).cuda() for x in (q, k, v, g, beta)]
        out = tl.tl_gated_delta_rule_decode(gpool, *dev, st, pt)
        torch.cuda.synchronize()
        ref = gdn_decode(opool, q, k, v, g, beta, slots, pos)
        got = out.cpu().numpy()
        worst_o = max(worst_o, row_rel_err(got.reshape(-1, wl.head_dim), ref.reshape(-1, wl.head_dim)))
        gp = gpool.cpu().numpy()
        worst_s = max(worst_s, row_rel_err(gp.reshape(-1, wl.head_dim), opool.reshape(-1, wl.head_dim)))
        assert np.all(got[slots == -1] == 0)
        pos = pos + 1  # next step: no row is fresh any more
        pt = torch.from_numpy(pos).cuda()
    return pool, gpool.cpu().numpy(), slots, worst_o, worst_s


@pytest.mark.parametrize("B,H,NS,steps", [(10, 3, 16, 3), (40, 8, 48, 2)])
def test_gdn_decode_matches_oracle_over_steps(torch_cuda, B, H, NS, steps):
    wl = W.GdnWorkload("gdn_test", 50 + B, B, H, NS)
    pool0, pool, slots, eo, es = run_steps(torch_cuda, wl, steps)
    assert eo <= 2e-5, f"output row error {eo:.3e}"
    assert es <= 2e-5, f"state row error {es:.3e}"
    untouched = np.setdiff1d(np.arange(NS), slots[slots >= 0])
    assert np.array_equal(pool[untouched], pool0[untouched])


def test_gdn_fresh_row_ignores_its_slot(torch_cuda):
    """Row 0 is at position 0: its result must not depend on what its slot held."""
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    wl = W.GdnWorkload("gdn_fresh", 60, 4, 2, 6)
    slots, pos = wl.slots_positions()
    assert pos[0] == 0
    q, k, v, g, beta = wl.step_inputs(0)
    outs = []
    for fill in (0.0, 1e3):
        pool = wl.initial_pool()
        pool[slots[0]] = fill
        gp = torch.from_numpy(pool).cuda()
        out = tl.tl_gated_delta_rule_decode(gp, *[torch.from_numpy(x).cuda() for x in (q, k, v, g, beta)],
                                            torch.from_numpy(slots).cuda(), torch.from_numpy(pos).cuda())
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy()[0], gp.cpu().numpy()[slots[0]]))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    for h in range(2):
        S, o = gated_delta_step(np.zeros((128, 128)), q[0, h], k[0, h], v[0, h], g[0, h], beta[0, h])
        assert row_rel_err(outs[0][0][h][None], o[None]) <= 2e-5


def test_gdn_full_size_sampled(torch_cuda):
    """c6 (128 rows x 16 heads, 160 slots) in one call, sampled rows against the oracle."""
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    wl = W.make("c6")
    pool = wl.initial_pool()
    slots, pos = wl.slots_positions()
    q, k, v, g, beta = wl.step_inputs(0)
    gp = torch.from_numpy(pool).cuda()
    out = tl.tl_gated_delta_rule_decode(gp, *[torch.from_numpy(x).cuda() for x in (q, k, v, g, beta)],
                                        torch.from_numpy(slots).cuda(), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    got, gpn = out.cpu().numpy(), gp.cpu().numpy()
    for b in (0, 1, 3, 9, 64, wl.batch - 1):
        for h in (0, wl.num_heads - 1):
            if slots[b] < 0:
                assert np.all(got[b] == 0)
                continue
            S0 = np.zeros((128, 128)) if pos[b] == 0 else pool[slots[b], h]
            S, o = gated_delta_step(S0, q[b, h], k[b, h], v[b, h], g[b, h], beta[b, h])
            assert row_rel_err(got[b, h][None], o[None]) <= 2e-5
            assert row_rel_err(gpn[slots[b], h], S) <= 2e-5
