"""The int8 decode tile on the integer matrix cores (G = 4, D = 128, pages of >= 16).

It writes the scaled queries, and a head's probabilities times the V scales, as a power
of two and four 7-bit integer limbs, so both products are exact integer sums.  These
tests hold it to the oracle at the f32 bound on inputs whose magnitudes vary widely:
- V rows spanning 2^-20 .. 2^20, so a tile's p * v_scale spans many binades;
- K rows spanning 2^-3 .. 2^3;
- query heads spanning 2^-12 .. 2^2, and one all-zero head.
They also check that a sequence's output does not depend on the batch around it.
"""
import numpy as np
import pytest

import oracle
from paged_kv_attention_cache_amd import workloads as W
from paged_kv_attention_cache_amd import runner as R
from tests.helpers import row_rel_err
from tests.test_gpu_parity import assert_pool_equal, torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu


def _wide_pools(torch, wl, rng):
    import paged_kv_attention_cache_amd as tl
    op = oracle.KVPool(wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, sentinel=R.SENTINEL)
    gp = R.make_pool(wl)
    for k, v, s in list(wl.history_batches()) + [wl.decode_step_rows()]:
        n = len(s)
        fk = np.exp2(rng.uniform(-3, 3, size=(n, wl.num_kv_heads, 1))).astype(np.float32)
        fv = np.exp2(rng.uniform(-20, 20, size=(n, wl.num_kv_heads, 1))).astype(np.float32)
        k2 = (k * fk).astype(np.float32)
        v2 = (v * fv).astype(np.float32)
        op.write(k2, v2, s)
        tl.tl_kv_cache_write(gp, torch.from_numpy(k2).cuda(), torch.from_numpy(v2).cuda(),
                             torch.from_numpy(np.ascontiguousarray(s)).cuda())
    return gp, op


@pytest.mark.parametrize("S", [16, 64])
def test_int8_tile_wide_magnitudes(torch_cuda, S):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    lens = [5000, 1025, 64, 3, 2100]
    wl = W.custom_decode(950 + S, lens, 8, 2, 128, S, "int8", spare_pages=3)
    rng = np.random.default_rng(951 + S)
    gp, op = _wide_pools(torch, wl, rng)
    torch.cuda.synchronize()
    assert_pool_equal(gp, op)
    q = wl.decode_q() * np.exp2(rng.uniform(-12, 2, size=(len(lens), wl.num_q_heads, 1))).astype(np.float32)
    q[1, 5, :] = 0.0  # a head with no query at all: uniform attention
    q = q.astype(np.float32)
    st = R.DecodeStep(wl, gp)
    out = tl.tl_paged_attn_decode(gp, torch.from_numpy(q).cuda(), st.tables, st.seq_lens, 0, wl.scale,
                                  workspace=st.workspace)
    got = out.cpu().numpy()
    ref = oracle.decode(op, q, wl.block_tables, wl.seq_lens, 0, wl.scale)
    err = row_rel_err(got, ref)
    assert err <= 2e-5, f"max row error {err:.3e}"


def test_int8_tile_batch_invariance_bitwise(torch_cuda):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    wl = W.custom_decode(960, [1500, 77, 3000, 515, 1024, 4097], 8, 2, 128, 16, "int8")
    gp = R.make_pool(wl)
    R.write_history(gp, wl)
    st = R.DecodeStep(wl, gp)
    full = st.run().clone()
    for b in range(wl.batch):
        one = tl.tl_paged_attn_decode(gp, st.q[b:b + 1].contiguous(), st.tables[b:b + 1].contiguous(),
                                      st.seq_lens[b:b + 1].contiguous(), 0, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[b]), f"sequence {b} differs alone vs in batch"
