"""The in-place merge of decode splits, repeated.

On the exact-split decode kernels (bf16 and int8 at G = 4, fp8 at G = 8) the
workgroup that stores a (sequence, head group)'s last split merges all of its splits,
reading the other workgroups' partial states after an arrival counter says they are
all stored.  Its correctness rests on ordering (coherent stores, a wait for their
completion before the count, loads issued only after the count has returned), so a
rare ordering failure would show as a call whose output differs from the others.  Each
workload below is decoded 200 times back to back on one workspace, and every output
must equal the first one bit for bit (the first one is checked against the oracle
elsewhere); the loop stops at the first mismatch.
"""
import numpy as np
import pytest

from paged_kv_attention_cache_amd import workloads as W
from paged_kv_attention_cache_amd import runner as R
from tests.test_gpu_parity import torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu

CALLS = 200


def _repeat(torch, st):
    first = st.attend().clone()
    torch.cuda.synchronize()
    outs = [torch.empty_like(first) for _ in range(8)]
    for i in range(CALLS):
        o = outs[i % len(outs)]
        st.out = o
        st.attend()
        if i % len(outs) == len(outs) - 1 or i == CALLS - 1:
            torch.cuda.synchronize()
            for j, x in enumerate(outs[:(i % len(outs)) + 1]):
                assert torch.equal(x, first), f"call {i - (i % len(outs)) + j} differs from the first"
    return first


@pytest.mark.parametrize("cfg", ["c2", "c5", "c2i"])
def test_in_place_merge_gives_the_same_bits_on_every_call(torch_cuda, cfg):
    torch = torch_cuda
    wl = W.make(cfg)
    gp = R.make_pool(wl, fill_byte=None)
    R.write_history(gp, wl)
    st = R.DecodeStep(wl, gp)
    st.write()
    first = _repeat(torch, st)
    assert torch.all(torch.isfinite(first))


def test_in_place_merge_at_64_head_groups_repeats(torch_cuda):
    """64 KV heads at G = 8: the most head groups the arrival counters cover."""
    torch = torch_cuda
    wl = W.custom_decode(950, [5000, 9000, 100, 4097], 512, 64, 128, 16, "fp8")
    gp = R.make_pool(wl)
    R.write_history(gp, wl)
    st = R.DecodeStep(wl, gp)
    st.write()
    _repeat(torch, st)
    assert np.all(np.isfinite(st.out.cpu().numpy()))
