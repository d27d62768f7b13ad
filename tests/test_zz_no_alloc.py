"""tl_paged_attn_decode_static, the decode entry point that allocates nothing (its
workspace is the library's static per-device scratch), against tl_paged_attn_decode
with a caller workspace: the same kernels, so the same bits.  Two calls in a row,
the second with a smaller input, on both decode kernels (the register-tile kernel
with its merge kernel, and the exact-split kernel that merges in place through the
arrival counters of the workspace header); and a call that needs more than the
static scratch is refused before anything is enqueued."""
import numpy as np
import pytest

from paged_kv_attention_cache_amd import workloads as W
from paged_kv_attention_cache_amd import runner as R
from tests.test_gpu_parity import torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu


def _both(tl, torch, wl, gp, window):
    st = R.DecodeStep(wl, gp)
    st.write()
    ref = tl.tl_paged_attn_decode(gp, st.q, st.tables, st.seq_lens, window, wl.scale)
    out = torch.full_like(st.q, float("nan"))
    got = tl.tl_paged_attn_decode_static(gp, st.q, st.tables, st.seq_lens, window, wl.scale, out=out)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("kv_dtype,hq,hkv,S", [("bf16", 32, 8, 16), ("fp8", 64, 8, 64)])
def test_static_decode_equals_the_workspace_entry(torch_cuda, kv_dtype, hq, hkv, S):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    rng = np.random.default_rng([71, hq])
    big = rng.integers(600, 9000, size=40)
    small = rng.integers(1, 2500, size=7)
    small[2] = 0
    for i, (lens, win) in enumerate([(big, 0), (small, 700)]):  # second call smaller, with a window
        wl = W.custom_decode(700 + 10 * hq + i, lens, hq, hkv, 128, S, kv_dtype)
        gp = R.make_pool(wl)
        R.write_history(gp, wl)
        got, ref = _both(tl, torch, wl, gp, win)
        assert torch.equal(got, ref), f"call {i}: static scratch result differs from the workspace entry"
        assert torch.all(torch.isfinite(got))


def test_static_decode_refuses_a_call_beyond_its_scratch(torch_cuda):
    torch = torch_cuda
    import paged_kv_attention_cache_amd as tl
    B, Hq, D, S = 1024, 64, 128, 16
    gp = tl.KVPool.allocate(4, S, 8, D, "bf16", fill_byte=0)
    q = torch.zeros((B, Hq, D), device="cuda")
    tables = torch.zeros((B, 4096), dtype=torch.int32, device="cuda")  # 64K keys: 128 splits of 512
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 3.0)
    need = tl.tl_paged_attn_decode_workspace_size(gp, B, Hq, 4096)
    assert need > 64 << 20
    with pytest.raises(tl.TLError) as e:
        tl.tl_paged_attn_decode_static(gp, q, tables, lens, out=out)
    assert e.value.code == tl.TL_ERR_WORKSPACE and "static scratch" in e.value.message
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
