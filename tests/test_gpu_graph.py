"""The decode step replayed as a captured HIP graph, the way bench.py times it.

The step (KV_CACHE_WRITE of the new rows, then the decode call) is captured once and
replayed several times, with eager calls and synchronisations between the replays;
after every replay the output and the whole pool equal the eager step's bit for bit.
Both decode kernels are covered (the register tile and the exact-split tiles: bf16 and
int8 at G = 4, fp8 at G = 8), which between them make every kind of launch a decode
call makes.
"""
import pytest

from paged_kv_attention_cache_amd import workloads as W
from paged_kv_attention_cache_amd import runner as R
from tests.test_gpu_parity import torch_cuda  # noqa: F401

pytestmark = pytest.mark.gpu

CASES = [
    ("g4_bf16_exact_split", [1, 513, 3000, 40], 8, 2, 128, 16, "bf16"),
    ("g8_fp8_exact_split", [4097, 900, 70], 16, 2, 128, 64, "fp8"),
    ("g2_bf16_register_tile", [300, 1500, 17], 4, 2, 128, 16, "bf16"),
    ("g8_int8_register_tile_merge_kernel", [2000, 33], 16, 2, 128, 16, "int8"),
    ("g4_int8_integer_tile", [2000, 33, 1100], 8, 2, 128, 16, "int8"),
]


def _pool_bytes(torch, gp):
    return [t.clone() for t in (gp.k, gp.v, gp.k_scale, gp.v_scale) if t is not None]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_the_eager_step(torch_cuda, case):
    torch = torch_cuda
    name, lens, Hq, Hkv, D, S, dt = case
    wl = W.custom_decode(900 + CASES.index(case), lens, Hq, Hkv, D, S, dt, spare_pages=3)
    gp = R.make_pool(wl)
    R.write_history(gp, wl)
    st = R.DecodeStep(wl, gp)
    st.run()
    torch.cuda.synchronize()
    ref_out = st.out.clone()
    ref_pool = _pool_bytes(torch, gp)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    for i in range(4):
        st.out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out, ref_out), f"{name}: replay {i} output differs from the eager step"
        for a, b in zip(_pool_bytes(torch, gp), ref_pool):
            assert torch.equal(a, b), f"{name}: replay {i} left different pool bytes"
        st.attend()  # eager work between replays on the same workspace
        torch.cuda.synchronize()
        assert torch.equal(st.out, ref_out), f"{name}: eager call after replay {i} differs"
