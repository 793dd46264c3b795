"""qkv_prep_run allocates nothing and issues no memset, so a caller may capture
it in a HIP graph.  Each replay is checked against the eager result, with the
program's own eager work and synchronizations between replays."""
import pytest
import torch

from fp8_kv_cache_amd import qkv_prep as qp
from fp8_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("T,H,kv_store", [(1, 64, qp.KV_FP8), (64, 64, qp.KV_FP8),
                                          (17, 128, qp.KV_BF16)])
def test_graph_replays_match_eager(T, H, kv_store):
    w = W.custom(T, H, seed=800 + T)
    inp = W.make_inputs(w, device=DEV)
    slot_bytes = 584 if kv_store == qp.KV_FP8 else 1024
    cache0 = torch.randint(0, 256, (w.num_blocks, w.block_size * slot_bytes), dtype=torch.uint8,
                           device=DEV)
    q0 = inp["q"].clone()
    op = qp.QkvPrep(H, block_size=w.block_size, eps=w.eps, kv_store=kv_store)
    rest = (inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"],
            inp["slot_mapping"])

    q_e, c_e = q0.clone(), cache0.clone()
    op(q_e, *rest, c_e)
    torch.cuda.synchronize()

    q_g, c_g = q0.clone(), cache0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        op(q_g, *rest, c_g)                      # warm-up launch outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op(q_g, *rest, c_g)
    for _ in range(4):
        q_g.copy_(q0)
        c_g.copy_(cache0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q_g.view(torch.int16), q_e.view(torch.int16))
        assert torch.equal(c_g, c_e)
