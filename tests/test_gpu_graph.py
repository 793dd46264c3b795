"""qkv_prep_run, qkv_prep_gather and qkv_prep_mxfp8_norm_quant allocate
nothing and issue no memset, so a caller may capture them in a HIP graph.
Each replay is checked against the eager result, with the program's own eager
work and synchronizations between replays."""
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


def _capture(fn):
    """A warm-up call on a side stream, then the capture of one call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gather_graph_replays_match_eager(dtype):
    # qkv_prep_gather allocates nothing either.
    w = W.custom(300, 8, seed=810, num_skip=5)
    inp = W.make_inputs(w, device=DEV)
    op = qp.QkvPrep(8, block_size=w.block_size, eps=w.eps)
    op(inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"], inp["slot_mapping"],
       inp["cache"])
    slots = inp["slot_mapping"].flip(0).contiguous()
    want = torch.empty((slots.numel(), 512), dtype=dtype, device=DEV)
    op.gather(inp["cache"], slots, want)
    out = torch.empty_like(want)
    g = _capture(lambda: op.gather(inp["cache"], slots, out))
    for k in range(4):
        out.fill_(float(k + 1))                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), want.view(torch.uint8))


def test_mxfp8_graph_replays_match_eager():
    # qkv_prep_mxfp8_norm_quant allocates nothing either; the outputs are
    # passed in.
    m, hidden = 300, 2048
    gen = torch.Generator(device=DEV).manual_seed(820)
    x = torch.randn((m, hidden), generator=gen, device=DEV).to(torch.bfloat16)
    r = torch.randn((m, hidden), generator=gen, device=DEV).to(torch.bfloat16)
    gamma = (0.1 * torch.randn(hidden, generator=gen, device=DEV)).to(torch.bfloat16)
    nsc = qp.qkv_prep_mxfp8_scale_bytes(m, hidden)
    res_e = torch.empty_like(x)
    codes_e, scales_e = qp.mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=res_e)
    codes = torch.empty((m, hidden), dtype=torch.uint8, device=DEV)
    scales = torch.empty(nsc, dtype=torch.uint8, device=DEV)
    res = torch.empty_like(x)
    g = _capture(lambda: qp.mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=res,
                                             quant_out=codes, scale_out=scales))
    for k in range(4):
        codes.fill_(k + 1)
        scales.fill_(0xEE)
        res.fill_(float(k))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, codes_e) and torch.equal(scales, scales_e)
        assert torch.equal(res.view(torch.int16), res_e.view(torch.int16))
