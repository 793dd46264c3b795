"""Prepared launches (QkvPrep.prepare, QkvPrep.prepare_gather,
prepare_mxfp8_norm_quant): the checks and the argument struct are done once,
and each call is one C call.  Every prepared launch must write exactly what
the direct call writes, on the stream it was prepared for, and must refuse to
run once its handle is destroyed."""
import pytest
import torch

from fp8_kv_cache_amd import qkv_prep as qp
from fp8_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _op_case(T, H, seed, kv_store=qp.KV_FP8):
    w = W.custom(T, H, seed=seed)
    inp = W.make_inputs(w, device=DEV)
    slot_bytes = qp.SLOT_BYTES if kv_store == qp.KV_FP8 else qp.BF16_SLOT_BYTES
    gen = torch.Generator(device=DEV).manual_seed(seed)
    cache = torch.randint(0, 256, (w.num_blocks, w.block_size * slot_bytes), dtype=torch.uint8,
                          device=DEV, generator=gen)
    rest = (inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"], inp["cos_sin"], inp["slot_mapping"])
    return w, inp["q"], rest, cache


@pytest.mark.parametrize("T,H,kv_store", [(1, 64, qp.KV_FP8), (16, 8, qp.KV_FP8),
                                          (333, 64, qp.KV_FP8), (2048, 64, qp.KV_FP8),
                                          (65, 16, qp.KV_BF16)])
def test_prepared_op_matches_direct_calls(T, H, kv_store):
    """Three launches in a row (q drifts in place, so each launch sees the
    previous one's output) give the same bytes through both routes."""
    print("prepared op T=%d H=%d kv_store=%d" % (T, H, kv_store), flush=True)
    w, q0, rest, cache0 = _op_case(T, H, 900 + T, kv_store)
    op = qp.QkvPrep(H, block_size=w.block_size, eps=w.eps, kv_store=kv_store)
    q_d, c_d = q0.clone(), cache0.clone()
    q_p, c_p = q0.clone(), cache0.clone()
    launch = op.prepare(q_p, *rest, c_p)
    for _ in range(3):
        op(q_d, *rest, c_d)
        launch()
    torch.cuda.synchronize()
    assert torch.equal(q_p.view(torch.int16), q_d.view(torch.int16))
    assert torch.equal(c_p, c_d)


def test_prepared_op_runs_on_its_stream():
    """A launch prepared for a side stream is ordered on that stream: work
    queued on the side stream before it is seen, and the main stream waits
    for it only through an explicit dependency."""
    print("prepared op on a side stream", flush=True)
    w, q0, rest, cache0 = _op_case(256, 64, 950)
    op = qp.QkvPrep(64, block_size=w.block_size, eps=w.eps)
    q_d, c_d = q0.clone(), cache0.clone()
    op(q_d, *rest, c_d)
    q_p = torch.zeros_like(q0)
    c_p = torch.zeros_like(cache0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    launch = op.prepare(q_p, *rest, c_p, stream=side.cuda_stream)
    with torch.cuda.stream(side):
        q_p.copy_(q0)
        c_p.copy_(cache0)
    launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(q_p.view(torch.int16), q_d.view(torch.int16))
    assert torch.equal(c_p, c_d)


def test_prepared_op_checks_at_prepare_time_and_refuses_after_close():
    w, q0, rest, cache0 = _op_case(64, 64, 960)
    op = qp.QkvPrep(64, block_size=w.block_size, eps=w.eps)
    with pytest.raises(ValueError):
        op.prepare(q0[:, :32], *rest, cache0)
    with pytest.raises(TypeError):
        op.prepare(q0.float(), *rest, cache0)
    q = q0.clone()
    cache = cache0.clone()
    launch = op.prepare(q, *rest, cache)
    op.close()
    with pytest.raises(qp.QkvPrepError) as e:
        launch()
    assert e.value.code == qp.ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), q0.view(torch.int16))     # nothing was launched
    assert torch.equal(cache, cache0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prepared_gather_matches_direct_call(dtype):
    print("prepared gather %s" % dtype, flush=True)
    nb, bs = 40, 64
    gen = torch.Generator(device=DEV).manual_seed(970)
    cache = torch.randint(0, 256, (nb, bs * qp.SLOT_BYTES), dtype=torch.uint8, device=DEV, generator=gen)
    cache[:, bs * 576:].random_(0, 256, generator=gen)
    slots = torch.randint(-3, nb * bs + 3, (1000,), dtype=torch.int64, device=DEV, generator=gen)
    op = qp.QkvPrep(64, block_size=bs)
    out_d = torch.full((slots.numel(), 512), 7.0, dtype=dtype, device=DEV)
    out_p = out_d.clone()
    op.gather(cache, slots, out_d)
    launch = op.prepare_gather(cache, slots, out_p)
    launch()
    torch.cuda.synchronize()
    view = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(out_p.view(view), out_d.view(view))


@pytest.mark.parametrize("m,hidden,residual", [(1, 7168, True), (300, 1024, False), (129, 4096, True)])
def test_prepared_mxfp8_matches_wrapper(m, hidden, residual):
    print("prepared mxfp8 m=%d hidden=%d residual=%d" % (m, hidden, residual), flush=True)
    gen = torch.Generator(device=DEV).manual_seed(980 + m)
    x = torch.randn((m, hidden), generator=gen, device=DEV).to(torch.bfloat16)
    gamma = (0.1 * torch.randn(hidden, generator=gen, device=DEV)).to(torch.bfloat16)
    r = torch.randn((m, hidden), generator=gen, device=DEV).to(torch.bfloat16) if residual else None
    ro_d = torch.empty_like(x) if residual else None
    ro_p = torch.empty_like(x) if residual else None
    codes_d, scales_d = qp.mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=ro_d)
    launch = qp.prepare_mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=ro_p)
    launch()
    launch()
    codes_p, scales_p = launch.outputs
    torch.cuda.synchronize()
    assert torch.equal(codes_p, codes_d)
    assert torch.equal(scales_p, scales_d)
    if residual:
        assert torch.equal(ro_p.view(torch.int16), ro_d.view(torch.int16))


def test_prepared_op_captured_in_a_graph():
    """A launch prepared inside the capture runs on the capturing stream; the
    graph (two launches) replays to the bytes of two direct calls, four times,
    with eager work and synchronizations between replays."""
    print("prepared op in a graph", flush=True)
    w, q0, rest, cache0 = _op_case(300, 16, 990)
    op = qp.QkvPrep(16, block_size=w.block_size, eps=w.eps)
    q_d, c_d = q0.clone(), cache0.clone()
    op(q_d, *rest, c_d)
    op(q_d, *rest, c_d)
    q_g, c_g = q0.clone(), cache0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        op(q_g, *rest, c_g)                      # warm-up launch outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch = op.prepare(q_g, *rest, c_g)
        launch()
        launch()
    for _ in range(4):
        q_g.copy_(q0)
        c_g.copy_(cache0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q_g.view(torch.int16), q_d.view(torch.int16))
        assert torch.equal(c_g, c_d)


def test_launch_moved_onto_the_capturing_stream():
    """A launch prepared outside a capture, moved with on_stream onto the
    capturing stream, records into the graph; replays equal the direct call."""
    print("prepared gather moved into a graph", flush=True)
    nb, bs = 24, 64
    gen = torch.Generator(device=DEV).manual_seed(995)
    cache = torch.randint(0, 256, (nb, bs * qp.SLOT_BYTES), dtype=torch.uint8, device=DEV, generator=gen)
    slots = torch.randperm(nb * bs, device=DEV, generator=gen).to(torch.int64)
    op = qp.QkvPrep(64, block_size=bs)
    want = torch.empty((slots.numel(), 512), dtype=torch.float32, device=DEV)
    op.gather(cache, slots, want)
    out = torch.empty_like(want)
    launch = op.prepare_gather(cache, slots, out)
    launch()                                   # warm-up outside the graph
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch.on_stream(torch.cuda.current_stream().cuda_stream)()
    for k in range(4):
        out.fill_(float(k))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32))
