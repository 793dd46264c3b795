"""GPU check of the MXFP8 norm-quant operator (include/qkv_prep_mxfp8.h)
against the oracle: every code, every swizzled scale byte (the scale buffer is
poisoned first, so a byte written twice, missed or outside the layout shows)
and the residual output."""
import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_amd import qkv_prep as qp
from fp8_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def draw(m, hidden, seed, scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = (scale * torch.randn((m, hidden), generator=g, device=DEV)).to(torch.bfloat16)
    r = (0.5 * torch.randn((m, hidden), generator=g, device=DEV)).to(torch.bfloat16)
    gamma = (0.1 * torch.randn(hidden, generator=g, device=DEV)).to(torch.bfloat16)
    return x, r, gamma


@pytest.mark.parametrize("m,hidden,with_res,with_out", [
    (1, 512, False, False), (5, 1024, True, True), (127, 1536, True, False),
    (128, 4096, False, True), (300, 7168, True, True), (129, 8192, True, True),
    (64, 2560, False, False), (1000, 3072, True, True),
    # hidden a multiple of 128 but not of 512 (a partial last group of 16, 32
    # or 48 chunks), and past 8192 (an odd group count above 16 is launched
    # with one empty group more)
    (3, 128, True, True), (130, 384, True, False), (17, 640, False, True), (64, 1152, True, True),
    (257, 3200, True, True), (40, 8704, True, True), (33, 12288, False, True), (129, 16384, True, True),
    (5, 16256, True, True)])
def test_mxfp8_matches_the_oracle(m, hidden, with_res, with_out):
    x, r, gamma = draw(m, hidden, 900 + m + hidden)
    eps = 1e-6
    nbytes = qp.qkv_prep_mxfp8_scale_bytes(m, hidden)
    scales = torch.full((nbytes,), 0xEE, dtype=torch.uint8, device=DEV)
    codes = torch.full((m, hidden), 0xEE, dtype=torch.uint8, device=DEV)
    res_out = torch.full((m, hidden), float("nan"), dtype=torch.bfloat16, device=DEV) if with_out else None
    qp.mxfp8_norm_quant(x, gamma, eps, residual=r if with_res else None, residual_out=res_out,
                        quant_out=codes, scale_out=scales)
    torch.cuda.synchronize()
    want_codes, want_scales, want_pre = oracle.mxfp8_norm_quant(
        W.as_u16(x), W.as_u16(gamma), eps, residual=W.as_u16(r) if with_res else None)
    got_codes = codes.cpu().numpy()
    got_scales = scales.cpu().numpy()
    assert np.array_equal(got_scales, want_scales), np.count_nonzero(got_scales != want_scales)
    assert np.count_nonzero(got_codes != want_codes) == 0, int(np.count_nonzero(got_codes != want_codes))
    if with_out:
        want = want_pre if with_res else W.as_u16(x)
        assert np.array_equal(W.as_u16(res_out), want)


def test_mxfp8_at_the_measured_size():
    # The size the bench times (16384 x 7168, residual in and out), every code,
    # scale byte and residual value against the oracle.
    m, hidden = 16384, 7168
    print("case mxfp8 %dx%d residual" % (m, hidden), flush=True)
    x, r, gamma = draw(m, hidden, 990)
    scales = torch.full((qp.qkv_prep_mxfp8_scale_bytes(m, hidden),), 0xEE, dtype=torch.uint8, device=DEV)
    codes = torch.empty((m, hidden), dtype=torch.uint8, device=DEV)
    res_out = torch.empty_like(x)
    qp.mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=res_out, quant_out=codes, scale_out=scales)
    torch.cuda.synchronize()
    want_codes, want_scales, want_pre = oracle.mxfp8_norm_quant(W.as_u16(x), W.as_u16(gamma), 1e-6,
                                                                residual=W.as_u16(r))
    assert np.array_equal(scales.cpu().numpy(), want_scales)
    assert np.array_equal(codes.cpu().numpy(), want_codes)
    assert np.array_equal(W.as_u16(res_out), want_pre)


def test_mxfp8_outlier_rows_and_zero_rows():
    m, hidden = 256, 2048
    x, r, gamma = draw(m, hidden, 950, scale=1.0)
    x[3] *= 1000.0
    x[7] = 0.0
    eps = 1e-5
    codes, scales = qp.mxfp8_norm_quant(x, gamma, eps)
    torch.cuda.synchronize()
    wc, ws, _ = oracle.mxfp8_norm_quant(W.as_u16(x), W.as_u16(gamma), eps)
    assert np.array_equal(codes.cpu().numpy(), wc)
    assert np.array_equal(scales.cpu().numpy(), ws)


def test_mxfp8_empty_is_a_no_op():
    x = torch.zeros((0, 512), dtype=torch.bfloat16, device=DEV)
    gamma = torch.zeros(512, dtype=torch.bfloat16, device=DEV)
    codes, scales = qp.mxfp8_norm_quant(x, gamma, 1e-6)
    assert codes.numel() == 0 and scales.numel() == 0


@pytest.mark.parametrize("eps,with_res", [(1e-6, False), (1e-6, True), (1e-30, True)])
def test_mxfp8_subnormal_inputs(eps, with_res):
    # bf16 subnormal x (and residual): the squares underflow, the normalized
    # values are tiny, and the scale bytes sit at the bottom of the range
    # (2 and 3 at eps = 1e-6, so the inverse scale is 2^125).
    m, hidden = 130, 1024
    g = torch.Generator().manual_seed(960)
    def subnormal_bits():
        b = torch.randint(0, 128, (m, hidden), generator=g, dtype=torch.int32)
        b |= torch.randint(0, 2, (m, hidden), generator=g, dtype=torch.int32) << 15
        return b.to(torch.int16).view(torch.bfloat16).to(DEV)
    x = subnormal_bits()
    r = subnormal_bits() if with_res else None
    gamma = (0.1 * torch.randn(hidden, generator=g)).to(torch.bfloat16).to(DEV)
    res_out = torch.empty_like(x) if with_res else None
    codes, scales = qp.mxfp8_norm_quant(x, gamma, eps, residual=r, residual_out=res_out)
    torch.cuda.synchronize()
    wc, ws, wp = oracle.mxfp8_norm_quant(W.as_u16(x), W.as_u16(gamma), eps,
                                         residual=W.as_u16(r) if with_res else None)
    assert np.array_equal(scales.cpu().numpy(), ws)
    assert np.array_equal(codes.cpu().numpy(), wc)
    if with_res:
        assert np.array_equal(W.as_u16(res_out), wp)
    if eps == 1e-6:
        assert set(np.unique(ws).tolist()) <= {0, 1, 2, 3, 4}       # the bottom of the scale range


def test_mxfp8_partial_group_decides_the_sum_order():
    # hidden 640: one full group of 64 chunks and a partial one of 16.  Large
    # values in the partial group and tiny ones elsewhere make the sum depend
    # on where the partial group's sum joins the tree, so a kernel that added
    # it anywhere else than the oracle's odd-carry position would differ.
    m, hidden = 64, 640
    x, r, gamma = draw(m, hidden, 970)
    x[:, 512:] *= 4096.0
    x[:, :8] = 1.0
    codes, scales = qp.mxfp8_norm_quant(x, gamma, 1e-6)
    torch.cuda.synchronize()
    wc, ws, _ = oracle.mxfp8_norm_quant(W.as_u16(x), W.as_u16(gamma), 1e-6)
    assert np.array_equal(codes.cpu().numpy(), wc)
    assert np.array_equal(scales.cpu().numpy(), ws)


def _reading_cases():
    """The CPU pins' rows that decide a reading (tests/test_oracle_mxfp8.py):
    eps inside the root, the norm reading the bf16 residual sum (two seeds),
    the Gemma weight applied after inv.  Returns (name, x, residual, gamma,
    eps) with bf16 bit patterns."""
    from fractions import Fraction
    import test_oracle_mxfp8 as T
    import mx_exact as X
    cases = [("eps inside the root", T._bits([2] * 128), None, T._bits([0] * 128), 5.0)]
    for seed in (12, 40):
        x, r, g = T._residual_case(seed)
        cases.append(("bf16 residual sum, seed %d" % seed, T._bits(x), T._bits(r), T._bits(g), 0.0))
    rng = np.random.default_rng(0)
    g = [X.bf16(Fraction(int(v), 512)) for v in rng.integers(-200, 201, 128)]
    cases.append(("weight after inv", T._bits([7] * 128), None, T._bits(g), 0.0))
    return cases


def test_mxfp8_rows_that_decide_a_reading():
    # The kernel takes the same side of each reading as the oracle, on the rows
    # where the alternatives give other codes.
    for name, x, r, g, eps in _reading_cases():
        print("case mxfp8 reading: %s" % name, flush=True)
        hidden = x.size
        xt = torch.from_numpy(x.view(np.int16).reshape(1, hidden)).view(torch.bfloat16).to(DEV)
        gt = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).to(DEV)
        rt = None if r is None else torch.from_numpy(r.view(np.int16).reshape(1, hidden)).view(torch.bfloat16).to(DEV)
        scales = torch.full((qp.qkv_prep_mxfp8_scale_bytes(1, hidden),), 0xEE, dtype=torch.uint8, device=DEV)
        codes = torch.full((1, hidden), 0xEE, dtype=torch.uint8, device=DEV)
        qp.mxfp8_norm_quant(xt, gt, eps, residual=rt, quant_out=codes, scale_out=scales)
        torch.cuda.synchronize()
        want_codes, want_scales, _ = oracle.mxfp8_norm_quant(x.reshape(1, hidden), g, eps,
                                                            residual=None if r is None else r.reshape(1, hidden))
        assert np.array_equal(codes.cpu().numpy(), want_codes), name
        assert np.array_equal(scales.cpu().numpy(), want_scales), name
