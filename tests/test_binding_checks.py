"""The Python binding's tensor checks (host only, CPU tensors): the C ABI takes
bare pointers, so shapes, dtypes, contiguity and devices are checked in the
binding before any launch.  A good set passes; each single fault raises."""
import pytest
import torch

from fp8_kv_cache_amd import qkv_prep as qp

T, H, B, P = 5, 3, 4, 10


def good():
    return dict(q=torch.zeros((T, H, 512), dtype=torch.bfloat16), kv=torch.zeros((T, 512), dtype=torch.bfloat16),
                q_norm_w=torch.zeros(512, dtype=torch.bfloat16), kv_norm_w=torch.zeros(512, dtype=torch.bfloat16),
                positions=torch.zeros(T, dtype=torch.int64), cos_sin=torch.zeros((P, 64), dtype=torch.float32),
                slot_mapping=torch.zeros(T, dtype=torch.int64),
                kv_cache=torch.zeros((2, B * qp.SLOT_BYTES), dtype=torch.uint8))


def check(t, device="cpu", slot_bytes=qp.SLOT_BYTES):
    qp.check_op_tensors(H, B, slot_bytes, device, t["q"], t["kv"], t["q_norm_w"], t["kv_norm_w"],
                        t["positions"], t["cos_sin"], t["slot_mapping"], t["kv_cache"])


def test_good_operator_tensors_pass():
    check(good())
    t = good()
    t["q_norm_w"] = None                      # weightless q norm
    check(t)
    t["kv_cache"] = torch.zeros((3, B * 1024), dtype=torch.uint8)
    check(t, slot_bytes=qp.BF16_SLOT_BYTES)


@pytest.mark.parametrize("name,bad,err", [
    ("q", torch.zeros((T, H + 1, 512), dtype=torch.bfloat16), ValueError),
    ("q", torch.zeros((T, H, 448), dtype=torch.bfloat16), ValueError),
    ("kv", torch.zeros((T - 1, 512), dtype=torch.bfloat16), ValueError),
    ("kv", torch.zeros((T, 512), dtype=torch.float16), TypeError),
    ("kv", torch.zeros((512, T), dtype=torch.bfloat16).t(), ValueError),
    ("q_norm_w", torch.zeros(448, dtype=torch.bfloat16), ValueError),
    ("kv_norm_w", torch.zeros(512, dtype=torch.float32), TypeError),
    ("positions", torch.zeros(T + 1, dtype=torch.int64), ValueError),
    ("positions", torch.zeros(T, dtype=torch.int32), TypeError),
    ("slot_mapping", torch.zeros(T - 1, dtype=torch.int64), ValueError),
    ("cos_sin", torch.zeros((P, 32), dtype=torch.float32), ValueError),
    ("cos_sin", torch.zeros((0, 64), dtype=torch.float32), ValueError),
    ("cos_sin", torch.zeros((P, 64), dtype=torch.float64), TypeError),
    ("kv_cache", torch.zeros(B * qp.SLOT_BYTES + 1, dtype=torch.uint8), ValueError),
    ("kv_cache", torch.zeros(B * qp.SLOT_BYTES, dtype=torch.int8), TypeError),
])
def test_each_operator_fault_raises(name, bad, err):
    t = good()
    t[name] = bad
    with pytest.raises(err):
        check(t)


def test_wrong_device_raises():
    with pytest.raises(ValueError, match="must be on"):
        check(good(), device="cuda:0")


def test_gather_checks():
    cache = torch.zeros((2, B * qp.SLOT_BYTES), dtype=torch.uint8)
    slots = torch.zeros(7, dtype=torch.int64)
    qp.check_gather_tensors(B, "cpu", cache, slots, torch.zeros((7, 512), dtype=torch.float32))
    qp.check_gather_tensors(B, "cpu", cache, slots, torch.zeros((7, 512), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        qp.check_gather_tensors(B, "cpu", cache, slots, torch.zeros((6, 512), dtype=torch.float32))
    with pytest.raises(TypeError):
        qp.check_gather_tensors(B, "cpu", cache, slots, torch.zeros((7, 512), dtype=torch.float16))
    with pytest.raises(ValueError):
        qp.check_gather_tensors(B, "cpu", cache[:, 1:], slots, torch.zeros((7, 512), dtype=torch.float32))
    with pytest.raises(ValueError):
        qp.check_gather_tensors(B, "cpu", cache, slots.view(7, 1), torch.zeros((7, 512), dtype=torch.float32))
    with pytest.raises(ValueError):
        qp.check_gather_tensors(B, "cuda:0", cache, slots, torch.zeros((7, 512), dtype=torch.float32))


def test_mxfp8_checks():
    m, h = 130, 1024
    x = torch.zeros((m, h), dtype=torch.bfloat16)
    g = torch.zeros(h, dtype=torch.bfloat16)
    codes = torch.zeros((m, h), dtype=torch.uint8)
    scales = torch.zeros(qp.qkv_prep_mxfp8_scale_bytes(m, h), dtype=torch.uint8)
    qp.check_mxfp8_tensors(x, g, x.clone(), x.clone(), codes, scales)
    qp.check_mxfp8_tensors(x, g, None, None, codes, scales)
    for args in ((x, g[:-1], None, None, codes, scales),
                 (x, g, x[:-1], None, codes, scales),
                 (x, g, None, x[:, :-8], codes, scales),
                 (x, g, None, None, codes[:-1], scales),
                 (x, g, None, None, codes, scales[:-1])):
        with pytest.raises(ValueError):
            qp.check_mxfp8_tensors(*args)
    with pytest.raises(TypeError):
        qp.check_mxfp8_tensors(x.float(), g, None, None, codes, scales)


def test_mxfp8_wrapper_rejects_host_tensors():
    """The wrapper refuses host tensors before any device call (their
    pointers would reach the kernel otherwise)."""
    x = torch.zeros((4, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        qp.mxfp8_norm_quant(x, torch.zeros(512, dtype=torch.bfloat16), 1e-6,
                            quant_out=torch.zeros((4, 512), dtype=torch.uint8),
                            scale_out=torch.zeros(qp.qkv_prep_mxfp8_scale_bytes(4, 512), dtype=torch.uint8),
                            stream=0)
