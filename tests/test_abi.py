"""The C ABI library on the host: it loads, exports every function the header
declares, checks its arguments with the documented codes, and reports the
launch shape it would use.  None of this launches a kernel."""
import ctypes
import os
import re

import pytest
import torch

from fp8_kv_cache_amd import probe
from fp8_kv_cache_amd import qkv_prep as qp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


PROBE_HEADER = os.path.join(ROOT, "include", "qkv_prep_probe.h")


def declared_functions(headers):
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(qkv_prep_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def operator_headers():
    return [h for h in HEADERS if h != PROBE_HEADER]


def test_header_and_binding_agree():
    assert declared_functions(operator_headers()) == sorted(qp.EXPORTED)
    assert declared_functions([PROBE_HEADER]) == sorted(probe.EXPORTED)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(qp.LIB_PATH)
    for name in declared_functions(operator_headers()):
        assert hasattr(lib, name), name
    plib = ctypes.CDLL(probe.LIB_PATH)
    for name in declared_functions([PROBE_HEADER]):
        assert hasattr(plib, name), name


def test_operator_library_exports_no_probe():
    # The measurement probes live in their own library: an application that
    # links libqkv_prep.so gets the operators only.
    lib = ctypes.CDLL(qp.LIB_PATH)
    for name in probe.EXPORTED:
        assert not hasattr(lib, name), name


def test_struct_sizes_match_the_header_layout():
    assert ctypes.sizeof(qp.QkvPrepConfig) == 40
    assert ctypes.sizeof(qp.QkvPrepArgs) == 88
    assert ctypes.sizeof(qp.QkvPrepLaunch) == 48
    assert ctypes.sizeof(qp.QkvPrepGatherArgs) == 48
    assert ctypes.sizeof(qp.QkvPrepMxfp8Args) == 64


def test_strerror_and_supported():
    assert qp.qkv_prep_strerror(qp.OK) == "ok"
    assert "misaligned" in qp.qkv_prep_strerror(qp.ERR_MISALIGNED)
    assert "unknown" in qp.qkv_prep_strerror(99)
    assert qp.qkv_prep_supported(64)
    assert qp.qkv_prep_supported(1)
    assert not qp.qkv_prep_supported(0)
    assert not qp.qkv_prep_supported(64, 576, 64)
    assert not qp.qkv_prep_supported(64, 512, 32)


def _good_args(T=16, num_blocks=4):
    base = 1 << 20
    return qp.QkvPrepArgs(base, base + 0x100000, base + 0x200000, base + 0x200400,
                          base + 0x300000, base + 0x400000, 4096, base + 0x500000,
                          base + 0x600000, num_blocks, T)


def test_validate_accepts_good_arguments_and_empty_batch():
    cfg = qp.make_config(8)
    assert qp.qkv_prep_validate(cfg, _good_args()) == qp.OK
    a = _good_args(T=0)
    a.q = None
    a.kv = None
    assert qp.qkv_prep_validate(cfg, a) == qp.OK
    a = _good_args()
    a.q_norm_w = None                     # weightless q norm is allowed
    assert qp.qkv_prep_validate(cfg, a) == qp.OK


@pytest.mark.parametrize("field,value,code", [
    ("q", None, qp.ERR_INVALID_ARG),
    ("kv", None, qp.ERR_INVALID_ARG),
    ("kv_norm_w", None, qp.ERR_INVALID_ARG),
    ("positions", None, qp.ERR_INVALID_ARG),
    ("cos_sin", None, qp.ERR_INVALID_ARG),
    ("slot_mapping", None, qp.ERR_INVALID_ARG),
    ("kv_cache", None, qp.ERR_INVALID_ARG),
    ("num_tokens", -1, qp.ERR_INVALID_ARG),
    ("num_blocks", -1, qp.ERR_INVALID_ARG),
    ("max_position", 0, qp.ERR_INVALID_ARG),
    ("q", (1 << 20) + 8, qp.ERR_MISALIGNED),
    ("kv", (1 << 20) + 0x100002, qp.ERR_MISALIGNED),
    ("q_norm_w", (1 << 20) + 0x200004, qp.ERR_MISALIGNED),
    ("cos_sin", (1 << 20) + 0x400004, qp.ERR_MISALIGNED),
    ("kv_cache", (1 << 20) + 0x600008, qp.ERR_MISALIGNED),
    ("positions", (1 << 20) + 0x300004, qp.ERR_MISALIGNED),
    ("slot_mapping", (1 << 20) + 0x500002, qp.ERR_MISALIGNED),
    ("num_tokens", 1 << 30, qp.ERR_UNSUPPORTED),      # T*H rows past 2^31
    ("max_position", (1 << 40) + 1, qp.ERR_UNSUPPORTED),
])
def test_validate_rejects(field, value, code):
    a = _good_args()
    setattr(a, field, value)
    assert qp.qkv_prep_validate(qp.make_config(8), a) == code


def test_cache_may_be_null_without_blocks():
    a = _good_args(num_blocks=0)
    a.kv_cache = None
    assert qp.qkv_prep_validate(qp.make_config(8), a) == qp.OK


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads=0), qp.ERR_INVALID_ARG),
    (dict(block_size=0), qp.ERR_INVALID_ARG),
    (dict(eps=-1.0), qp.ERR_INVALID_ARG),
    (dict(eps=float("nan")), qp.ERR_INVALID_ARG),
    (dict(rows_per_wave=3), qp.ERR_INVALID_ARG),
    (dict(waves_per_block=16), qp.ERR_INVALID_ARG),
    (dict(convert=3), qp.ERR_INVALID_ARG),
    (dict(kv_store=2), qp.ERR_INVALID_ARG),
    (dict(kv_per_wave=3), qp.ERR_INVALID_ARG),
    (dict(kv_per_wave=8), qp.ERR_INVALID_ARG),
])
def test_bad_config(kw, code):
    base = dict(num_heads=8, block_size=64, eps=1e-6)
    base.update(kw)
    cfg = qp.make_config(base.pop("num_heads"), **base)
    assert qp.qkv_prep_validate(cfg, _good_args()) == code
    with pytest.raises(qp.QkvPrepError) as e:
        qp.qkv_prep_launch_shape(cfg, 256, 16)
    assert e.value.code == code


def test_unsupported_head_dim():
    cfg = qp.make_config(8)
    cfg.head_dim = 576
    assert qp.qkv_prep_validate(cfg, _good_args()) == qp.ERR_UNSUPPORTED


def _shape(H, T, **forced):
    s = qp.qkv_prep_launch_shape(qp.make_config(H, **forced), 256, T)
    return (s.rows_per_wave, s.waves_per_block, s.kv_per_wave)


def test_launch_shape_heuristic():
    cfg = qp.make_config(64)
    small = qp.qkv_prep_launch_shape(cfg, 256, 16)
    # decode-sized: two heads of a token per wavefront, one kv token
    assert small.rows_per_wave == 2 and small.waves_per_block == 1 and small.convert == 2
    assert small.kv_per_wave == 1
    assert small.kv_blocks == 16 and small.q_blocks == 16 * 32 and small.grid == 16 * 33
    # from 2^16 q rows: four consecutive tokens per kv wavefront, one q row
    # per wavefront (two heads, two wavefronts per workgroup with at most 56
    # heads from 2^14 tokens)
    at = qp.qkv_prep_launch_shape(cfg, 256, 1024)
    assert at.kv_per_wave == 4 and at.kv_blocks == 1024 // 4 and at.rows_per_wave == 1
    assert _shape(64, 2048) == (1, 1, 4)
    assert _shape(8, 8192) == (1, 1, 4)
    few = qp.qkv_prep_launch_shape(qp.make_config(8), 256, 16384)
    assert (few.rows_per_wave, few.waves_per_block, few.kv_per_wave) == (2, 2, 4)
    assert few.kv_blocks == 16384 // 8 and few.q_blocks == 16384 * 4 // 2
    assert _shape(16, 16384)[0] == 2 and _shape(17, 16384)[0] == 2 and _shape(56, 16384)[0] == 2
    assert _shape(57, 16384)[0] == 1 and _shape(40, 16383)[0] == 1 and _shape(64, 65536)[0] == 1
    # below 2^16: one row and four kv tokens from 49152 q rows, from 2^15
    # with more than 4096 tokens, from 24576 with more than 8192
    assert _shape(64, 1023) == (1, 1, 4)                                     # 65472 rows
    assert _shape(12, 4096) == (1, 1, 4) and _shape(11, 4096) == (2, 2, 2)   # 49152 / 45056 rows
    assert _shape(8, 4097) == (1, 1, 4) and _shape(8, 4096) == (2, 2, 2)     # 2^15 rows, > 4096 tokens
    assert _shape(2, 16384) == (1, 1, 4)
    assert _shape(3, 8193) == (1, 1, 4) and _shape(3, 8192) == (1, 1, 2)     # 24579 / 24576 rows
    assert _shape(1, 24576) == (1, 1, 4) and _shape(1, 32768) == (1, 1, 4)
    # else from 2^15 q rows with at least 2048 tokens: two heads, two kv
    # tokens, two wavefronts per workgroup
    mid = qp.qkv_prep_launch_shape(qp.make_config(16), 256, 2048)
    assert (mid.rows_per_wave, mid.waves_per_block, mid.kv_per_wave) == (2, 2, 2)
    assert mid.kv_blocks == 2048 // 4 and mid.q_blocks == 2048 * 8 // 2
    # else from 3072 tokens, or 2048 with an odd head count: one row per
    # wavefront, two kv tokens from 2^14 q rows or above 8192 tokens
    assert _shape(2, 3072) == (1, 1, 1) and _shape(2, 3071) == (2, 1, 1)
    assert _shape(7, 2048) == (1, 1, 1) and _shape(7, 2047) == (2, 1, 1) and _shape(8, 2048) == (2, 1, 1)
    assert _shape(11, 2048) == (1, 1, 2)                                     # 22528 rows
    assert _shape(4, 4096) == (1, 1, 2) and _shape(4, 4095) == (1, 1, 1)     # 2^14 rows
    assert _shape(1, 8193) == (1, 1, 2) and _shape(1, 8192) == (1, 1, 1)
    assert _shape(6, 4096) == (1, 1, 2)
    # else two heads per wavefront, one kv token
    for H, T in ((32, 1024), (8, 2047), (64, 511), (16, 1024)):
        assert _shape(H, T) == (2, 1, 1)
    one_head = qp.qkv_prep_launch_shape(qp.make_config(1), 256, 100)
    assert one_head.rows_per_wave == 1 and one_head.q_blocks == 100
    odd_heads = qp.qkv_prep_launch_shape(qp.make_config(5), 256, 10)
    assert odd_heads.rows_per_wave == 2 and odd_heads.q_blocks == 10 * 3      # ceil(5 / 2) per token
    assert qp.qkv_prep_launch_shape(cfg, 256, 0).grid == 0
    big = qp.qkv_prep_launch_shape(qp.make_config(128), 256, 131072)
    assert big.rows_per_wave == 1 and big.waves_per_block == 1
    assert big.q_blocks == 131072 * 128 and big.kv_blocks == 131072 // 4
    # a batch whose grid passes 2^32 work-items keeps one row per wavefront
    # (qkv_prep_run splits the grid into consecutive dispatches)
    huge = qp.qkv_prep_launch_shape(qp.make_config(128), 256, 600000)
    assert huge.rows_per_wave == 1 and huge.q_blocks == 600000 * 128
    assert huge.grid * 64 * huge.waves_per_block >= 2 ** 32
    # forced fields: each overrides its part; the workgroup width follows the
    # q rows per wavefront in use (two with two heads where the rule takes
    # several kv tokens)
    ragged = qp.qkv_prep_launch_shape(qp.make_config(64, kv_per_wave=4), 256, 17)
    assert ragged.kv_per_wave == 4 and ragged.kv_blocks == 5                  # ceil(17 / 4)
    assert qp.qkv_prep_launch_shape(qp.make_config(64, kv_per_wave=2, waves_per_block=2),
                                    256, 9).kv_blocks == 3                    # ceil(9 / (2 * 2))
    assert _shape(6, 8192, rows_per_wave=2) == (2, 2, 4)
    assert _shape(8, 4096, rows_per_wave=1) == (1, 1, 2)
    assert _shape(8, 16384, waves_per_block=1) == (2, 1, 4)
    forced = qp.qkv_prep_launch_shape(qp.make_config(64, rows_per_wave=2, waves_per_block=8,
                                                     convert=1), 256, 1000)
    assert (forced.rows_per_wave, forced.waves_per_block, forced.convert) == (2, 8, 1)
    assert forced.kv_per_wave == 4                                            # 64000 rows
    assert forced.q_blocks == -(-(1000 * 32) // 8)
    assert forced.kv_blocks == -(-1000 // (4 * 8))
    # the row limit of qkv_prep_run also bounds the shape query (no overflow)
    for T in (2 ** 31 // 64, 2 ** 62, 2 ** 63 - 1):
        with pytest.raises(qp.QkvPrepError) as e:
            qp.qkv_prep_launch_shape(cfg, 256, T)
        assert e.value.code == qp.ERR_UNSUPPORTED
    assert qp.qkv_prep_launch_shape(cfg, 256, 2 ** 31 // 64 - 1).grid > 0
    odd = qp.qkv_prep_launch_shape(qp.make_config(3, waves_per_block=4), 256, 5)
    assert odd.rows_per_wave == 2 and odd.q_blocks == 3 and odd.kv_blocks == 2   # 5 * 2 wavefronts / 4


def _grid_roles(s):
    """The kernel's grid-index mapping, restated: for every workgroup of a
    launch, ("kv", j) or ("q", j) with j its index among its kind."""
    K, Q, P = s.kv_blocks, s.q_blocks, s.kv_period
    roles = []
    for b in range(K + Q):
        if P:
            j = b // P
            if j < K and b == j * P:
                roles.append(("kv", j))
            else:
                roles.append(("q", b - min(j + 1, K)))
        else:
            roles.append(("kv", b) if b < K else ("q", b - K))
    return roles


def test_kv_workgroups_spread_over_large_two_heads_grids():
    # kv first, except with two heads and four kv tokens per wavefront from
    # 2^18 q rows: kv workgroup j at grid index j * P, P = floor(3N / 4K)
    # made odd by rounding down, so the kv workgroups cover the first 55-75%
    # of the grid and fall on every XCD (index mod 8) in turn.
    for H, T, P in ((16, 16384, 23), (8, 32768, 11), (2, 131072, 3), (16, 131072, 23), (4, 65536, 5)):
        s = qp.qkv_prep_launch_shape(qp.make_config(H), 256, T)
        assert (s.rows_per_wave, s.kv_per_wave) == (2, 4) and s.kv_period == P
        assert P % 2 == 1 and P == (3 * s.grid // (4 * s.kv_blocks)) - (3 * s.grid // (4 * s.kv_blocks) + 1) % 2
        last = (s.kv_blocks - 1) * P
        assert 0.55 * s.grid <= last < 0.75 * s.grid
        assert len({(j * P) % 8 for j in range(min(s.kv_blocks, 8))}) == min(s.kv_blocks, 8)
    for H, T in ((8, 16384), (16, 16383), (64, 65536), (32, 16383), (2, 65535), (57, 32768)):
        assert qp.qkv_prep_launch_shape(qp.make_config(H), 256, T).kv_period == 0      # below 2^18 rows, or one row
    forced = qp.qkv_prep_launch_shape(qp.make_config(64, rows_per_wave=2, kv_per_wave=4), 256, 8192)
    assert forced.kv_period > 0 and forced.waves_per_block == 2                            # the shape in use decides
    assert qp.qkv_prep_launch_shape(qp.make_config(16, kv_per_wave=2), 256, 16384).kv_period == 0
    assert qp.qkv_prep_launch_shape(qp.make_config(16), 256, 0).kv_period == 0


def test_grid_mapping_covers_every_workgroup_once():
    # Every kv and q workgroup index appears exactly once, with and without
    # the spread, on ragged sizes around the threshold and the forced shapes.
    cases = [(9, 29127, {}), (9, 29128, {}), (3, 87382, {}), (16, 16385, {}), (5, 60000, {"waves_per_block": 1}),
             (12, 40000, {"waves_per_block": 4}), (64, 4099, {"rows_per_wave": 2, "kv_per_wave": 4}), (8, 1000, {})]
    seen_spread = 0
    for H, T, forced in cases:
        s = qp.qkv_prep_launch_shape(qp.make_config(H, **forced), 256, T)
        seen_spread += s.kv_period > 0
        roles = _grid_roles(s)
        kv = sorted(j for r, j in roles if r == "kv")
        q = sorted(j for r, j in roles if r == "q")
        assert kv == list(range(s.kv_blocks)) and q == list(range(s.q_blocks)), (H, T, forced)
    assert seen_spread >= 5


def test_fast_division_used_by_the_kernel():
    # The kernel divides row indices by H and slots by the block size with a
    # multiply-high and shift (constants from the host).  Check the scheme on
    # the host with the same formula, against Python's integer division.
    import random
    rng = random.Random(3)
    for d in list(range(1, 300)) + [511, 512, 513, 1000, 4095, 4096, 65535, 65536, 1 << 20,
                                   (1 << 31) - 1, 1 << 31]:
        l = 0
        while (1 << l) < d:
            l += 1
        m = ((1 << 32) * ((1 << l) - d)) // d + 1
        assert 0 < m < (1 << 32) or d == 1 or d == (1 << l)
        ns = [0, 1, d - 1, d, d + 1, (1 << 31) - 1] + [rng.randrange(1 << 31) for _ in range(300)]
        for n in ns:
            if n >= (1 << 31):
                continue
            assert ((((n * m) >> 32) + n) >> l) == n // d, (d, n)


def test_probes_reject_bad_arguments_without_launching():
    lib = probe.library()
    assert lib.qkv_prep_probe_copy(None, None, 0, None) == qp.OK
    assert lib.qkv_prep_probe_copy(None, None, 16, None) == qp.ERR_INVALID_ARG
    assert lib.qkv_prep_probe_copy(1 << 20, 2 << 20, 15, None) == qp.ERR_INVALID_ARG
    assert lib.qkv_prep_probe_copy((1 << 20) + 8, 2 << 20, 16, None) == qp.ERR_INVALID_ARG
    assert lib.qkv_prep_probe_copy(1 << 20, 2 << 20, -16, None) == qp.ERR_INVALID_ARG
    assert lib.qkv_prep_probe_update(None, 0, None) == qp.OK
    assert lib.qkv_prep_probe_update(None, 16, None) == qp.ERR_INVALID_ARG
    assert lib.qkv_prep_probe_update(1 << 20, 15, None) == qp.ERR_INVALID_ARG
    assert lib.qkv_prep_probe_update((1 << 20) + 8, 16, None) == qp.ERR_INVALID_ARG
    assert lib.qkv_prep_probe_update(1 << 20, -16, None) == qp.ERR_INVALID_ARG
    st = lib.qkv_prep_probe_stream
    A, B = 1 << 20, 1 << 30                     # aligned, non-overlapping stand-in addresses
    R, Wr, C, U = probe.READ, probe.WRITE, probe.COPY, probe.UPDATE
    NT, SC1, SC0 = probe.NT, probe.SC1, probe.SC0
    # Good arguments with nothing to do return OK without launching.
    assert st(R, NT, 0, 0, 256, 1, 0, A, B, 0, 0, None) == qp.OK
    assert st(Wr, 0, NT | SC1, 0, 64, 1, 0, A, None, 0, 0, None) == qp.OK
    assert st(C, NT, NT | SC1, 1, 1024, 1, 0, A, B, 0, 0, None) == qp.OK
    assert st(U, NT, SC0 | NT | SC1, 1, 64, 1, 0, A, None, 0, 0, None) == qp.OK
    assert st(R, 0, 0, 0, 256, 1, 0, A + 4, B, 0, 0, None) == qp.OK        # a read's sink is a word
    for depth in (2, 4, 8, 16):
        assert st(R, NT, 0, 0, 64, depth, 0, A, B, 0, 0, None) == qp.OK
        assert st(Wr, 0, NT | SC1, 0, 64, depth, 0, A, None, 0, 0, None) == qp.OK
        assert st(C, NT, NT | SC1, 0, 64, depth, 0, A, B, 0, 0, None) == qp.OK
        assert st(U, NT, NT | SC1, 0, 1024, depth, 0, A, None, 0, 0, None) == qp.OK
    bad = [
        (4, NT, 0, 0, 256, 1, 0, A, B, 16),            # no such kind
        (-1, NT, 0, 0, 256, 1, 0, A, B, 16),
        (R, NT, 0, 0, 256, 1, 0, A, B, 15),            # not whole chunks
        (R, NT, 0, 0, 256, 1, 0, A, B, -16),
        (R, NT, 0, 0, 32, 1, 0, A, B, 16),             # lanes per block
        (R, NT, 0, 0, 2048, 1, 0, A, B, 16),
        (R, NT, 0, 0, 96, 1, 0, A, B, 16),
        (R, SC1, 0, 0, 256, 1, 0, A, B, 16),           # load policy outside the accepted set
        (R, SC0 | NT, 0, 0, 256, 1, 0, A, B, 16),
        (R, NT, NT, 0, 256, 1, 0, A, B, 16),           # a read makes no store
        (Wr, NT, NT, 0, 256, 1, 0, A, None, 16),       # a write makes no load
        (Wr, 0, SC0, 0, 256, 1, 0, A, None, 16),       # store policy outside the accepted set
        (Wr, 0, NT | SC0, 0, 256, 1, 0, A, None, 16),
        (R, NT, 0, 1, 256, 1, 0, A, B, 16),            # sleep only in a copy or an update
        (Wr, 0, NT, 1, 256, 1, 0, A, None, 16),
        (C, NT, NT, 2, 256, 1, 0, A, B, 16),           # sleep is 0 or 1
        (R, NT, 0, 0, 256, 1, 0, None, B, 16),         # NULL sink
        (R, NT, 0, 0, 256, 1, 0, A + 2, B, 16),        # misaligned sink
        (R, NT, 0, 0, 256, 1, 0, A, None, 16),         # NULL source
        (R, NT, 0, 0, 256, 1, 0, A, B + 8, 16),        # misaligned source
        (Wr, 0, NT, 0, 256, 1, 0, A + 4, None, 16),    # misaligned destination
        (Wr, 0, NT, 0, 256, 1, 0, A, B, 16),           # a write takes no source
        (U, NT, NT, 0, 256, 1, 0, A, B, 16),           # an update takes no source
        (C, NT, NT, 0, 256, 1, 0, A, A + 16, 32),      # overlapping copy
        (C, NT, NT, 0, 256, 1, 0, A + 16, A, 32),
        (C, NT, NT, 0, 256, 1, 0, A, None, 16),
        (Wr, 0, NT, 0, 64, 1, 0, A, None, (1 << 31) * 64 * 16),  # 2^31 workgroups
        (Wr, 0, NT | SC1, 0, 64, 16, 0, A, None, (1 << 31) * 64 * 16 * 16),
        (R, NT, 0, 0, 256, 3, 0, A, B, 16),         # depth 1, 2, 4, 8 or 16
        (R, NT, 0, 0, 256, 32, 0, A, B, 16),
        (R, NT, 0, 0, 256, 0, 0, A, B, 16),
        (R, NT | SC1, 0, 0, 256, 2, 0, A, B, 16),   # depth > 1: nt loads, nt sc1 stores, no pause
        (Wr, 0, NT, 0, 256, 4, 0, A, None, 16),
        (C, NT, NT, 0, 256, 8, 0, A, B, 16),
        (C, 0, NT | SC1, 0, 256, 8, 0, A, B, 16),
        (U, NT, NT | SC1, 1, 256, 2, 0, A, None, 16),
    ]
    for a in bad:
        assert st(*a, 0, None) == qp.ERR_INVALID_ARG, a
    for xcd in (0, 1):
        assert st(C, NT, NT | SC1, 0, 64, 1, xcd, A, B, 0, 0, None) == qp.OK
    for xcd in (-1, 2):
        assert st(C, NT, NT | SC1, 0, 64, 1, xcd, A, B, 16, 0, None) == qp.ERR_INVALID_ARG
    # the padded grid must stay below 2^31 workgroups too
    assert st(Wr, 0, NT, 0, 64, 1, 1, A, None, ((1 << 31) - 7) * 64 * 16, 0, None) == qp.ERR_INVALID_ARG
    mx = lib.qkv_prep_probe_mxfp8_pattern
    X, Rs, Gm, Ro, Cd, Sc = 1 << 20, 2 << 20, 6 << 20, 3 << 20, 4 << 20, 5 << 20
    assert mx(X, Rs, Gm, Ro, Cd, Sc, 0, 7168, 15, None) == qp.OK             # no rows
    assert mx(X, None, Gm, None, Cd, None, 0, 512, 2, None) == qp.OK         # codes only
    assert mx(X, None, Gm, None, None, Sc + 4, 0, 16384, 12, None) == qp.OK  # scales + barrier
    assert mx(X, Rs, None, Ro, None, None, 0, 1024, 9, None) == qp.OK        # no gamma without codes/scales
    for a in [
        (X, Rs, Gm, Ro, Cd, Sc, 0, 7168, 0),          # no stream
        (X, Rs, Gm, Ro, Cd, Sc, 0, 7168, 8),          # a barrier alone stores nothing
        (X, Rs, Gm, Ro, Cd, Sc, 0, 7168, 16),
        (X, Rs, Gm, Ro, Cd, Sc, -1, 7168, 15),
        (X, Rs, Gm, Ro, Cd, Sc, 0, 7040, 15),         # hidden a multiple of 512
        (X, Rs, Gm, Ro, Cd, Sc, 0, 0, 15),
        (X, Rs, Gm, Ro, Cd, Sc, 0, 16896, 15),        # above 16384
        (X, Rs, Gm, Ro, Cd, Sc, 0, 512 * 17, 15),     # 17 groups: odd above 15
        (None, Rs, Gm, Ro, Cd, Sc, 0, 7168, 15),
        (X + 8, Rs, Gm, Ro, Cd, Sc, 0, 7168, 15),
        (X, None, Gm, Ro, Cd, Sc, 0, 7168, 1),
        (X, Rs, Gm, None, Cd, Sc, 0, 7168, 1),
        (X, Rs + 8, Gm, Ro, Cd, Sc, 0, 7168, 1),
        (X, Rs, Gm, Ro + 8, Cd, Sc, 0, 7168, 1),
        (X, Rs, Gm, Ro, None, Sc, 0, 7168, 2),
        (X, Rs, Gm, Ro, Cd + 4, Sc, 0, 7168, 2),
        (X, Rs, Gm, Ro, Cd, None, 0, 7168, 4),
        (X, Rs, Gm, Ro, Cd, Sc + 2, 0, 7168, 4),
        (X, Rs, None, Ro, Cd, Sc, 0, 7168, 2),        # codes need gamma
        (X, Rs, None, Ro, Cd, Sc, 0, 7168, 4),        # scales need gamma
        (X, Rs, Gm + 8, Ro, Cd, Sc, 0, 7168, 6),
        (X, Rs, Gm, Ro, Cd, Sc, (1 << 32) // 448, 7168, 15),   # 2^32 work-items
    ]:
        assert mx(*a, None) == qp.ERR_INVALID_ARG, a
    conv = lib.qkv_prep_probe_convert
    assert conv(None, 0, None, None, 2, None) == qp.OK
    assert conv(None, 4, None, None, 2, None) == qp.ERR_INVALID_ARG            # NULL input
    assert conv(1 << 20, 6, None, None, 2, None) == qp.ERR_INVALID_ARG         # n not a multiple of 4
    assert conv(1 << 20, 4, None, None, 3, None) == qp.ERR_INVALID_ARG         # bad path
    assert conv((1 << 20) + 4, 4, None, None, 1, None) == qp.ERR_INVALID_ARG   # input misaligned
    assert conv(1 << 20, 4, (2 << 20) + 2, None, 1, None) == qp.ERR_INVALID_ARG
    assert conv(1 << 20, 4, None, (3 << 20) + 4, 1, None) == qp.ERR_INVALID_ARG
    assert conv(1 << 20, 1 << 33, None, None, 1, None) == qp.ERR_INVALID_ARG
    ue = lib.qkv_prep_probe_ue8m0
    assert ue(None, 0, None, None, None, None) == qp.OK                        # nothing to do
    assert ue(None, 4, None, None, None, None) == qp.ERR_INVALID_ARG           # NULL input
    assert ue(1 << 20, -4, None, None, None, None) == qp.ERR_INVALID_ARG
    assert ue((1 << 20) + 2, 4, None, None, None, None) == qp.ERR_INVALID_ARG  # input misaligned
    assert ue(1 << 20, 4, None, None, (2 << 20) + 1, None) == qp.ERR_INVALID_ARG
    assert ue(1 << 20, 1 << 38, None, None, None, None) == qp.ERR_INVALID_ARG


def test_gather_without_handle_is_rejected():
    args = qp.QkvPrepGatherArgs(1 << 20, 4, 2 << 20, 8, 3 << 20, qp.OUT_F32)
    assert qp.library().qkv_prep_gather(None, ctypes.byref(args), None) == qp.ERR_INVALID_ARG


def test_run_without_handle_is_rejected():
    assert qp.library().qkv_prep_run(None, ctypes.byref(_good_args()), None) == qp.ERR_INVALID_ARG
    assert qp.library().qkv_prep_destroy(None) == qp.OK


def test_prepared_launch_reports_the_c_code_and_keeps_its_arguments_alive():
    """A Launch is one C call plus the return-code check.  With a cleared
    handle cell (what QkvPrep.close leaves behind) the run is refused with
    ERR_INVALID_ARG, before any device work."""
    args = _good_args()
    cell = ctypes.c_void_p(None)
    launch = qp.Launch(qp.library().qkv_prep_run, (cell, ctypes.byref(args), None), "qkv_prep_run",
                       (args,))
    del args
    with pytest.raises(qp.QkvPrepError) as e:
        launch()
    assert e.value.code == qp.ERR_INVALID_ARG
    assert "qkv_prep_run" in str(e.value)
    calls = []
    ok = qp.Launch(lambda *a: calls.append(a) or qp.OK, (1, 2, 3), "x", ())
    ok()
    ok()
    assert calls == [(1, 2, 3), (1, 2, 3)]
    # on_stream replaces only the last argument (the stream)
    moved = ok.on_stream(9)
    moved()
    assert calls[-1] == (1, 2, 9) and type(moved) is qp.Launch


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")
def test_create_without_a_device_reports_no_device():
    with pytest.raises(qp.QkvPrepError) as e:
        qp.qkv_prep_create(qp.make_config(8), 0)
    assert e.value.code == qp.ERR_NO_DEVICE


def test_create_rejects_bad_config_before_touching_a_device():
    with pytest.raises(qp.QkvPrepError) as e:
        qp.qkv_prep_create(qp.make_config(0), 0)
    assert e.value.code == qp.ERR_INVALID_ARG


def test_ctypes_layout_matches_the_c_compiler(tmp_path):
    # Compile a few lines of C against the header and compare every field
    # offset with the ctypes mirror.
    import subprocess
    fields = {"qkv_prep_config": qp.QkvPrepConfig, "qkv_prep_args": qp.QkvPrepArgs,
              "qkv_prep_launch": qp.QkvPrepLaunch, "qkv_prep_gather_args": qp.QkvPrepGatherArgs,
              "qkv_prep_mxfp8_args": qp.QkvPrepMxfp8Args}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "qkv_prep.h"',
             '#include "qkv_prep_mxfp8.h"', "int main(void){"]
    for cname, cls in fields.items():
        lines.append('printf("%%zu\\n", sizeof(%s));' % cname)
        for f, _ in cls._fields_:
            lines.append('printf("%%zu\\n", offsetof(%s, %s));' % (cname, f))
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = []
    for cls in fields.values():
        want.append(ctypes.sizeof(cls))
        want += [getattr(cls, f).offset for f, _ in cls._fields_]
    assert got == want


def test_mxfp8_scale_bytes_and_argument_checks():
    assert qp.qkv_prep_mxfp8_scale_bytes(1, 512) == 128 * 16
    assert qp.qkv_prep_mxfp8_scale_bytes(128, 7168) == 128 * 224
    assert qp.qkv_prep_mxfp8_scale_bytes(129, 1024) == 256 * 32
    assert qp.qkv_prep_mxfp8_scale_bytes(0, 512) == 0
    assert qp.qkv_prep_mxfp8_scale_bytes(4, 96) == -1
    good = dict(x=1 << 20, residual=None, residual_out=None, gamma=2 << 20, quant_out=3 << 20,
                scale_out=4 << 20, m=4, hidden=1024, eps=1e-6)

    def code(**kw):
        d = dict(good)
        d.update(kw)
        a = qp.QkvPrepMxfp8Args(d["x"], d["residual"], d["residual_out"], d["gamma"],
                                d["quant_out"], d["scale_out"], d["m"], d["hidden"], d["eps"])
        return qp.library().qkv_prep_mxfp8_norm_quant(ctypes.byref(a), d.get("device", 0), None)
    assert code(m=0) == qp.OK
    assert code(m=-1) == qp.ERR_INVALID_ARG
    assert code(eps=-1.0) == qp.ERR_INVALID_ARG
    assert code(x=None) == qp.ERR_INVALID_ARG
    assert code(gamma=None) == qp.ERR_INVALID_ARG
    assert code(scale_out=None) == qp.ERR_INVALID_ARG
    assert code(hidden=96) == qp.ERR_UNSUPPORTED             # not a multiple of 128
    assert code(hidden=200) == qp.ERR_UNSUPPORTED
    assert code(hidden=16512) == qp.ERR_UNSUPPORTED          # above 16384
    assert code(hidden=-128) == qp.ERR_UNSUPPORTED
    assert code(scale_out=(4 << 20) + 2) == qp.ERR_MISALIGNED
    assert code(x=(1 << 20) + 2) == qp.ERR_MISALIGNED
    assert code(residual=(5 << 20) + 4) == qp.ERR_MISALIGNED
    assert code(residual_out=(6 << 20) + 8) == qp.ERR_MISALIGNED
    assert code(m=1 << 26) == qp.ERR_UNSUPPORTED
    # The grid limit: round_up(m, 128) workgroups of W lanes must stay below
    # 2^32 work-items (W = 64 at hidden 128, 192 at 1152, 1024 at 16384).
    # Sizes that fit reach the device check (device -1: nothing is launched).
    for hidden, lanes in ((128, 64), (1152, 192), (16384, 1024)):
        top = (2 ** 32 - 1) // lanes // 128 * 128
        assert code(hidden=hidden, m=top, device=-1) == qp.ERR_NO_DEVICE
        assert code(hidden=hidden, m=top + 1) == qp.ERR_UNSUPPORTED
    # Good arguments on a device that does not exist: rejected before any launch.
    assert code(device=-1) == qp.ERR_NO_DEVICE
    assert code(device=1 << 20) == qp.ERR_NO_DEVICE


def test_binding_fails_loudly_without_the_library(tmp_path):
    # A copy of the package with no libqkv_prep.so: importing the binding must
    # raise, never fall back to anything else.
    import shutil
    import subprocess
    import sys
    src = os.path.dirname(qp.__file__)
    pkg = tmp_path / "fp8_kv_cache_amd"
    pkg.mkdir()
    for f in ("__init__.py", "qkv_prep.py", "workloads.py"):
        shutil.copy(os.path.join(src, f), pkg / f)
    code = ("import sys; sys.path.insert(0, sys.argv[1])\n"
            "try:\n"
            "    import fp8_kv_cache_amd.qkv_prep\n"
            "except ImportError as e:\n"
            "    print('ImportError:', e); sys.exit(0)\n"
            "sys.exit(3)\n")
    res = subprocess.run([sys.executable, "-c", code, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "libqkv_prep.so is not built" in res.stdout


def test_public_headers_compile_as_c99_and_cpp(tmp_path):
    # Every public header, alone and together, from plain C (C99, pedantic,
    # warnings as errors) and from C++11: a C consumer needs nothing else.
    import shutil
    import subprocess
    headers = sorted({os.path.basename(h) for h in HEADERS + [PROBE_HEADER]})
    src = tmp_path / "hdr.c"
    src.write_text("".join('#include "%s"\n' % h for h in headers) + "int main(void) { return 0; }\n")
    for cc, std, lang in (("gcc", "-std=c99", "c"), ("g++", "-std=c++11", "c++")):
        if shutil.which(cc) is None:
            pytest.skip("%s not available" % cc)
        res = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                              os.path.join(ROOT, "include"), "-x", lang, str(src), "-o", str(tmp_path / "hdr")],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
