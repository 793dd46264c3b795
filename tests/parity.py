"""Helpers for the GPU-vs-oracle parity tests (not a test module).

The comparison is element by element on every token: q as bf16 ulps, the
cache split by what each byte is (E4M3 code, bf16 rope value, exponent byte,
pad byte, or a byte no slot owns).  The bar:
  * exponent bytes, pad bytes, untouched bytes and slot placement: bit-exact;
  * q and rope bf16 values: within 1 bf16 ulp;
  * E4M3 codes: within 1 step.
The counts of inexact values are returned too; with the pinned arithmetic
they are expected to be zero."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from fp8_kv_cache_amd import workloads as W

UNTOUCHED, CODE, ROPE, EXP, PAD = 0, 1, 2, 3, 4


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bf16_ord(u):
    u = np.asarray(u, np.uint16).astype(np.int32)
    m = u & 0x7FFF
    return np.where(u & 0x8000, -m, m)


def e4m3_ord(c):
    c = np.asarray(c, np.uint8).astype(np.int32)
    m = c & 0x7F
    return np.where(c & 0x80, -m, m)


def byte_roles(slots, num_blocks, block_size):
    """Role of every cache byte given the slot mapping."""
    roles = np.zeros(num_blocks * block_size * W.SLOT_BYTES, np.uint8)
    s = np.asarray(slots, np.int64)
    s = np.unique(s[(s >= 0) & (s < num_blocks * block_size)])
    blk, sib = s // block_size, s % block_size
    base = blk * block_size * W.SLOT_BYTES
    data = base + sib * 576
    scale = base + block_size * 576 + sib * 8
    roles[(data[:, None] + np.arange(448)[None, :]).ravel()] = CODE
    roles[(data[:, None] + 448 + np.arange(128)[None, :]).ravel()] = ROPE
    roles[(scale[:, None] + np.arange(7)[None, :]).ravel()] = EXP
    roles[scale + 7] = PAD
    return roles


def compare_cache(got, want, roles):
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want).reshape(-1)
    exact = (roles == UNTOUCHED) | (roles == EXP) | (roles == PAD)
    out = {"cache_exact_mismatch": int(np.count_nonzero(got[exact] != want[exact]))}
    code = roles == CODE
    dc = np.abs(e4m3_ord(got[code]) - e4m3_ord(want[code]))
    out["code_max_step"] = int(dc.max()) if dc.size else 0
    out["code_inexact"] = int(np.count_nonzero(dc))
    rope_idx = np.nonzero(roles == ROPE)[0]
    lo = rope_idx[::2]
    g16 = got[lo].astype(np.uint16) | (got[lo + 1].astype(np.uint16) << 8)
    w16 = want[lo].astype(np.uint16) | (want[lo + 1].astype(np.uint16) << 8)
    dr = np.abs(bf16_ord(g16) - bf16_ord(w16))
    out["rope_max_ulp"] = int(dr.max()) if dr.size else 0
    out["rope_inexact"] = int(np.count_nonzero(dr))
    out["cache_bytes_differ"] = int(np.count_nonzero(got != want))
    return out


def compare_bf16_cache(got, want, slots, num_slots):
    """bf16-store cache: every valid slot's 512 values within 1 bf16 ulp, every
    other byte untouched."""
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want).reshape(-1)
    s = np.asarray(slots, np.int64)
    s = np.unique(s[(s >= 0) & (s < num_slots)])
    mask = np.zeros(got.size, bool)
    mask[(s[:, None] * 1024 + np.arange(1024)[None, :]).ravel()] = True
    out = {"cache_exact_mismatch": int(np.count_nonzero(got[~mask] != want[~mask]))}
    g16 = got[mask].view(np.uint16)
    w16 = want[mask].view(np.uint16)
    d = np.abs(bf16_ord(g16) - bf16_ord(w16))
    out["rope_max_ulp"] = int(d.max()) if d.size else 0      # all 512 values are bf16 here
    out["rope_inexact"] = int(np.count_nonzero(d))
    out["code_max_step"] = 0
    out["code_inexact"] = 0
    out["cache_bytes_differ"] = int(np.count_nonzero(got != want))
    return out


def run_and_compare(w, inp, *, q_weight=True, chunk_tokens=4096, kv_store=0, **cfg):
    """Run the HIP operator on the GPU-made inputs ``inp`` and check every
    token against the oracle.  The inputs stay untouched (q and the cache are
    cloned on the device first)."""
    from fp8_kv_cache_amd.qkv_prep import QkvPrep

    T, H = w.num_tokens, w.num_heads
    q_w = inp["q_w"] if q_weight else None
    q_run = inp["q"].clone()
    if kv_store == 0:
        cache_run = inp["cache"].clone()
    else:
        cache_run = torch.randint(0, 256, (w.num_blocks, w.block_size * 1024), dtype=torch.uint8,
                                  device=q_run.device, generator=torch.Generator(
                                      device=q_run.device).manual_seed(w.seed + 77))
    torch.cuda.synchronize()
    want_cache = cache_run.cpu().numpy().copy()      # the poison, before the launch
    op = QkvPrep(H, device=q_run.device.index or 0, block_size=w.block_size, eps=w.eps,
                 kv_store=kv_store, **cfg)
    op(q_run, inp["kv"], q_w, inp["kv_w"], inp["positions"], inp["cos_sin"],
       inp["slot_mapping"], cache_run)
    torch.cuda.synchronize()

    pos = inp["positions"].cpu().numpy()
    slots = inp["slot_mapping"].cpu().numpy()
    cs = inp["cos_sin"].cpu().numpy()
    kvh = W.as_u16(inp["kv"])
    qw = None if q_w is None else W.as_u16(q_w)
    kvw = W.as_u16(inp["kv_w"])
    res = {"q_max_ulp": 0, "q_inexact": 0, "tokens": T}
    nth = oracle_threads()
    for t0 in range(0, T, chunk_tokens):
        t1 = min(T, t0 + chunk_tokens)
        qb = W.as_u16(inp["q"][t0:t1])
        qa = W.as_u16(q_run[t0:t1])
        want = oracle.qkv_prep(qb, kvh[t0:t1], qw, kvw, pos[t0:t1], cs, slots[t0:t1], want_cache,
                               w.num_blocks, w.block_size, w.eps, nth,
                               kv_store="fp8" if kv_store == 0 else "bf16")
        d = np.abs(bf16_ord(qa) - bf16_ord(want))
        res["q_max_ulp"] = max(res["q_max_ulp"], int(d.max()) if d.size else 0)
        res["q_inexact"] += int(np.count_nonzero(d))
    if kv_store == 0:
        roles = byte_roles(slots, w.num_blocks, w.block_size)
        res.update(compare_cache(cache_run.cpu().numpy(), want_cache, roles))
    else:
        res.update(compare_bf16_cache(cache_run.cpu().numpy(), want_cache, slots,
                                      w.num_blocks * w.block_size))
    res["valid_slots"] = int(((slots >= 0) & (slots < w.num_blocks * w.block_size)).sum())
    return res


def tiny_weights(seed, lo, hi, device):
    """bf16 weights of magnitude 2^lo .. 2^(hi+1), random signs (bf16
    subnormals included below 2^-126): they drive y down to ~1e-38, so kv
    blocks reach the exponent clamp (scale byte 0) with non-zero codes and q
    outputs become subnormal."""
    g = torch.Generator().manual_seed(seed)
    e = torch.randint(lo, hi, (512,), generator=g).float()
    sign = torch.where(torch.rand(512, generator=g) < 0.5, -1.0, 1.0)
    return (sign * torch.exp2(e) * (1 + torch.rand(512, generator=g))).to(torch.bfloat16).to(device)


def assert_within_bar(res):
    assert res["cache_exact_mismatch"] == 0, res
    assert res["q_max_ulp"] <= 1, res
    assert res["rope_max_ulp"] <= 1, res
    assert res["code_max_step"] <= 1, res


def assert_bit_exact(res):
    assert_within_bar(res)
    assert res["q_inexact"] == 0 and res["cache_bytes_differ"] == 0, res
