"""Measured launch targets: the operator on a workload, and the neighbouring
paths (the bf16-store cache mode, the cache reader, the MXFP8 norm-quant
operator) on fixed synthetic inputs.

Each target names the kernel that runs, the sources that define it (their hash
marks a counter summary as current), its workload label and the bytes one
launch must move (read and written), so that bench.py times it and
rocprof_harness.py profiles it with the same inputs and the same byte count.
Inputs are drawn with torch's seeded generators on the GPU; none of the
operators' arithmetic is here.
"""
from __future__ import annotations

import dataclasses
from typing import Callable

from fp8_kv_cache_amd import workloads as W

# Sources per kernel family (file names under csrc/).
SOURCES = {
    "op": ("qkv_prep_kernels.hip", "qkv_prep_launch.h", "qkvp_device.h", "qkv_prep_internal.h"),
    "gather": ("qkv_prep_gather.hip", "qkv_prep_gather.h", "qkvp_device.h", "qkv_prep_internal.h"),
    "mxfp8": ("mxfp8_norm_quant.hip", "mxfp8_launch.h", "qkvp_device.h", "qkv_prep_internal.h"),
}
KERNELS = {"op": "qkv_prep_kernel", "gather": "gather_kernel", "mxfp8": "mxfp8_kernel"}
PREFIX = {"op": "qkv_prep", "gather": "qkv_prep_gather", "mxfp8": "mxfp8_norm_quant"}

# The reader reads every slot of the Decode-like cache (4096 blocks x 64),
# either as a block-table walk (blocks in a random order, each block's slots in
# order: how attention reads a sequence) or, for the "_shuffled" targets, every
# slot in a random order.
GATHER_WORKLOAD = "decode"
MX_ROWS, MX_HIDDEN = 16384, 7168


@dataclasses.dataclass(frozen=True)
class Target:
    name: str
    family: str           # key of SOURCES / KERNELS / PREFIX
    label: str            # workload label used in profile file names
    read_bytes: int
    write_bytes: int

    @property
    def kernel(self) -> str:
        return KERNELS[self.family]

    @property
    def prefix(self) -> str:
        return PREFIX[self.family]

    @property
    def alg_bytes(self) -> int:
        return self.read_bytes + self.write_bytes


def _op_bytes(w, slot_bytes):
    valid = w.num_tokens - w.num_skip
    read = w.num_tokens * (1024 * w.num_heads + 1024 + 16 + 256) + 2048
    write = w.num_tokens * 1024 * w.num_heads + slot_bytes * valid
    return read, write


def mxfp8_scale_bytes(m: int, hidden: int) -> int:
    """Size of the swizzled scale buffer: rows padded to 128, scale columns
    (hidden / 32) padded to 4."""
    return ((m + 127) // 128 * 128) * ((hidden // 32 + 3) // 4 * 4)


VARIANTS = ("bf16store_prefill", "gather_bf16", "gather_f32", "gather_f32_shuffled", "mxfp8")


def target(name: str) -> Target:
    if name in W.WORKLOADS:
        w = W.WORKLOADS[name]
        r, wr = _op_bytes(w, W.SLOT_BYTES)
        return Target(name, "op", "%s_%dx%d" % (w.name, w.num_tokens, w.num_heads), r, wr)
    if name == "bf16store_prefill":
        w = W.WORKLOADS["prefill"]
        r, wr = _op_bytes(w, 1024)
        return Target(name, "op", "bf16store_prefill_%dx%d" % (w.num_tokens, w.num_heads), r, wr)
    if name in ("gather_bf16", "gather_f32", "gather_bf16_shuffled", "gather_f32_shuffled"):
        w = W.WORKLOADS[GATHER_WORKLOAD]
        n = w.num_blocks * w.block_size
        per = 2 if name.startswith("gather_bf16") else 4
        return Target(name, "gather", "%s_%d" % (name, n), n * (8 + W.SLOT_BYTES), n * 512 * per)
    if name == "mxfp8":
        m, h = MX_ROWS, MX_HIDDEN
        return Target(name, "mxfp8", "mxfp8_%dx%d_residual" % (m, h), 2 * m * h * 2 + 2 * h,
                      m * h * 2 + m * h + mxfp8_scale_bytes(m, h))
    raise KeyError(name)


def setup(t: Target, torch, qp) -> Callable[[], None]:
    """Allocate and draw the target's inputs on the current GPU; return a
    prepared launch (a zero-argument callable, checked once) that enqueues
    one launch on the current stream.  It holds the tensors; drop it to free
    them."""
    if t.family == "op":
        w = W.WORKLOADS["prefill" if t.name == "bf16store_prefill" else t.name]
        inp = W.make_inputs(w, device="cuda")
        if t.name == "bf16store_prefill":
            cache = torch.zeros((w.num_blocks, w.block_size * 1024), dtype=torch.uint8, device="cuda")
            op = qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps, kv_store=qp.KV_BF16)
        else:
            cache = inp["cache"]
            op = qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps)
        return op.prepare(inp["q"], inp["kv"], inp["q_w"], inp["kv_w"], inp["positions"],
                          inp["cos_sin"], inp["slot_mapping"], cache)
    if t.family == "gather":
        w = W.WORKLOADS[GATHER_WORKLOAD]
        cap = w.num_blocks * w.block_size
        gen = torch.Generator(device="cuda").manual_seed(78)
        cache = torch.randint(0, 256, (w.num_blocks, w.block_size * W.SLOT_BYTES), dtype=torch.uint8,
                              device="cuda", generator=gen)
        cache[:, w.block_size * 576:].zero_()           # scale bytes 0: finite values
        if t.name.endswith("_shuffled"):
            # every slot in a random order: the worst case for the cache lines
            slots = torch.randperm(cap, device="cuda", generator=gen).to(torch.int64)
        else:
            # a block-table walk: blocks in a random order, each block's slots in order
            blocks = torch.randperm(w.num_blocks, device="cuda", generator=gen).to(torch.int64)
            slots = (blocks[:, None] * w.block_size +
                     torch.arange(w.block_size, device="cuda", dtype=torch.int64)[None, :]).reshape(-1)
        dtype = torch.bfloat16 if t.name.startswith("gather_bf16") else torch.float32
        rows = torch.empty((cap, 512), dtype=dtype, device="cuda")
        op = qp.QkvPrep(w.num_heads, block_size=w.block_size, eps=w.eps)
        return op.prepare_gather(cache, slots, rows)
    if t.family == "mxfp8":
        m, h = MX_ROWS, MX_HIDDEN
        gen = torch.Generator(device="cuda").manual_seed(77)
        x = torch.randn((m, h), generator=gen, device="cuda").to(torch.bfloat16)
        r = torch.randn((m, h), generator=gen, device="cuda").to(torch.bfloat16)
        gamma = (0.1 * torch.randn(h, generator=gen, device="cuda")).to(torch.bfloat16)
        res_out = torch.empty_like(x)
        codes = torch.empty((m, h), dtype=torch.uint8, device="cuda")
        scales = torch.empty(mxfp8_scale_bytes(m, h), dtype=torch.uint8, device="cuda")
        return qp.prepare_mxfp8_norm_quant(x, gamma, 1e-6, residual=r, residual_out=res_out,
                                           quant_out=codes, scale_out=scales)
    raise KeyError(t.family)
