"""Seeded synthetic inputs for the q/kv prep operator.

This module only draws inputs: it holds none of the operator's arithmetic
(no norm, rotation, rounding rule or quantizer).  Both the GPU path's tests and
the CPU oracle's tests take their inputs from here, so it is the one module the
two sides share.

Workloads (tokens x q heads, head_dim 512 = 448 nope + 64 rope):

  tiny          16 x 8      positions uniform in [0, 4096), cache 4 x 64 slots,
                            16 distinct slots of a random permutation, 2 set to -1
  decode        2048 x 64   positions uniform in [0, 131072), 1% of q rows and of
                            kv rows scaled by 100, cache 4096 x 64, random
                            distinct slots
  prefill       32768 x 64  8 sequences of positions 0..4095, cache 1024 x 64,
                            each sequence owns 64 random blocks, filled in order
  prefill_wide  32768 x 128 positions 0..32767, cache 1024 x 64, one random block
                            per 64-token group
  long          131072 x 128 positions 0..131071, cache 2048 x 64, a random
                            permutation of all blocks, one per 64-token group

q and kv are bf16 ~ N(0, 1); the norm weights are bf16(1 + 0.1 N(0, 1));
eps = 1e-6; RoPE base 10000 with the cos/sin table built in float64 and stored
as float32 [max_position, 64] (32 cos then 32 sin per row).  The cache starts
as seeded random bytes ("poison") so that a slot written by mistake, or one
that should have been written and was not, shows up byte for byte.

Draws use torch's seeded generator on the device the tensors are made on, in
fixed token chunks, so a case is reproducible on a given device type.  CPU and
GPU draws differ; a test that checks the GPU against the oracle copies the
GPU-made inputs to the host.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

HEAD_DIM = 512
ROPE_DIM = 64
SLOT_BYTES = 584
GEN_CHUNK_TOKENS = 2048


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_tokens: int
    num_heads: int
    max_position: int
    num_blocks: int
    block_size: int
    positions: str          # "uniform" | "sequences" | "arange"
    slots: str              # "subset" | "unique" | "seq_blocks" | "group_blocks"
    seed: int
    num_seqs: int = 1
    outlier_frac: float = 0.0
    num_skip: int = 0
    eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def label(self) -> str:
        return "%s %dx%d" % (self.name, self.num_tokens, self.num_heads)


WORKLOADS = {
    "tiny": Workload("tiny", 16, 8, 4096, 4, 64, "uniform", "subset", 1001, num_skip=2),
    "decode": Workload("decode", 2048, 64, 131072, 4096, 64, "uniform", "unique", 1002,
                       outlier_frac=0.01),
    "prefill": Workload("prefill", 32768, 64, 4096, 1024, 64, "sequences", "seq_blocks", 1003,
                        num_seqs=8),
    "prefill_wide": Workload("prefill_wide", 32768, 128, 32768, 1024, 64, "arange",
                             "group_blocks", 1004),
    "long": Workload("long", 131072, 128, 131072, 2048, 64, "arange", "group_blocks", 1005),
}


def custom(num_tokens, num_heads, *, seed=7, max_position=4096, block_size=64,
           num_blocks=None, num_skip=0, positions="uniform", slots="unique",
           outlier_frac=0.0, eps=1e-6) -> Workload:
    """A workload of any size, for edge-case and ragged-shape tests."""
    if num_blocks is None:
        num_blocks = max(1, -(-max(num_tokens, 1) // block_size) * 2)
    return Workload("custom", num_tokens, num_heads, max_position, num_blocks, block_size,
                    positions, slots, seed, outlier_frac=outlier_frac, num_skip=num_skip,
                    eps=eps)


def rope_table(max_position: int, base: float = 10000.0) -> np.ndarray:
    """cos/sin table [max_position, 64] fp32: angle(p, i) = p * base^(-2i/64)."""
    i = np.arange(ROPE_DIM // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / ROPE_DIM)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _bf16_rows(shape_tail, num_tokens, device, g, outlier_frac):
    """N(0,1) bf16 of shape [num_tokens, *shape_tail], drawn in token chunks."""
    out = torch.empty((num_tokens,) + tuple(shape_tail), dtype=torch.bfloat16, device=device)
    for t0 in range(0, num_tokens, GEN_CHUNK_TOKENS):
        t1 = min(num_tokens, t0 + GEN_CHUNK_TOKENS)
        x = torch.randn((t1 - t0,) + tuple(shape_tail), generator=g, device=device,
                        dtype=torch.float32)
        if outlier_frac > 0.0:
            row_shape = (t1 - t0,) + tuple(shape_tail[:-1]) + (1,)
            hit = torch.rand(row_shape, generator=g, device=device) < outlier_frac
            x = torch.where(hit, x * 100.0, x)
        out[t0:t1] = x.to(torch.bfloat16)
        del x
    return out


def _positions(w: Workload, device, g):
    T = w.num_tokens
    if w.positions == "uniform":
        return torch.randint(0, w.max_position, (T,), generator=g, device=device,
                             dtype=torch.int64)
    if w.positions == "arange":
        return torch.arange(T, device=device, dtype=torch.int64) % w.max_position
    if w.positions == "sequences":
        per = T // w.num_seqs
        return (torch.arange(T, device=device, dtype=torch.int64) % per) % w.max_position
    raise ValueError(w.positions)


def _slots(w: Workload, device, g):
    T, B, NB = w.num_tokens, w.block_size, w.num_blocks
    cap = NB * B
    if w.slots in ("subset", "unique"):
        if T > cap:
            raise ValueError("more tokens than cache slots")
        s = torch.randperm(cap, generator=g, device=device)[:T].to(torch.int64)
    elif w.slots == "seq_blocks":
        per = T // w.num_seqs
        nblk_seq = -(-per // B)
        blocks = torch.randperm(NB, generator=g, device=device)[: nblk_seq * w.num_seqs]
        j = torch.arange(T, device=device) % per
        seq = torch.arange(T, device=device) // per
        s = (blocks[seq * nblk_seq + j // B] * B + j % B).to(torch.int64)
    elif w.slots == "group_blocks":
        ngroups = -(-T // B)
        if ngroups > NB:
            raise ValueError("more 64-token groups than cache blocks")
        blocks = torch.randperm(NB, generator=g, device=device)[:ngroups]
        t = torch.arange(T, device=device)
        s = (blocks[t // B] * B + t % B).to(torch.int64)
    else:
        raise ValueError(w.slots)
    if w.num_skip:
        k = torch.randperm(T, generator=g, device=device)[: w.num_skip]
        s[k] = -1
    return s


def make_inputs(w: Workload, device="cpu", *, seed=None, q_weight=True):
    """Draw every operator input for workload ``w`` on ``device``.

    Returns a dict: q [T,H,512] bf16, kv [T,512] bf16, q_w/kv_w [512] bf16
    (q_w None when q_weight is False), positions [T] int64, cos_sin
    [max_position,64] fp32, slot_mapping [T] int64, cache [NB, B*584] uint8,
    plus the scalars num_blocks, block_size, eps."""
    seed = w.seed if seed is None else seed
    g = _gen(device, seed)
    T, H = w.num_tokens, w.num_heads
    q = _bf16_rows((H, HEAD_DIM), T, device, g, w.outlier_frac)
    kv = _bf16_rows((HEAD_DIM,), T, device, g, w.outlier_frac)
    q_w = (1.0 + 0.1 * torch.randn(HEAD_DIM, generator=g, device=device)).to(torch.bfloat16)
    kv_w = (1.0 + 0.1 * torch.randn(HEAD_DIM, generator=g, device=device)).to(torch.bfloat16)
    positions = _positions(w, device, g)
    slots = _slots(w, device, g) if T > 0 else torch.empty(0, dtype=torch.int64, device=device)
    cos_sin = torch.from_numpy(rope_table(w.max_position, w.rope_base)).to(device)
    cache = torch.randint(0, 256, (w.num_blocks, w.block_size * SLOT_BYTES), generator=g,
                          device=device, dtype=torch.uint8)
    return dict(q=q, kv=kv, q_w=q_w if q_weight else None, kv_w=kv_w, positions=positions,
                cos_sin=cos_sin, slot_mapping=slots, cache=cache, num_blocks=w.num_blocks,
                block_size=w.block_size, eps=w.eps)


def algorithmic_bytes(num_tokens: int, num_heads: int, num_valid_slots: int,
                      slot_bytes: int = SLOT_BYTES) -> int:
    """Bytes the operator must move once: q read and written (2 x 1 KiB per head),
    the kv row read (1 KiB), position and slot read (16 B), the token's cos/sin
    row read (256 B), the slot written for each valid slot (584 bytes in the
    FP8 cache, 1024 in the bf16 one), and the two 512-entry bf16 weights read
    once (2 KiB)."""
    return (num_tokens * (2048 * num_heads + 1024 + 16 + 256)
            + slot_bytes * num_valid_slots + 2048)


def gather_bytes(num_rows: int, num_valid: int, out_bytes_per_value: int) -> int:
    """Bytes the cache reader must move: the 8-byte slot index per row, the
    584-byte slot of each valid row, and the 512-value output row."""
    return num_rows * (8 + 512 * out_bytes_per_value) + SLOT_BYTES * num_valid


def as_u16(t: torch.Tensor) -> np.ndarray:
    """A bf16 tensor's bit patterns as a host uint16 array."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
