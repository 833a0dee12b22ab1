"""Seeded synthetic decode workloads for the paged KV cache.

This module only draws inputs. It holds none of the attention or write arithmetic, so both
the HIP path and the CPU oracle can be fed from it without sharing any computation.

The shapes follow the decode sweeps of "vLLM-Style Llama Inference Engine with Tensor
Parallelism" (Benchmarks table: batch x sequence points, Llama 3.2 1B/3B attention with
grouped-query heads) and the long-context / ragged batches of a continuous-batching step
(mini-vLLM README, paged KV-cache paragraph: a fixed pool of physical blocks, each holding
block_size token slots, with a per-sequence block table).

Recipe, per workload (one ``torch.Generator`` seeded with the workload's seed, draws taken
in this fixed order):
  1. a random permutation of the NB physical block ids;
  2. the context lengths (fixed, or uniform integers in [1, max_len]);
  3. q      ~ N(0,1) * q_std, rounded to bf16 (round-to-nearest-even);
  4. pool K ~ N(0,1) bf16, shape [NB, block_size, Hkv, D];
  5. pool V ~ N(0,1) bf16, same shape;
  6. new k  ~ N(0,1) bf16, shape [T, Hkv, D];
  7. new v  ~ N(0,1) bf16, same shape.
Sequence b receives the next ceil(L_b / block_size) ids of the permutation as its block table
(table entries past the end are -1). Each sequence decodes one new token: it is written at
logical position L_b - 1, i.e. slot = table[b, (L_b-1)//bs] * bs + (L_b-1) % bs, and the
attention then reads all L_b positions.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

BF16_QNAN_BITS = 0x7FC0  # a quiet-NaN bit pattern, used to poison memory that must never be read


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int          # NB, physical blocks in the pool
    max_blocks: int          # MB, block-table width
    seed: int
    context_len: Optional[int] = None    # fixed length for every sequence, or
    max_context_len: Optional[int] = None  # uniform integer lengths in [1, max_context_len]
    q_std: float = 1.0
    description: str = ""

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The five decode workloads (the fifth is two calls: 64 x 8192 and 2 x 32768).
WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", batch=1, num_q_heads=32, num_kv_heads=8, head_dim=64, block_size=16,
                   num_blocks=64, max_blocks=8, seed=1001, context_len=128,
                   description="batch 1 x context 128, 32q:8kv, D=64, pool 64 blocks"),
    "c2": Workload("c2", batch=4, num_q_heads=24, num_kv_heads=8, head_dim=128, block_size=16,
                   num_blocks=512, max_blocks=32, seed=1002, context_len=512,
                   description="batch 4 x context 512, 24q:8kv, D=128, pool 512 blocks"),
    "c3": Workload("c3", batch=16, num_q_heads=32, num_kv_heads=8, head_dim=64, block_size=16,
                   num_blocks=4096, max_blocks=128, seed=1003, context_len=2048,
                   description="batch 16 x context 2048, 32q:8kv, D=64, pool 4096 blocks"),
    "c4": Workload("c4", batch=48, num_q_heads=24, num_kv_heads=8, head_dim=128, block_size=16,
                   num_blocks=16384, max_blocks=256, seed=1004, max_context_len=4096,
                   description="ragged batch 48, context U{1..4096}, 24q:8kv, D=128, "
                               "pool 16384 blocks"),
    "c5a": Workload("c5a", batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                    block_size=16, num_blocks=32768, max_blocks=512, seed=1005,
                    context_len=8192, q_std=3.0,
                    description="batch 64 x context 8192, 32q:8kv, D=128, logits std ~3"),
    "c5b": Workload("c5b", batch=2, num_q_heads=32, num_kv_heads=8, head_dim=128,
                    block_size=16, num_blocks=4096, max_blocks=2048, seed=1006,
                    context_len=32768, q_std=3.0,
                    description="batch 2 x context 32768, 32q:8kv, D=128, logits std ~3"),
}


INPUT_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


def _bf16_normal(shape, gen: torch.Generator, device, std: float = 1.0,
                 dtype: str = "bf16") -> torch.Tensor:
    """Normal draws in fp32, rounded (nearest-even) to the 16-bit input format."""
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(INPUT_DTYPES[dtype])


def make_inputs(w: Workload, device: str = "cpu", poison: bool = False,
                lengths: Optional[list] = None, dtype: str = "bf16") -> Dict[str, object]:
    """Draw one decode step's inputs for workload ``w``.

    device: where the random numbers are drawn ("cpu" gives the canonical inputs; "cuda"
            draws on the GPU with a GPU generator of the same seed, a different stream of
            numbers of the same distribution, used for the largest pools).
    poison: overwrite every pool slot that attention must never read (unreferenced blocks
            and the stale slots after position L_b - 1 in a sequence's last block) with a
            quiet-NaN bit pattern.
    lengths: optional explicit per-sequence context lengths (overrides the workload's).
    dtype:  format of q, the pools and the new rows: "bf16" or "f16" (the same fp32 draws,
            rounded to that format).
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    B, bs, NB, MB = w.batch, w.block_size, w.num_blocks, w.max_blocks
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim

    perm = torch.randperm(NB, generator=gen, device=device).to("cpu")
    if lengths is not None:
        ctx = torch.tensor(lengths, dtype=torch.int32)
        assert ctx.numel() == B
    elif w.context_len is not None:
        ctx = torch.full((B,), w.context_len, dtype=torch.int32)
    else:
        ctx = torch.randint(1, w.max_context_len + 1, (B,), generator=gen,
                            device=device).to("cpu", torch.int32)
    nblk = [(int(L) + bs - 1) // bs for L in ctx.tolist()]
    if sum(nblk) > NB or max(nblk) > MB:
        raise ValueError(f"{w.name}: lengths need {sum(nblk)} blocks (pool {NB}), "
                         f"max {max(nblk)} per sequence (table width {MB})")
    tables = torch.full((B, MB), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n

    q = _bf16_normal((B, Hq, D), gen, device, w.q_std, dtype)
    k_cache = _bf16_normal((NB, bs, Hkv, D), gen, device, dtype=dtype)
    v_cache = _bf16_normal((NB, bs, Hkv, D), gen, device, dtype=dtype)
    k_new = _bf16_normal((B, Hkv, D), gen, device, dtype=dtype)
    v_new = _bf16_normal((B, Hkv, D), gen, device, dtype=dtype)

    slots = torch.empty(B, dtype=torch.int64)
    for b, L in enumerate(ctx.tolist()):
        if L == 0:
            slots[b] = -1
        else:
            slots[b] = int(tables[b, (L - 1) // bs]) * bs + (L - 1) % bs

    if poison:
        poison_unread_slots(k_cache, v_cache, tables, ctx, bs)

    dev = torch.device(device)
    return {
        "workload": w,
        "q": q,
        "k_cache": k_cache,
        "v_cache": v_cache,
        "block_tables": tables.to(dev),
        "context_lens": ctx.to(dev),
        "k_new": k_new,
        "v_new": v_new,
        "slot_mapping": slots.to(dev),
        "scale": w.scale,
        "dtype": dtype,
    }


def poison_unread_slots(k_cache: torch.Tensor, v_cache: torch.Tensor, tables: torch.Tensor,
                        ctx: torch.Tensor, bs: int) -> None:
    """Write quiet-NaN bits into every slot no sequence reads (in place)."""
    NB = k_cache.shape[0]
    used = torch.zeros(NB, dtype=torch.bool)
    tail = []  # (block id, first stale offset)
    for b, L in enumerate(ctx.tolist()):
        n = (L + bs - 1) // bs
        if n:
            ids = tables[b, :n].to(torch.int64)
            used[ids] = True
            if L % bs:
                tail.append((int(tables[b, n - 1]), L % bs))
    unused = (~used).nonzero().flatten().to(k_cache.device)
    for c in (k_cache, v_cache):
        bits = c.view(torch.int16)
        bits[unused] = BF16_QNAN_BITS
        for blk, off in tail:
            bits[blk, off:] = BF16_QNAN_BITS


def to_bits(t: torch.Tensor) -> np.ndarray:
    """16-bit float tensor -> numpy uint16 array of its raw bit patterns (host copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def to_host_numpy(inp: Dict[str, object]) -> Dict[str, object]:
    """Host numpy views of an input dict: bf16 as uint16 bits, indices as integers."""
    out = {"workload": inp["workload"], "scale": inp["scale"], "dtype": inp.get("dtype", "bf16")}
    for key in ("q", "k_cache", "v_cache", "k_new", "v_new"):
        out[key] = to_bits(inp[key])
    for key in ("block_tables", "context_lens", "slot_mapping", "cu_seqlens_q"):
        if key in inp:
            out[key] = inp[key].detach().to("cpu").numpy()
    return out


def algorithmic_bytes(w: Workload, context_lens, out_bytes: int = 4) -> Dict[str, int]:
    """Bytes the decode step must move at minimum: K and V of every context token (16-bit),
    q (16-bit) and out (out_bytes per element: 4 for fp32, 2 for a 16-bit output); the write
    moves T rows of K and V in and out."""
    total_tokens = int(sum(int(x) for x in context_lens))
    Hq, Hkv, D, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.batch
    kv = total_tokens * Hkv * D * 2 * 2
    q = B * Hq * D * 2
    o = B * Hq * D * out_bytes
    write = B * Hkv * D * 2 * 2 * 2
    return {"kv": kv, "q": q, "out": o, "attention": kv + q + o, "write": write,
            "tokens": total_tokens}


# --------------------------------------------------------------------------------------------
# Multi-query (prefill / chunked prefill) workloads. Sequence b has a cached prefix of
# L_b - Q_b tokens and appends a chunk of Q_b new tokens (Q_b = L_b: full prefill or
# recompute). Recipe (one torch.Generator per workload, draws in this order): block-id
# permutation, q [T, Hq, D] * q_std, pool K, pool V, new k [T, Hkv, D], new v; T = sum Q_b.
# The new tokens occupy positions L_b - Q_b .. L_b - 1, so token i of sequence b goes to
# slot table[b][p // bs] * bs + p % bs with p = L_b - Q_b + i.
# --------------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks: int
    seed: int
    context_lens: tuple
    query_lens: tuple
    q_std: float = 1.0
    description: str = ""

    @property
    def batch(self) -> int:
        return len(self.context_lens)

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


PREFILL_WORKLOADS: Dict[str, PrefillWorkload] = {
    "p1": PrefillWorkload("p1", num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                          num_blocks=2048, max_blocks=256, seed=2001,
                          context_lens=(4096,) * 8, query_lens=(512,) * 8,
                          description="chunked prefill: 8 sequences, 3584 cached + 512 new "
                                      "tokens each, 32q:8kv, D=128"),
    "p2": PrefillWorkload("p2", num_q_heads=24, num_kv_heads=8, head_dim=128, block_size=16,
                          num_blocks=600, max_blocks=256, seed=2002,
                          context_lens=(1, 17, 300, 1000, 2048, 4000),
                          query_lens=(1, 17, 64, 1000, 256, 100),
                          description="ragged mix of full prefills and chunks, 24q:8kv, D=128"),
    "p3": PrefillWorkload("p3", num_q_heads=32, num_kv_heads=8, head_dim=64, block_size=16,
                          num_blocks=300, max_blocks=128, seed=2003,
                          context_lens=(2048, 2048), query_lens=(2048, 2048),
                          description="full prefill (recompute) of 2 x 2048 tokens, 32q:8kv, "
                                      "D=64"),
}


def make_prefill_inputs(w: PrefillWorkload, device: str = "cpu", poison: bool = False,
                        dtype: str = "bf16") -> Dict[str, object]:
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    B, bs, NB, MB = w.batch, w.block_size, w.num_blocks, w.max_blocks
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    ctx = torch.tensor(w.context_lens, dtype=torch.int32)
    ql = torch.tensor(w.query_lens, dtype=torch.int32)
    if (ql > ctx).any() or (ql < 0).any():
        raise ValueError("query lengths must be within [0, context length]")
    perm = torch.randperm(NB, generator=gen, device=device).to("cpu")
    nblk = [(int(L) + bs - 1) // bs for L in ctx.tolist()]
    if sum(nblk) > NB or max(nblk) > MB:
        raise ValueError(f"{w.name}: lengths need {sum(nblk)} blocks (pool {NB})")
    tables = torch.full((B, MB), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
    T = int(ql.sum())
    q = _bf16_normal((T, Hq, D), gen, device, w.q_std, dtype)
    k_cache = _bf16_normal((NB, bs, Hkv, D), gen, device, dtype=dtype)
    v_cache = _bf16_normal((NB, bs, Hkv, D), gen, device, dtype=dtype)
    k_new = _bf16_normal((T, Hkv, D), gen, device, dtype=dtype)
    v_new = _bf16_normal((T, Hkv, D), gen, device, dtype=dtype)
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(ql, 0)
    slots = torch.empty(T, dtype=torch.int64)
    for b in range(B):
        L, Q = int(ctx[b]), int(ql[b])
        for i in range(Q):
            p = L - Q + i
            slots[int(cu[b]) + i] = int(tables[b, p // bs]) * bs + p % bs
    if poison:
        poison_unread_slots(k_cache, v_cache, tables, ctx, bs)
    dev = torch.device(device)
    return {"workload": w, "q": q, "k_cache": k_cache, "v_cache": v_cache,
            "block_tables": tables.to(dev), "context_lens": ctx.to(dev),
            "cu_seqlens_q": cu.to(dev), "k_new": k_new, "v_new": v_new,
            "slot_mapping": slots.to(dev), "scale": w.scale,
            "max_q_len": int(ql.max()) if B else 0, "dtype": dtype}


def prefill_algorithmic(w: PrefillWorkload) -> Dict[str, int]:
    """Useful work of one multi-query call: flops of q.K and p.V over the causal keys of
    every query row (4 * (p+1) * D per row and query head), and bytes of K/V of every cached
    position read once, q (bf16) and out (fp32)."""
    flops = 0
    for L, Q in zip(w.context_lens, w.query_lens):
        keys = sum(L - Q + i + 1 for i in range(Q))
        flops += 4 * keys * w.head_dim * w.num_q_heads
    T = sum(w.query_lens)
    kv = sum(w.context_lens) * w.num_kv_heads * w.head_dim * 2 * 2
    return {"flops": flops, "kv": kv, "q": T * w.num_q_heads * w.head_dim * 2,
            "out": T * w.num_q_heads * w.head_dim * 4,
            "bytes": kv + T * w.num_q_heads * w.head_dim * 6}
