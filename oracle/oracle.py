"""Plain, slow CPU oracle for paged KV decode attention and the slot-mapping KV write.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the benchmark's CPU
baseline leg may import this module. The product path (the HIP kernels behind the C ABI)
never calls it, and it imports nothing from that path.

What it computes, and where the pages state it:
  * KV write: each new token's K and V row goes to its slot in a pool of physical blocks
    ("vLLM-Style Llama Inference Engine with Tensor Parallelism", Features and scope /
    Implemented: paged KV caching with block tables and slot mappings; How it works, step 3:
    each rank writes to its paged KV cache; mini-vLLM README, benchmarks/baseline_hf.py
    discussion: the per-sequence loop that writes K/V into the block pool).
  * Decode attention: one query token per sequence attends to every cached key of that
    sequence, gathered through its block table (mini-vLLM README, paged KV-cache paragraph:
    the block table maps logical positions to physical storage; llm-stack, Serving engine /
    KV cache bullet: a decode query sees all cached keys, no causal mask), with grouped-query
    heads (vLLM-Style Llama engine, Implemented: grouped-query attention), bf16 inputs and
    softmax(q K^T * scale) V ("tiny-vLLM" blog, The Precision Trade-off: BF16; llm-stack,
    Attention kernel).

The method reaches exactly (up to rounding order) the plain definition of softmax
attention, so this oracle is that definition written out in float64 on the bf16 input
values. Readings taken where the pages are silent:
  * cache layout [num_blocks, block_size, num_kv_heads, head_dim]; slot = block*bs + offset;
  * query head h uses KV head h // (Hq / Hkv) (consecutive grouping);
  * a negative slot means "no write"; duplicate non-negative slots are a caller error;
  * context length 0 gives an all-zero output row;
  * the fp32 scale a GPU receives is applied to the fp64 dot product.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------------------
# bf16 decoding ("tiny-vLLM" blog, The Precision Trade-off: BF16 -- 8 exponent bits as in
# float32, 7 fraction bits; a bf16 value is the top half of a float32 bit pattern).
# ---------------------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return as_f32.astype(np.float64)


# ---------------------------------------------------------------------------------------
# fp16 decoding (IEEE 754 binary16: sign bit, 5 exponent bits with bias 15, 10 fraction
# bits; exponent field 0 holds zero and the subnormals, 31 holds infinity and NaN). The
# fp16-input variant of the path reads its q and caches in this format: the mini-vLLM
# serving results were measured with an fp16 model (mini-vLLM README, Results, hardware
# line), and the "tiny-vLLM" blog (The Precision Trade-off: BF16) sets fp16's narrower
# exponent against bf16's.
# ---------------------------------------------------------------------------------------
def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of binary16 bit patterns (uint16) to float64, from the field layout."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + f / 1024.0, e - 15)
    subnormal = np.ldexp(f / 1024.0, -14)
    val = np.where(e == 0, subnormal, normal)
    val = np.where(e == 31, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


INPUT_DTYPES = ("bf16", "f16")


def decode_bits(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Exact float64 values of 16-bit input bit patterns of the given format."""
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    raise ValueError(f"unknown input format {dtype!r} (expected one of {INPUT_DTYPES})")


# ---------------------------------------------------------------------------------------
# KV write (slot-mapping scatter), on raw bit patterns: no float conversion, so every
# payload, NaN included, lands unchanged.
# ---------------------------------------------------------------------------------------
def kv_write(k_bits: np.ndarray, v_bits: np.ndarray, slot_mapping: np.ndarray,
             k_cache_bits: np.ndarray, v_cache_bits: np.ndarray
             ) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the two pools with token t's K/V rows stored at slot_mapping[t].

    k_bits, v_bits: uint16 [T, Hkv, D]; slot_mapping: int [T]; caches: uint16
    [NB, bs, Hkv, D]. Slot s addresses block s // bs, offset s % bs.
    """
    NB, bs, Hkv, D = k_cache_bits.shape
    kc = np.array(k_cache_bits, dtype=np.uint16, copy=True).reshape(NB * bs, Hkv, D)
    vc = np.array(v_cache_bits, dtype=np.uint16, copy=True).reshape(NB * bs, Hkv, D)
    seen = set()
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue  # padding token: nothing to write
        if s >= NB * bs:
            raise ValueError(f"slot {s} of token {t} is outside the pool ({NB * bs} slots)")
        if s in seen:
            raise ValueError(f"slot {s} is written twice")
        seen.add(s)
        kc[s] = k_bits[t]
        vc[s] = v_bits[t]
    return kc.reshape(NB, bs, Hkv, D), vc.reshape(NB, bs, Hkv, D)


# ---------------------------------------------------------------------------------------
# Decode attention.
# ---------------------------------------------------------------------------------------
def kv_head_for(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head shared by query head h: consecutive groups of Hq/Hkv query heads."""
    return h // (num_q_heads // num_kv_heads)


def gather_dense(cache_bits: np.ndarray, table_row: np.ndarray, length: int,
                 dtype: str = "bf16") -> np.ndarray:
    """Logical positions 0..length-1 of one sequence as a dense float64 [length, Hkv, D]
    array, reading physical block table_row[j] for logical block j."""
    NB, bs, Hkv, D = cache_bits.shape
    n = (length + bs - 1) // bs
    ids = np.asarray(table_row[:n], dtype=np.int64)
    if n > len(table_row):
        raise ValueError("context needs more blocks than the table holds")
    if n and (ids.min() < 0 or ids.max() >= NB):
        raise ValueError("block id outside the pool")
    dense = decode_bits(cache_bits[ids], dtype).reshape(n * bs, Hkv, D)
    return dense[:length]


def attend_one(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale_eff: float) -> np.ndarray:
    """softmax(K qh * scale) V for one query vector; K, V are [L, D] float64."""
    s = (K @ qh) * scale_eff
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum()


def effective_scale(scale: float) -> float:
    """The scale as the GPU receives it: rounded to float32."""
    return float(np.float32(scale))


def decode_attention(q_bits: np.ndarray, k_cache_bits: np.ndarray, v_cache_bits: np.ndarray,
                     block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                     rows: Optional[Iterable[Tuple[int, int]]] = None,
                     dtype: str = "bf16") -> np.ndarray:
    """Float64 output [B, Hq, D] of one-token decode attention over the paged cache.

    q_bits uint16 [B, Hq, D]; caches uint16 [NB, bs, Hkv, D]; block_tables int [B, MB];
    context_lens int [B]; dtype: format of q and the caches ("bf16" or "f16"). With ``rows``
    (an iterable of (b, h) pairs) only those output rows are computed; the others stay zero.
    """
    B, Hq, D = q_bits.shape
    Hkv = k_cache_bits.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    scale_eff = effective_scale(scale)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    wanted = {}
    if rows is None:
        for b in range(B):
            wanted[b] = list(range(Hq))
    else:
        for b, h in rows:
            wanted.setdefault(int(b), []).append(int(h))
    for b, heads in sorted(wanted.items()):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = gather_dense(k_cache_bits, block_tables[b], L, dtype)
        V = gather_dense(v_cache_bits, block_tables[b], L, dtype)
        qd = decode_bits(q_bits[b], dtype)
        for h in heads:
            g = kv_head_for(h, Hq, Hkv)
            out[b, h] = attend_one(qd[h], K[:, g, :], V[:, g, :], scale_eff)
    return out


def prefill_attention(q_bits: np.ndarray, cu_seqlens_q: np.ndarray, k_cache_bits: np.ndarray,
                      v_cache_bits: np.ndarray, block_tables: np.ndarray,
                      context_lens: np.ndarray, scale: float,
                      rows: Optional[Iterable[Tuple[int, int]]] = None,
                      dtype: str = "bf16") -> np.ndarray:
    """Float64 output [T, Hq, D] of multi-query causal attention over the paged cache.

    Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (Q_b of them), which are
    its last Q_b logical positions: query i sits at position p = L_b - Q_b + i and attends to
    positions 0..p (causal). Q_b = L_b is a full prefill or recompute; Q_b < L_b is a chunk
    appended to a cached prefix; Q_b = 1 is the decode case. This is the causal SDPA the
    Llama engine uses for prefill and recomputation ("vLLM-Style Llama Inference Engine with
    Tensor Parallelism", Features and scope / Implemented, How it works step 4) with keys
    gathered through the block table, the ragged attention over block tables that llm-stack's
    Roadmap plans. Its keys must already be in the cache (write them first). With ``rows``
    (an iterable of (query row, head) pairs) only those outputs are computed. dtype is the
    format of q and the caches ("bf16" or "f16").
    """
    T, Hq, D = q_bits.shape
    B = len(context_lens)
    Hkv = k_cache_bits.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    if len(cu) != B + 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens_q must be [B+1] non-decreasing offsets from 0 to T")
    scale_eff = effective_scale(scale)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    wanted = None
    if rows is not None:
        wanted = {}
        for r, h in rows:
            wanted.setdefault(int(r), []).append(int(h))
    for b in range(B):
        L = int(context_lens[b])
        Q = int(cu[b + 1] - cu[b])
        if Q == 0:
            continue
        if Q > L:
            raise ValueError(f"sequence {b}: {Q} queries but only {L} cached positions")
        if wanted is not None and not any(cu[b] <= r < cu[b + 1] for r in wanted):
            continue
        K = gather_dense(k_cache_bits, block_tables[b], L, dtype)
        V = gather_dense(v_cache_bits, block_tables[b], L, dtype)
        qd = decode_bits(q_bits[cu[b]:cu[b + 1]], dtype)
        positions = L - Q + np.arange(Q)  # row i sits at position L - Q + i
        for h in range(Hq):
            if wanted is None:
                idx = np.arange(Q)
            else:
                idx = np.array([i for i in range(Q) if h in wanted.get(int(cu[b]) + i, [])],
                               dtype=np.int64)
                if idx.size == 0:
                    continue
            g = kv_head_for(h, Hq, Hkv)
            out[cu[b] + idx, h] = attend_causal(qd[idx, h], np.ascontiguousarray(K[:, g, :]),
                                                np.ascontiguousarray(V[:, g, :]),
                                                positions[idx], scale_eff)
    return out


def attend_causal(Qh: np.ndarray, K: np.ndarray, V: np.ndarray, positions: np.ndarray,
                  scale_eff: float) -> np.ndarray:
    """Row i: softmax(K[:positions[i]+1] Qh[i] * scale) V[:positions[i]+1], for a block of
    query rows of one head at once. Keys after a row's position get score -inf (the causal
    mask), so each row is the one-query definition of attend_one over its own prefix."""
    s = (Qh @ K.T) * scale_eff                       # [rows, L]
    s[np.arange(K.shape[0])[None, :] > positions[:, None]] = -np.inf
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def decode_step(inp: dict, rows=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Write the step's new tokens, then attend over the updated pools (the decode step
    writes position L_b - 1 first and then reads positions 0..L_b-1).

    inp holds host numpy arrays: q, k_cache, v_cache, k_new, v_new (uint16 bits),
    block_tables, context_lens, slot_mapping, scale. Returns (out, k_cache', v_cache').
    """
    kc, vc = kv_write(inp["k_new"], inp["v_new"], inp["slot_mapping"],
                      inp["k_cache"], inp["v_cache"])
    out = decode_attention(inp["q"], kc, vc, inp["block_tables"], inp["context_lens"],
                           inp["scale"], rows=rows)
    return out, kc, vc


# ---------------------------------------------------------------------------------------
# Rotary position embedding at absolute positions, applied before keys enter the cache
# (llm-stack, Serving engine / KV cache bullet: RoPE at absolute positions before the keys
# are cached; "tiny-vLLM" blog, CUDA Kernel Engineering: RoPE rotates pairs of hidden-state
# components by position-dependent angles with sine and cosine).
# Pair i of a head vector is rotated by angle theta_i = position * inv_freq[i]. Pairs are
# (i, i + D/2) ("half" pairing) or (2i, 2i+1) ("interleaved"). The angle is formed in fp32
# (as a GPU receives position and frequency), everything after it in float64; the rotated
# value is rounded to bf16 (round-to-nearest-even) when it is stored.
# ---------------------------------------------------------------------------------------
def rope_pairs(D: int, interleaved: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Index arrays (first, second) of the D/2 rotated pairs."""
    i = np.arange(D // 2)
    if interleaved:
        return 2 * i, 2 * i + 1
    return i, i + D // 2


def rope_angles(position: int, inv_freq: np.ndarray) -> np.ndarray:
    """theta_i = fp32(position) * fp32(inv_freq[i]), the product rounded to fp32."""
    return (np.float32(position) * np.asarray(inv_freq, dtype=np.float32)).astype(np.float64)


def rope_rotate(x: np.ndarray, position: int, inv_freq: np.ndarray, interleaved: bool
                ) -> np.ndarray:
    """Rotate the last axis (D) of float64 array x by the angles of `position`."""
    D = x.shape[-1]
    a, b = rope_pairs(D, interleaved)
    th = rope_angles(position, inv_freq)
    c, s = np.cos(th), np.sin(th)
    y = np.array(x, dtype=np.float64, copy=True)
    y[..., a] = x[..., a] * c - x[..., b] * s
    y[..., b] = x[..., b] * c + x[..., a] * s
    return y


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round-to-nearest-even) bit patterns, via an exact
    float64 -> fp32 rounding first only where that cannot double-round: the rounding is
    done directly on the float64 value's bits."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    sign = (bits >> np.uint64(63)).astype(np.uint16) << np.uint16(15)
    ax = np.abs(x)
    out = np.empty(x.shape, dtype=np.uint16)
    # exact decomposition: ax = m * 2^e with m in [1, 2)
    m, e = np.frexp(ax)          # m in [0.5, 1)
    m = m * 2.0
    e = e - 1
    # bf16 keeps 8 significant bits; spacing 2^(e-7) for normals, 2^-133 for subnormals
    e_eff = np.maximum(e, -126)
    ulp = np.ldexp(1.0, (e_eff - 7).astype(np.int64))
    q = ax / ulp                  # exact (power-of-two scaling)
    r = np.rint(q)                # round half to even
    val = r * ulp
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = val.astype(np.float32)
    fbits = f32.view(np.uint32)
    out[:] = (fbits >> np.uint32(16)).astype(np.uint16) & np.uint16(0x7FFF)
    out[ax == 0] = 0
    out[ax >= np.ldexp(1.0, 128) - np.ldexp(1.0, 119)] = 0x7F80  # rounds to infinity
    out[np.isnan(x)] = 0x7FC0
    return (out | sign).astype(np.uint16)


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to binary16 (round-to-nearest-even) bit patterns: 11 significant
    bits for normals (exponents -14..15), spacing 2^-24 below 2^-14, overflow to infinity
    from 65520 (the midpoint above 65504, whose tie goes to the even, infinite, side)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    ax = np.abs(x)
    m, e = np.frexp(np.where(np.isfinite(ax), ax, 0.0))  # ax = m 2^e, m in [0.5, 1)
    e_eff = np.maximum(e - 1, -14)
    ulp = np.ldexp(1.0, (e_eff - 10).astype(np.int64))
    val = np.rint(ax / ulp) * ulp  # exact scaling, round half to even; val is an fp16 value
    with np.errstate(over="ignore", invalid="ignore"):
        out = np.where(val >= 65536.0, np.inf, val).astype(np.float16).view(np.uint16)
    out = np.where(np.isinf(ax), np.uint16(0x7C00), out)
    out = np.where(np.isnan(x), np.uint16(0x7E00), out).astype(np.uint16)
    return np.where(neg & ~np.isnan(x), out | np.uint16(0x8000), out).astype(np.uint16)


def round_output(x: np.ndarray, out_dtype: str) -> np.ndarray:
    """Float64 values as the output format stores them (float64 again): "f32" rounds to fp32,
    "bf16" and "f16" to those formats, all round-to-nearest-even."""
    if out_dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if out_dtype == "bf16":
        return bf16_bits_to_f64(f64_to_bf16_bits(x))
    if out_dtype == "f16":
        return f16_bits_to_f64(f64_to_f16_bits(x))
    raise ValueError(f"unknown output format {out_dtype!r}")


def kv_write_rope(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                  positions: np.ndarray, inv_freq: np.ndarray, interleaved: bool,
                  slot_mapping: np.ndarray, k_cache_bits: np.ndarray, v_cache_bits: np.ndarray
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rotate q and k of token t at positions[t], write rotated k and raw v to slot
    slot_mapping[t] (negative: no write). Returns (q rotated bits, k_cache', v_cache')."""
    q_rot = np.empty_like(q_bits)
    k_rot = np.empty_like(k_bits)
    for t, p in enumerate(np.asarray(positions).tolist()):
        q_rot[t] = f64_to_bf16_bits(rope_rotate(bf16_bits_to_f64(q_bits[t]), p, inv_freq,
                                                interleaved))
        k_rot[t] = f64_to_bf16_bits(rope_rotate(bf16_bits_to_f64(k_bits[t]), p, inv_freq,
                                                interleaved))
    kc, vc = kv_write(k_rot, v_bits, slot_mapping, k_cache_bits, v_cache_bits)
    return q_rot, kc, vc


# ---------------------------------------------------------------------------------------
# Partitioned softmax (split-K) identity. The pages never write it out; it is the running
# max / running sum rescaling behind the tiled online softmax of llm-stack's Attention
# kernel section and the FlashAttention-2 paper the Llama engine lists under References.
# For a split of the keys into parts p with m_p = max score, l_p = sum exp(s - m_p),
# a_p = sum exp(s - m_p) v: out = sum_p e^{m_p - M} a_p / sum_p e^{m_p - M} l_p, M = max m_p.
# ---------------------------------------------------------------------------------------
def partial_stats(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale_eff: float
                  ) -> Tuple[float, float, np.ndarray]:
    """(m, l, a) of one part of the keys; an empty part gives (-inf, 0, 0)."""
    if K.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(V.shape[1])
    s = (K @ qh) * scale_eff
    m = float(s.max())
    p = np.exp(s - m)
    return m, float(p.sum()), p @ V


def merge_partials(parts: Sequence[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Combine per-part (m, l, a) into the softmax output; parts with l == 0 weigh 0."""
    live = [(m, l, a) for (m, l, a) in parts if l > 0]
    if not live:
        return np.zeros_like(parts[0][2])
    M = max(m for m, _, _ in live)
    num = sum(math.exp(m - M) * a for m, _, a in live)
    den = sum(math.exp(m - M) * l for m, l, _ in live)
    return num / den


def split_attend_one(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale_eff: float,
                     bounds: List[int]) -> np.ndarray:
    """Attention of one query evaluated part by part over keys [bounds[i], bounds[i+1])."""
    parts = [partial_stats(qh, K[lo:hi], V[lo:hi], scale_eff)
             for lo, hi in zip(bounds[:-1], bounds[1:])]
    return merge_partials(parts)
