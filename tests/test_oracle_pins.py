"""Pins of the CPU oracle to facts fixed by the pages and by mathematics (no GPU).

Each test ties the oracle to something other than itself: exact bf16 decoding, hand-worked
closed forms, library attention (torch SDPA in float64), brute force in pure Python,
invariants of the paged layout, and planted mutations that must be caught.
"""
import json
import math
import os
import struct

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.oracle as orc
from paged_kv_decode_write_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
QNAN = 0x7FC0


# ------------------------------------------------------------------------------ helpers
def rand_bits(rng, shape, std=1.0):
    """bf16 bit patterns of N(0, std^2) samples (round-to-nearest-even via torch)."""
    x = torch.from_numpy(rng.standard_normal(shape) * std).to(torch.float32)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_bf16_bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def scatter_to_pool(rng, dense_k, dense_v, lengths, NB, bs, MB, fill=QNAN):
    """Place each sequence's dense rows [L, Hkv, D] into randomly chosen physical blocks of
    a pool filled with `fill` bits; return the pool and block table. Written independently
    of the oracle's gather."""
    B = len(lengths)
    Hkv, D = dense_k[0].shape[1:] if lengths[0] else dense_k[1].shape[1:]
    kc = np.full((NB, bs, Hkv, D), fill, dtype=np.uint16)
    vc = np.full((NB, bs, Hkv, D), fill, dtype=np.uint16)
    perm = rng.permutation(NB)
    tables = np.full((B, MB), -1, dtype=np.int32)
    nxt = 0
    for b, L in enumerate(lengths):
        for t in range(L):
            j, off = divmod(t, bs)
            if off == 0:
                tables[b, j] = perm[nxt]
                nxt += 1
            blk = tables[b, j]
            kc[blk, off] = dense_k[b][t]
            vc[blk, off] = dense_v[b][t]
    return kc, vc, tables


def sdpa_dense(q_bits, dense_k, dense_v, lengths, scale, Hq, D):
    """Library reference: torch SDPA in float64 on the dense (unpaged) sequences."""
    B = len(lengths)
    out = np.zeros((B, Hq, D))
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        q = torch.from_numpy(oracle.bf16_bits_to_f64(q_bits[b]))[None, :, None, :]  # [1,Hq,1,D]
        k = torch.from_numpy(oracle.bf16_bits_to_f64(dense_k[b])).permute(1, 0, 2)[None]
        v = torch.from_numpy(oracle.bf16_bits_to_f64(dense_v[b])).permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(q, k, v, scale=float(np.float32(scale)),
                                           enable_gqa=True)
        out[b] = o[0, :, 0, :].numpy()
    return out


def random_case(seed, B=3, Hq=8, Hkv=2, D=16, bs=4, lengths=None, NB=None, q_std=1.0):
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = [int(x) for x in rng.integers(1, 40, size=B)]
    B = len(lengths)
    MB = max(1, max((L + bs - 1) // bs for L in lengths))
    need = sum((L + bs - 1) // bs for L in lengths)
    NB = NB or need + 5
    dense_k = [rand_bits(rng, (L, Hkv, D)) for L in lengths]
    dense_v = [rand_bits(rng, (L, Hkv, D)) for L in lengths]
    q = rand_bits(rng, (B, Hq, D), std=q_std)
    kc, vc, tables = scatter_to_pool(rng, dense_k, dense_v, lengths, NB, bs, MB)
    return dict(q=q, dense_k=dense_k, dense_v=dense_v, kc=kc, vc=vc, tables=tables,
                lengths=np.array(lengths, dtype=np.int32), Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                scale=1.0 / math.sqrt(D), rng=rng)


def run_oracle(c):
    return oracle.decode_attention(c["q"], c["kc"], c["vc"], c["tables"], c["lengths"], c["scale"])


def run_sdpa(c):
    return sdpa_dense(c["q"], c["dense_k"], c["dense_v"], c["lengths"].tolist(), c["scale"],
                      c["Hq"], c["D"])


# --------------------------------------------------------------------- bf16 decoding
def test_bf16_decode_known_patterns():
    # bf16 keeps float32's 8 exponent bits and 7 fraction bits ("tiny-vLLM" blog, BF16).
    cases = {0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0xC000: -2.0, 0x4049: 3.140625,
             0x3F81: 1.0 + 2.0 ** -7, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133,
             0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127}
    for bits, val in cases.items():
        assert oracle.bf16_bits_to_f64(np.array([bits], np.uint16))[0] == val
    assert oracle.bf16_bits_to_f64(np.array([0x7F80], np.uint16))[0] == math.inf
    assert oracle.bf16_bits_to_f64(np.array([0xFF80], np.uint16))[0] == -math.inf
    assert math.isnan(oracle.bf16_bits_to_f64(np.array([QNAN], np.uint16))[0])
    neg0 = oracle.bf16_bits_to_f64(np.array([0x8000], np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0


def test_bf16_decode_exhaustive_against_struct():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    for b in range(0, 65536, 1):
        ref = struct.unpack(">f", bytes([b >> 8, b & 0xFF, 0, 0]))[0]
        g = got[b]
        if math.isnan(ref):
            assert math.isnan(g)
        else:
            assert g == ref and math.copysign(1, g) == math.copysign(1, ref)


# --------------------------------------------------------------- worked examples (golden)
def _bits(a):
    return np.array([[[int(x, 16) for x in row] for row in hrows] for hrows in a], dtype=np.uint16)


def load_golden():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["cases"]


def closed_form(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e}))  # noqa: S307 (fixture text)


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c["name"])
def test_golden_worked_examples(case):
    NB, bs = case["num_blocks"], case["block_size"]
    Hq, Hkv, D = case["num_q_heads"], case["num_kv_heads"], case["head_dim"]
    tables = np.array(case["block_tables"], dtype=np.int32)
    lens = np.array(case["context_lens"], dtype=np.int32)
    q = np.array([[[int(x, 16) for x in h] for h in qb] for qb in case["q"]], dtype=np.uint16)
    kc = np.full((NB, bs, Hkv, D), QNAN, np.uint16)
    vc = np.full((NB, bs, Hkv, D), QNAN, np.uint16)
    for b, L in enumerate(lens.tolist()):
        for t in range(L):
            blk, off = tables[b, t // bs], t % bs
            kc[blk, off] = _bits(case["logical_k"][b][t:t + 1])[0]
            vc[blk, off] = _bits(case["logical_v"][b][t:t + 1])[0]
    out = oracle.decode_attention(q, kc, vc, tables, lens, case["scale"])
    exp = np.array([[[closed_form(x) for x in h] for h in ob] for ob in case["expected"]])
    np.testing.assert_allclose(out, exp, rtol=0, atol=1e-14)


# ---------------------------------------------------------- P1: paged == dense (SDPA)
@pytest.mark.parametrize("seed,Hq,Hkv,D,bs", [(1, 8, 2, 16, 4), (2, 6, 2, 8, 16),
                                              (3, 4, 4, 32, 1), (4, 12, 4, 64, 16),
                                              (5, 8, 1, 128, 8)])
def test_P1_paged_equals_dense_sdpa(seed, Hq, Hkv, D, bs):
    c = random_case(seed, Hq=Hq, Hkv=Hkv, D=D, bs=bs)
    np.testing.assert_allclose(run_oracle(c), run_sdpa(c), rtol=0, atol=1e-12)


def test_P1_workload_shapes_against_sdpa():
    """c2-shaped (G=3, D=128) and c3-shaped (G=4, D=64) heads and lengths, smaller batch."""
    for seed, Hq, Hkv, D, L in [(11, 24, 8, 128, [512, 77]), (12, 32, 8, 64, [2048, 1])]:
        c = random_case(seed, Hq=Hq, Hkv=Hkv, D=D, bs=16, lengths=L)
        np.testing.assert_allclose(run_oracle(c), run_sdpa(c), rtol=0, atol=1e-12)


# ---------------------------------------------------- P2: physical block permutation
def test_P2_block_permutation_bit_identical():
    c = random_case(21, B=4, lengths=[5, 17, 32, 1])
    base = run_oracle(c)
    NB = c["kc"].shape[0]
    pi = c["rng"].permutation(NB)
    kc2 = np.empty_like(c["kc"]); vc2 = np.empty_like(c["vc"])
    kc2[pi] = c["kc"]; vc2[pi] = c["vc"]
    t2 = np.where(c["tables"] >= 0, pi[np.maximum(c["tables"], 0)], -1).astype(np.int32)
    out = oracle.decode_attention(c["q"], kc2, vc2, t2, c["lengths"], c["scale"])
    assert np.array_equal(out, base)


# --------------------------------------------------------- P3/P4/P5: closed forms
def test_P3_length_one_returns_value_row():
    c = random_case(31, B=3, lengths=[1, 1, 1], D=32)
    out = run_oracle(c)
    for b in range(3):
        for h in range(c["Hq"]):
            g = h // (c["Hq"] // c["Hkv"])
            assert np.array_equal(out[b, h], oracle.bf16_bits_to_f64(c["dense_v"][b][0, g]))


def test_P4_constant_values():
    c = random_case(41, lengths=[9, 33, 64], D=16)
    const = f32_to_bf16_bits(np.full((c["Hkv"], c["D"]), 0.0))
    cvals = c["rng"].standard_normal((c["Hkv"], c["D"])).astype(np.float32)
    const = f32_to_bf16_bits(cvals)
    c["dense_v"] = [np.broadcast_to(const, dv.shape).copy() for dv in c["dense_v"]]
    c["kc"], c["vc"], c["tables"] = scatter_to_pool(c["rng"], c["dense_k"], c["dense_v"],
                                                    c["lengths"].tolist(), c["kc"].shape[0],
                                                    c["bs"], c["tables"].shape[1])
    out = run_oracle(c)
    G = c["Hq"] // c["Hkv"]
    cv = oracle.bf16_bits_to_f64(const)
    for h in range(c["Hq"]):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(cv[h // G], out[:, h].shape),
                                   rtol=1e-15, atol=1e-15)


def test_P5_zero_query_gives_mean():
    c = random_case(51, lengths=[3, 40, 17], D=8)
    c["q"][:] = 0
    out = run_oracle(c)
    G = c["Hq"] // c["Hkv"]
    for b, L in enumerate(c["lengths"].tolist()):
        V = oracle.bf16_bits_to_f64(c["dense_v"][b])
        for h in range(c["Hq"]):
            np.testing.assert_allclose(out[b, h], V[:, h // G].mean(axis=0), rtol=0, atol=1e-14)


# ------------------------------------------------------ P6: brute force, pure Python
def _brute_bf16(b):
    return struct.unpack(">f", bytes([b >> 8, b & 0xFF, 0, 0]))[0]


def brute_force(q, kc, vc, tables, lens, scale):
    """Pure-Python loops over a dict-of-lists page table, math.exp / math.fsum."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = kc.shape
    G = Hq // Hkv
    s32 = struct.unpack("f", struct.pack("f", scale))[0]
    pages = {b: [int(x) for x in tables[b] if x >= 0] for b in range(B)}
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            if L == 0:
                continue
            g = h // G
            scores = []
            for t in range(L):
                blk = pages[b][t // bs]
                krow = kc[blk][t % bs][g]
                scores.append(math.fsum(_brute_bf16(int(q[b][h][d])) * _brute_bf16(int(krow[d]))
                                        for d in range(D)) * s32)
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            den = math.fsum(w)
            for d in range(D):
                num = math.fsum(w[t] * _brute_bf16(int(vc[pages[b][t // bs]][t % bs][g][d]))
                                for t in range(L))
                out[b][h][d] = num / den
    return np.array(out)


@pytest.mark.parametrize("seed", range(12))
def test_P6_brute_force_tiny(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 3))
    D = int(rng.integers(1, 5))
    bs = int(rng.choice([1, 2, 4]))
    lengths = [int(x) for x in rng.integers(0, 10, size=B)]
    if max(lengths) == 0:
        lengths[0] = 1
    c = random_case(2000 + seed, Hq=Hq, Hkv=Hkv, D=D, bs=bs, lengths=lengths)
    got = run_oracle(c)
    ref = brute_force(c["q"], c["kc"], c["vc"], c["tables"], c["lengths"], c["scale"])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# --------------------------------------- P7: cached decode == full recompute (causal)
def test_P7_decode_equals_last_row_of_causal_recompute():
    rng = np.random.default_rng(71)
    Hq, Hkv, D, L, bs = 8, 2, 16, 37, 4
    qs = rand_bits(rng, (L, Hq, D))
    dk = rand_bits(rng, (L, Hkv, D))
    dv = rand_bits(rng, (L, Hkv, D))
    kc, vc, tables = scatter_to_pool(rng, [dk], [dv], [L], 20, bs, 10)
    scale = 1 / math.sqrt(D)
    dec = oracle.decode_attention(qs[L - 1:L][None][0:1].reshape(1, Hq, D), kc, vc, tables,
                                  np.array([L], np.int32), scale)[0]
    Q = torch.from_numpy(oracle.bf16_bits_to_f64(qs)).permute(1, 0, 2)[None]
    K = torch.from_numpy(oracle.bf16_bits_to_f64(dk)).permute(1, 0, 2)[None]
    V = torch.from_numpy(oracle.bf16_bits_to_f64(dv)).permute(1, 0, 2)[None]
    full = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=float(np.float32(scale)),
                                          enable_gqa=True)[0, :, L - 1, :].numpy()
    np.testing.assert_allclose(dec, full, rtol=0, atol=1e-12)
    # Mutation: a causal mask built as tril(1, L) for the single decode row exposes key 0 only.
    bad_mask = torch.tril(torch.ones(1, L, dtype=torch.bool))
    wrong = F.scaled_dot_product_attention(Q[:, :, L - 1:L], K, V, attn_mask=bad_mask,
                                           scale=float(np.float32(scale)),
                                           enable_gqa=True)[0, :, 0, :].numpy()
    assert np.abs(dec - wrong).max() > 1e-2


# ------------------------------------------------------------- P8: GQA == MHA
def test_P8_gqa_equals_repeated_mha():
    c = random_case(81, Hq=12, Hkv=3, D=8, lengths=[7, 20, 33])
    G = c["Hq"] // c["Hkv"]
    base = run_oracle(c)
    kc_m = np.repeat(c["kc"], G, axis=2)
    vc_m = np.repeat(c["vc"], G, axis=2)
    mha = oracle.decode_attention(c["q"], kc_m, vc_m, c["tables"], c["lengths"], c["scale"])
    assert np.array_equal(base, mha)
    q2 = c["q"].copy()
    for g in range(c["Hkv"]):
        q2[:, g * G:(g + 1) * G] = q2[:, g * G][:, None]
    out2 = oracle.decode_attention(q2, c["kc"], c["vc"], c["tables"], c["lengths"], c["scale"])
    for g in range(c["Hkv"]):
        for i in range(1, G):
            assert np.array_equal(out2[:, g * G + i], out2[:, g * G])


# --------------------------------------------------- P9: token order does not matter
def test_P9_token_permutation_invariance():
    c = random_case(91, lengths=[30, 45, 5])
    base = run_oracle(c)
    perm_k, perm_v = [], []
    for dk, dv in zip(c["dense_k"], c["dense_v"]):
        p = c["rng"].permutation(dk.shape[0])
        perm_k.append(dk[p]); perm_v.append(dv[p])
    kc, vc, tables = scatter_to_pool(c["rng"], perm_k, perm_v, c["lengths"].tolist(),
                                     c["kc"].shape[0], c["bs"], c["tables"].shape[1])
    out = oracle.decode_attention(c["q"], kc, vc, tables, c["lengths"], c["scale"])
    np.testing.assert_allclose(out, base, rtol=0, atol=1e-12)


# ----------------------------------------------- P10: unread slots never matter
@pytest.mark.parametrize("fill", [QNAN, 0x7149, 0xF149, 0x7F80])  # NaN, +-~1e30, +inf
def test_P10_garbage_in_unread_slots(fill):
    c = random_case(101, lengths=[13, 1, 16, 31])
    base = run_oracle(c)
    kc, vc, tables = scatter_to_pool(np.random.default_rng(101 + 7), c["dense_k"], c["dense_v"],
                                     c["lengths"].tolist(), c["kc"].shape[0] + 3, c["bs"],
                                     c["tables"].shape[1] + 2, fill=fill)
    out = oracle.decode_attention(c["q"], kc, vc, tables, c["lengths"], c["scale"])
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, base, rtol=0, atol=1e-15)


def test_P10_workload_poison_matches_clean():
    w = wl.Workload("tiny", batch=5, num_q_heads=8, num_kv_heads=2, head_dim=32, block_size=16,
                    num_blocks=40, max_blocks=6, seed=7, max_context_len=90)
    clean = wl.to_host_numpy(wl.make_inputs(w))
    dirty = wl.to_host_numpy(wl.make_inputs(w, poison=True))
    o1, _, _ = oracle.decode_step(clean)
    o2, _, _ = oracle.decode_step(dirty)
    assert np.array_equal(o1, o2)


# ------------------------------------------------------ P11: planted mutations fail
MUTATIONS = {
    "length_plus_one": lambda mp: mp.setattr(
        orc, "gather_dense", _wrap_gather(lambda cb, row, L: (cb, row, L + 1))),
    "length_minus_one": lambda mp: mp.setattr(
        orc, "gather_dense", _wrap_gather(lambda cb, row, L: (cb, row, max(L - 1, 1)))),
    "table_off_by_one": lambda mp: mp.setattr(
        orc, "gather_dense", _wrap_gather(lambda cb, row, L: (cb, np.roll(row, -1), L))),
    "k_v_swapped": lambda mp: mp.setattr(
        orc, "attend_one", _wrap_attend(lambda q, K, V, s: (q, V, K, s))),
    "head_map_modulo": lambda mp: mp.setattr(
        orc, "kv_head_for", lambda h, hq, hkv: h % hkv),
    "scale_dropped": lambda mp: mp.setattr(orc, "effective_scale", lambda s: 1.0),
}

_REAL_GATHER = orc.gather_dense
_REAL_ATTEND = orc.attend_one


def _wrap_gather(tf):
    def g(cache_bits, row, L, *fmt):
        cb, r, L2 = tf(cache_bits, row, L)
        NB, bs = cb.shape[:2]
        n = (L2 + bs - 1) // bs
        r = np.where(np.asarray(r[:n]) < 0, 0, np.asarray(r[:n]))  # keep the mutant runnable
        full = np.concatenate([r, np.zeros(max(0, n - len(r)), dtype=r.dtype)])
        return _REAL_GATHER(cb, full, L2, *fmt)
    return g


def _wrap_attend(tf):
    def a(q, K, V, s):
        return _REAL_ATTEND(*tf(q, K, V, s))
    return a


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_P11_mutations_are_caught(name, monkeypatch):
    # c2-shaped heads (G=3, D=128) with several lengths, blocks scattered over a pool.
    c = random_case(111, Hq=24, Hkv=8, D=128, bs=16, lengths=[512, 100, 47], NB=200)
    ref = run_sdpa(c)
    np.testing.assert_allclose(run_oracle(c), ref, rtol=0, atol=1e-12)
    MUTATIONS[name](monkeypatch)
    try:
        bad = run_oracle(c)
    except (ValueError, IndexError):
        return  # the mutant cannot even run on valid input: caught
    assert np.nanmax(np.abs(bad - ref)) > 2e-3 or not np.isfinite(bad).all(), name


# ------------------------------------------------------- P12: split-K identity
def test_P12_split_identity_random_partitions():
    rng = np.random.default_rng(121)
    for trial in range(30):
        L = int(rng.integers(1, 400))
        D = int(rng.choice([4, 64, 128]))
        qh = rng.standard_normal(D) * 3
        K = rng.standard_normal((L, D))
        V = rng.standard_normal((L, D))
        nb = int(rng.integers(0, 12))
        cuts = sorted(set(int(x) for x in rng.integers(0, L + 1, size=nb)) | {0, L})
        # allow empty parts too
        if trial % 3 == 0:
            cuts = sorted(cuts + [cuts[-1]])
        got = oracle.split_attend_one(qh, K, V, 1 / math.sqrt(D), cuts)
        ref = oracle.attend_one(qh, K, V, 1 / math.sqrt(D))
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # a part with no keys merges as weight zero
    m, l, a = oracle.partial_stats(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert m == -math.inf and l == 0.0 and not a.any()


# -------------------------------------------------------- W1-W5: the KV write
def _write_case(seed=201, NB=12, bs=4, Hkv=2, D=8, T=6):
    rng = np.random.default_rng(seed)
    kc = rand_bits(rng, (NB, bs, Hkv, D)); vc = rand_bits(rng, (NB, bs, Hkv, D))
    k = rand_bits(rng, (T, Hkv, D)); v = rand_bits(rng, (T, Hkv, D))
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int64)
    return kc, vc, k, v, slots


def test_W1_W2_written_rows_and_untouched_rest():
    kc, vc, k, v, slots = _write_case()
    kc2, vc2 = oracle.kv_write(k, v, slots, kc, vc)
    NB, bs = kc.shape[:2]
    flat_k, flat_v = kc2.reshape(NB * bs, *kc.shape[2:]), vc2.reshape(NB * bs, *vc.shape[2:])
    for t, s in enumerate(slots):
        assert np.array_equal(flat_k[s], k[t]) and np.array_equal(flat_v[s], v[t])
    mask = np.ones(NB * bs, bool); mask[slots] = False
    assert np.array_equal(flat_k[mask], kc.reshape(NB * bs, *kc.shape[2:])[mask])
    assert np.array_equal(flat_v[mask], vc.reshape(NB * bs, *vc.shape[2:])[mask])
    # inputs are not modified in place
    assert not np.shares_memory(kc2, kc)


def test_W2_nan_payloads_survive():
    kc, vc, k, v, slots = _write_case(seed=202)
    k[0, 0, 0] = 0x7FA1  # a NaN with a payload
    v[1, 1, 3] = 0xFFC3
    kc2, vc2 = oracle.kv_write(k, v, slots, kc, vc)
    NB, bs = kc.shape[:2]
    assert kc2.reshape(NB * bs, *kc.shape[2:])[slots[0]][0, 0] == 0x7FA1
    assert vc2.reshape(NB * bs, *vc.shape[2:])[slots[1]][1, 3] == 0xFFC3


def test_W3_write_then_gather_roundtrip():
    w = wl.WORKLOADS["c2"]
    inp = wl.to_host_numpy(wl.make_inputs(w))
    _, kc, vc = oracle.decode_step(inp, rows=[])
    for b, L in enumerate(inp["context_lens"].tolist()):
        K = oracle.gather_dense(kc, inp["block_tables"][b], L)
        V = oracle.gather_dense(vc, inp["block_tables"][b], L)
        assert np.array_equal(K[L - 1], oracle.bf16_bits_to_f64(inp["k_new"][b]))
        assert np.array_equal(V[L - 1], oracle.bf16_bits_to_f64(inp["v_new"][b]))


def test_W4_negative_slots_skipped():
    kc, vc, k, v, slots = _write_case(seed=204)
    slots2 = slots.copy(); slots2[[1, 3]] = -1
    kc2, vc2 = oracle.kv_write(k, v, slots2, kc, vc)
    keep = [0, 2, 4, 5]
    kc3, vc3 = oracle.kv_write(k[keep], v[keep], slots[keep], kc, vc)
    assert np.array_equal(kc2, kc3) and np.array_equal(vc2, vc3)


def test_W5_invalid_slots_rejected():
    kc, vc, k, v, slots = _write_case(seed=205)
    dup = slots.copy(); dup[2] = dup[0]
    with pytest.raises(ValueError):
        oracle.kv_write(k, v, dup, kc, vc)
    oob = slots.copy(); oob[1] = kc.shape[0] * kc.shape[1]
    with pytest.raises(ValueError):
        oracle.kv_write(k, v, oob, kc, vc)


def test_decode_step_orders_write_before_attention():
    """The new token is visible to the same step's attention: with L=1 the output equals
    the value row just written."""
    w = wl.Workload("one", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=16,
                    num_blocks=8, max_blocks=2, seed=5, context_len=1)
    inp = wl.to_host_numpy(wl.make_inputs(w))
    out, _, _ = oracle.decode_step(inp)
    vn = oracle.bf16_bits_to_f64(inp["v_new"])
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], vn[b, h // 2])


# ----------------------------------------------- multi-query causal (prefill) oracle pins
def prefill_case(seed, lens, qlens, Hq=8, Hkv=2, D=16, bs=4):
    rng = np.random.default_rng(seed)
    dense_k = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    dense_v = [rand_bits(rng, (L, Hkv, D)) for L in lens]
    MB = max(1, max((L + bs - 1) // bs for L in lens))
    NB = sum((L + bs - 1) // bs for L in lens) + 3
    kc, vc, tables = scatter_to_pool(rng, dense_k, dense_v, lens, NB, bs, MB)
    T = sum(qlens)
    q = rand_bits(rng, (T, Hq, D))
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return dict(q=q, cu=cu, kc=kc, vc=vc, tables=tables, lens=np.array(lens, np.int32),
                qlens=qlens, dense_k=dense_k, dense_v=dense_v, Hq=Hq, Hkv=Hkv, D=D,
                scale=1 / math.sqrt(D))


def run_prefill(c):
    return oracle.prefill_attention(c["q"], c["cu"], c["kc"], c["vc"], c["tables"], c["lens"],
                                    c["scale"])


def sdpa_prefill(c, offset=0):
    """torch SDPA in float64 with an explicit causal mask (row i sees keys <= L-Q+i+offset)."""
    out = np.zeros((c["q"].shape[0], c["Hq"], c["D"]))
    for b, (L, Q) in enumerate(zip(c["lens"].tolist(), c["qlens"])):
        if Q == 0:
            continue
        q = torch.from_numpy(oracle.bf16_bits_to_f64(c["q"][c["cu"][b]:c["cu"][b + 1]]))
        k = torch.from_numpy(oracle.bf16_bits_to_f64(c["dense_k"][b]))
        v = torch.from_numpy(oracle.bf16_bits_to_f64(c["dense_v"][b]))
        i = torch.arange(Q)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= (L - Q + i + offset)
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], k.permute(1, 0, 2)[None],
                                           v.permute(1, 0, 2)[None], attn_mask=mask,
                                           scale=float(np.float32(c["scale"])), enable_gqa=True)
        out[c["cu"][b]:c["cu"][b + 1]] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("seed,lens,qlens,Hq,Hkv,D,bs", [
    (301, [40, 7, 33], [40, 3, 16], 8, 2, 16, 4),
    (302, [100, 64], [1, 64], 12, 4, 32, 16),
    (303, [257, 1, 18], [31, 1, 18], 6, 2, 8, 8),
    (304, [600], [120], 16, 1, 64, 16)])
def test_P13_prefill_equals_masked_sdpa(seed, lens, qlens, Hq, Hkv, D, bs):
    c = prefill_case(seed, lens, qlens, Hq, Hkv, D, bs)
    np.testing.assert_allclose(run_prefill(c), sdpa_prefill(c), rtol=0, atol=1e-12)


def test_P14_full_prefill_equals_is_causal():
    c = prefill_case(311, [50, 33], [50, 33], 8, 2, 16, 4)
    out = run_prefill(c)
    for b in range(2):
        q = torch.from_numpy(oracle.bf16_bits_to_f64(c["q"][c["cu"][b]:c["cu"][b + 1]]))
        k = torch.from_numpy(oracle.bf16_bits_to_f64(c["dense_k"][b]))
        v = torch.from_numpy(oracle.bf16_bits_to_f64(c["dense_v"][b]))
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2)[None], k.permute(1, 0, 2)[None],
                                           v.permute(1, 0, 2)[None], is_causal=True,
                                           scale=float(np.float32(c["scale"])), enable_gqa=True)
        np.testing.assert_allclose(out[c["cu"][b]:c["cu"][b + 1]], o[0].permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_P15_single_query_prefill_equals_decode():
    c = prefill_case(321, [70, 5, 128], [1, 1, 1], 8, 2, 16, 16)
    dec = oracle.decode_attention(c["q"], c["kc"], c["vc"], c["tables"], c["lens"], c["scale"])
    np.testing.assert_allclose(run_prefill(c), dec, rtol=0, atol=1e-13)


def brute_force_prefill(c):
    q, cu, kc, vc, tables, lens = c["q"], c["cu"], c["kc"], c["vc"], c["tables"], c["lens"]
    T, Hq, D = q.shape
    bs, Hkv = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    s32 = struct.unpack("f", struct.pack("f", c["scale"]))[0]
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(T)]
    for b in range(len(lens)):
        L = int(lens[b])
        Q = int(cu[b + 1] - cu[b])
        pages = [int(x) for x in tables[b] if x >= 0]
        for i in range(Q):
            row = int(cu[b]) + i
            last = L - Q + i
            for h in range(Hq):
                g = h // G
                sc = [math.fsum(_brute_bf16(int(q[row][h][d])) *
                                _brute_bf16(int(kc[pages[t // bs]][t % bs][g][d])) for d in range(D)) * s32
                      for t in range(last + 1)]
                mx = max(sc)
                wts = [math.exp(x - mx) for x in sc]
                den = math.fsum(wts)
                for d in range(D):
                    out[row][h][d] = math.fsum(
                        wts[t] * _brute_bf16(int(vc[pages[t // bs]][t % bs][g][d]))
                        for t in range(last + 1)) / den
    return np.array(out)


@pytest.mark.parametrize("seed", range(6))
def test_P16_prefill_brute_force_tiny(seed):
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(1, 10, size=B)]
    qlens = [int(rng.integers(0, L + 1)) for L in lens]
    Hkv = int(rng.integers(1, 3))
    c = prefill_case(4000 + seed, lens, qlens, Hq=Hkv * int(rng.integers(1, 3)), Hkv=Hkv,
                     D=int(rng.integers(1, 5)), bs=int(rng.choice([1, 2, 4])))
    np.testing.assert_allclose(run_prefill(c), brute_force_prefill(c), rtol=0, atol=1e-12)


def test_P17_prefill_mutations_are_caught():
    c = prefill_case(331, [300, 120], [64, 120], 24, 8, 32, 16)
    ref = sdpa_prefill(c)
    np.testing.assert_allclose(run_prefill(c), ref, rtol=0, atol=1e-12)
    # causal offset off by one in either direction, and a mask that ignores the offset
    for off in (-1, 1):
        assert np.abs(sdpa_prefill(c, offset=off) - ref).max() > 2e-3
    qswap = dict(c)
    qswap["q"] = c["q"][::-1].copy()  # rows attached to the wrong positions
    assert np.abs(run_prefill(qswap) - ref).max() > 2e-3


def test_prefill_rejects_bad_arguments():
    c = prefill_case(341, [10, 10], [4, 4])
    with pytest.raises(ValueError):
        oracle.prefill_attention(c["q"], np.array([0, 4, 9], np.int32), c["kc"], c["vc"],
                                 c["tables"], c["lens"], c["scale"])
    with pytest.raises(ValueError):  # more queries than cached positions
        oracle.prefill_attention(c["q"], c["cu"], c["kc"], c["vc"], c["tables"],
                                 np.array([3, 10], np.int32), c["scale"])


# ------------------------------------------------------------ RoPE + write oracle pins
def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    keep = np.isfinite(vals) & ~((vals == 0) & (bits == 0x8000))
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], bits[keep][order]


def test_f64_to_bf16_rounding_against_neighbour_search():
    vals, bits = _all_finite_bf16()
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.standard_normal(2000) * 1e-38,
                        (vals[1:-1] + vals[2:]) / 2,  # exact midpoints: ties
                        [0.0, 1.0, -1.0, 3.3e38]])
    got = oracle.f64_to_bf16_bits(x)
    for xi, gi in zip(x, got):
        ax = abs(xi)
        j = np.searchsorted(vals, ax)
        lo, hi = vals[j - 1], vals[min(j, len(vals) - 1)]
        if ax == hi:
            want = bits[min(j, len(vals) - 1)]
        elif ax - lo < hi - ax:
            want = bits[j - 1]
        elif ax - lo > hi - ax:
            want = bits[j]
        else:  # tie: even significand
            want = bits[j - 1] if bits[j - 1] % 2 == 0 else bits[j]
        if xi < 0 or (xi == 0 and math.copysign(1, xi) < 0):
            want = want | 0x8000
        assert gi == want, (xi, hex(gi), hex(want))


def test_rope_known_values_and_identity():
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    for inter in (False, True):
        y = oracle.rope_rotate(x, 1, np.array([1.0]), inter)
        np.testing.assert_allclose(y[0], [math.cos(1), math.sin(1)], rtol=0, atol=1e-15)
        np.testing.assert_allclose(y[1], [-math.sin(1), math.cos(1)], rtol=0, atol=1e-15)
    rng = np.random.default_rng(7)
    qb = rand_bits(rng, (3, 4, 16))
    inv = (10000.0 ** (-np.arange(8) * 2 / 16)).astype(np.float32)
    q_rot, _, _ = oracle.kv_write_rope(qb, qb[:, :2], qb[:, :2], np.zeros(3, np.int32), inv,
                                       False, -np.ones(3, np.int64),
                                       np.zeros((2, 4, 2, 16), np.uint16),
                                       np.zeros((2, 4, 2, 16), np.uint16))
    assert np.array_equal(q_rot, qb)  # position 0 rotates nothing


def test_rope_frequency_of_each_pair_by_hand():
    """Pair i turns by position * inv_freq[i], for each pair separately. D = 8 with frequencies
    1, 1/2, 1/4, 1/8 (exact in fp32) at position 1: unit vector e_j must come out as the
    cosine / sine of its own pair's angle 2^-i at its own pair's two indices, for half pairing
    (i, i + 4) and interleaved pairing (2i, 2i + 1). A frequency list applied in another order
    (e.g. reversed) gives other angles and fails."""
    inv = np.array([1.0, 0.5, 0.25, 0.125], dtype=np.float32)
    eye = np.eye(8)
    for inter in (False, True):
        for i in range(4):
            a, b = (2 * i, 2 * i + 1) if inter else (i, i + 4)
            th = 2.0 ** -i
            want_a = np.zeros(8)
            want_a[a], want_a[b] = math.cos(th), math.sin(th)
            want_b = np.zeros(8)
            want_b[a], want_b[b] = -math.sin(th), math.cos(th)
            np.testing.assert_allclose(oracle.rope_rotate(eye[a], 1, inv, inter), want_a,
                                       rtol=0, atol=1e-15)
            np.testing.assert_allclose(oracle.rope_rotate(eye[b], 1, inv, inter), want_b,
                                       rtol=0, atol=1e-15)


def test_rope_angle_is_formed_in_fp32():
    """The angle is fp32(position) * inv_freq rounded to fp32, as a GPU forms it. Two cases
    worked by hand: position 2^24 + 1 becomes 2^24 in fp32; 3 * (1 + 2^-23) = 3 + 1.5 units in
    the last place of [2, 4), a tie that rounds to the even neighbour 3 + 2^-21."""
    x = np.array([1.0, 0.0])
    for pos, f, th in ((2 ** 24 + 1, 1.0, 2.0 ** 24), (3, 1.0 + 2.0 ** -23, 3.0 + 2.0 ** -21)):
        y = oracle.rope_rotate(x, pos, np.array([f], dtype=np.float32), False)
        np.testing.assert_allclose(y, [math.cos(th), math.sin(th)], rtol=0, atol=1e-15)


def test_rope_preserves_pair_norms_and_relative_positions():
    rng = np.random.default_rng(8)
    D = 64
    inv = 2.0 ** -np.arange(D // 2, dtype=np.float64)  # exact angles for small positions
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for inter in (False, True):
        a, b = oracle.rope_pairs(D, inter)
        y = oracle.rope_rotate(q, 37, inv, inter)
        np.testing.assert_allclose(y[a] ** 2 + y[b] ** 2, q[a] ** 2 + q[b] ** 2, rtol=1e-13)
        d1 = oracle.rope_rotate(q, 40, inv, inter) @ oracle.rope_rotate(k, 25, inv, inter)
        d2 = oracle.rope_rotate(q, 1040, inv, inter) @ oracle.rope_rotate(k, 1025, inv, inter)
        assert abs(d1 - d2) < 1e-9


def test_rope_interleaved_is_permuted_half():
    rng = np.random.default_rng(9)
    D = 16
    x = rng.standard_normal(D)
    inv = rng.random(D // 2).astype(np.float32)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])  # evens then odds
    inter = oracle.rope_rotate(x, 123, inv, True)
    half = oracle.rope_rotate(x[perm], 123, inv, False)
    np.testing.assert_allclose(inter[perm], half, rtol=0, atol=1e-15)


def test_kv_write_rope_stores_rotated_k_and_raw_v():
    rng = np.random.default_rng(10)
    T, Hq, Hkv, D, NB, bs = 5, 4, 2, 16, 6, 4
    q, k, v = rand_bits(rng, (T, Hq, D)), rand_bits(rng, (T, Hkv, D)), rand_bits(rng, (T, Hkv, D))
    kc, vc = rand_bits(rng, (NB, bs, Hkv, D)), rand_bits(rng, (NB, bs, Hkv, D))
    pos = np.array([0, 5, 17, 1000, 3], np.int32)
    slots = np.array([3, -1, 20, 7, 0], np.int64)
    inv = (500000.0 ** (-np.arange(D // 2) * 2 / D)).astype(np.float32)
    q_rot, kc2, vc2 = oracle.kv_write_rope(q, k, v, pos, inv, False, slots, kc, vc)
    flat_k, flat_v = kc2.reshape(NB * bs, Hkv, D), vc2.reshape(NB * bs, Hkv, D)
    for t in range(T):
        kr = oracle.f64_to_bf16_bits(oracle.rope_rotate(oracle.bf16_bits_to_f64(k[t]), pos[t],
                                                          inv, False))
        if slots[t] >= 0:
            assert np.array_equal(flat_k[slots[t]], kr)
            assert np.array_equal(flat_v[slots[t]], v[t])
    # slot -1: nothing stored, but q is still rotated
    assert not np.array_equal(q_rot[1], q[1])
    untouched = np.ones(NB * bs, bool)
    untouched[[3, 20, 7, 0]] = False
    assert np.array_equal(flat_k[untouched], kc.reshape(NB * bs, Hkv, D)[untouched])


# --------------------------------------------------- fp16 inputs and 16-bit output formats
F16_KNOWN = {0x0000: 0.0, 0x3C00: 1.0, 0xC000: -2.0, 0x3800: 0.5, 0x3555: 1365 / 4096,
             0x7BFF: 65504.0, 0x0400: 2.0 ** -14, 0x03FF: 1023 * 2.0 ** -24,
             0x0001: 2.0 ** -24, 0x8001: -(2.0 ** -24), 0x7C00: math.inf, 0xFC00: -math.inf}


def test_f16_decode_closed_forms():
    bits = np.array(list(F16_KNOWN), dtype=np.uint16)
    got = oracle.f16_bits_to_f64(bits)
    assert got.tolist() == list(F16_KNOWN.values())
    neg0 = oracle.f16_bits_to_f64(np.array([0x8000], np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0
    assert np.isnan(oracle.f16_bits_to_f64(np.array([0x7E00, 0x7C01, 0xFE00, 0xFFFF],
                                                    np.uint16))).all()


def test_f16_decode_matches_library_on_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(oracle.f16_bits_to_f64(bits), lib, equal_nan=True)


def test_decode_bits_dispatches_on_format():
    assert oracle.decode_bits(np.array([0x3C00], np.uint16), "f16")[0] == 1.0
    assert oracle.decode_bits(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0
    with pytest.raises(ValueError):
        oracle.decode_bits(np.array([0], np.uint16), "fp8")


def _all_finite_f16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.f16_bits_to_f64(bits)
    keep = np.isfinite(vals) & (vals >= 0) & ~((vals == 0) & (bits == 0x8000))
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], bits[keep][order]


def test_f64_to_f16_rounding_against_neighbour_search():
    vals, bits = _all_finite_f16()
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(2000) * 1e-6,
                        (vals[1:-1] + vals[2:]) / 2,  # exact midpoints: ties
                        -(vals[1:200] + vals[2:201]) / 2, [0.0, 1.0, -1.0, 65504.0]])
    got = oracle.f64_to_f16_bits(x)
    for xi, gi in zip(x, got):
        ax = abs(xi)
        j = np.searchsorted(vals, ax)
        lo, hi = vals[j - 1], vals[min(j, len(vals) - 1)]
        if ax == hi:
            want = bits[min(j, len(vals) - 1)]
        elif ax - lo < hi - ax:
            want = bits[j - 1]
        elif ax - lo > hi - ax:
            want = bits[j]
        else:  # tie: even significand
            want = bits[j - 1] if bits[j - 1] % 2 == 0 else bits[j]
        if xi < 0:
            want = want | 0x8000
        assert gi == want, (xi, hex(gi), hex(want))


def test_f64_to_f16_overflow_and_specials():
    x = np.array([65519.99, 65520.0, 1e6, -1e6, math.inf, 2.0 ** -25, 1.5 * 2.0 ** -25, -0.0])
    assert [int(b) for b in oracle.f64_to_f16_bits(x)] == [0x7BFF, 0x7C00, 0x7C00, 0xFC00,
                                                           0x7C00, 0x0000, 0x0001, 0x8000]
    n = oracle.f64_to_f16_bits(np.array([math.nan]))[0]
    assert (n & 0x7C00) == 0x7C00 and (n & 0x3FF) != 0


def test_round_output_closed_forms():
    one = np.array([1.0 + 2.0 ** -30, 1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24])
    assert oracle.round_output(one, "f32").tolist() == [1.0, 1.0, 1.0 + 2.0 ** -22]
    assert oracle.round_output(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]),
                               "bf16").tolist() == [1.0, 1.0 + 2.0 ** -6]
    assert oracle.round_output(np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]),
                               "f16").tolist() == [1.0, 1.0 + 2.0 ** -9]
    with pytest.raises(ValueError):
        oracle.round_output(np.zeros(1), "f64")


def _shared_value_case(seed, B=3, Hq=8, Hkv=2, D=16, bs=4):
    """Inputs whose values (multiples of 1/8 up to 3) are exact in bf16 and in fp16, encoded
    both ways, in the same paged layout."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(1, 30, size=B)]
    MB = max((L + bs - 1) // bs for L in lengths)
    NB = sum((L + bs - 1) // bs for L in lengths) + 3
    q = rng.integers(-24, 25, size=(B, Hq, D)) / 8.0
    dk = [rng.integers(-24, 25, size=(L, Hkv, D)) / 8.0 for L in lengths]
    dv = [rng.integers(-24, 25, size=(L, Hkv, D)) / 8.0 for L in lengths]
    enc = {"bf16": lambda a: f32_to_bf16_bits(np.asarray(a, np.float32)),
           "f16": lambda a: np.asarray(a, np.float16).view(np.uint16)}
    out = {}
    for name, e in enc.items():
        kc, vc, tables = scatter_to_pool(np.random.default_rng(seed + 1), [e(x) for x in dk],
                                         [e(x) for x in dv], lengths, NB, bs, MB)
        out[name] = (e(q), kc, vc, tables)
    return out, np.array(lengths, np.int32), q, dk, dv


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_f16_attention_equals_bf16_on_values_exact_in_both(seed):
    enc, lens, _, _, _ = _shared_value_case(seed)
    res = {}
    for name, (q, kc, vc, tables) in enc.items():
        res[name] = oracle.decode_attention(q, kc, vc, tables, lens, 0.25, dtype=name)
    assert np.array_equal(res["bf16"], res["f16"])
    # the format argument matters: fp16 bits read as bf16 are other numbers entirely
    q, kc, vc, tables = enc["f16"]
    wrong = oracle.decode_attention(q, kc, vc, tables, lens, 0.25, dtype="bf16")
    assert not np.allclose(np.nan_to_num(wrong), res["f16"], atol=1e-3)


def test_f16_attention_equals_sdpa_on_library_decoded_values():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D, bs = 3, 6, 2, 16, 4
    lengths = [5, 1, 23]
    f16 = lambda a: np.asarray(a, np.float16).view(np.uint16)
    q = f16(rng.standard_normal((B, Hq, D)) * 2)
    dk = [f16(rng.standard_normal((L, Hkv, D))) for L in lengths]
    dv = [f16(rng.standard_normal((L, Hkv, D))) for L in lengths]
    MB = max((L + bs - 1) // bs for L in lengths)
    kc, vc, tables = scatter_to_pool(rng, dk, dv, lengths, 20, bs, MB)
    got = oracle.decode_attention(q, kc, vc, tables, np.array(lengths), 0.3, dtype="f16")
    dec = lambda b: torch.from_numpy(b.view(np.float16).astype(np.float64))
    for b, L in enumerate(lengths):
        o = F.scaled_dot_product_attention(dec(q[b])[None, :, None, :],
                                           dec(dk[b]).permute(1, 0, 2)[None],
                                           dec(dv[b]).permute(1, 0, 2)[None],
                                           scale=float(np.float32(0.3)), enable_gqa=True)
        np.testing.assert_allclose(got[b], o[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


def test_f16_prefill_equals_bf16_on_values_exact_in_both():
    enc, lens, _, _, _ = _shared_value_case(4, B=2)
    qlens = [min(int(L), 3) for L in lens]
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    res = {}
    for name, (_, kc, vc, tables) in enc.items():
        rng = np.random.default_rng(9)
        qv = rng.integers(-24, 25, size=(int(cu[-1]), 8, 16)) / 8.0
        qb = (f32_to_bf16_bits(qv.astype(np.float32)) if name == "bf16"
              else qv.astype(np.float16).view(np.uint16))
        res[name] = oracle.prefill_attention(qb, cu, kc, vc, tables, lens, 0.25, dtype=name)
    assert np.array_equal(res["bf16"], res["f16"])


def test_workload_f16_inputs_are_the_same_draws_rounded():
    w = wl.WORKLOADS["c1"]
    a = wl.make_inputs(w, dtype="bf16")
    b = wl.make_inputs(w, dtype="f16")
    assert b["q"].dtype == torch.float16 and b["k_cache"].dtype == torch.float16
    assert torch.equal(a["block_tables"], b["block_tables"])
    assert torch.equal(a["slot_mapping"], b["slot_mapping"])
    # both are roundings of the same fp32 draws: they agree to bf16 precision
    assert (a["k_cache"].float() - b["k_cache"].float()).abs().max() <= 2.0 ** -7 * 4
