"""The seeded input generator: shapes, determinism and the block-table / slot recipe."""
import numpy as np
import pytest
import torch

from paged_kv_decode_write_amd import workloads as wl


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_shapes_tables_and_slots(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    B, Hq, Hkv, D, bs, NB, MB = (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                 w.block_size, w.num_blocks, w.max_blocks)
    assert inp["q"].shape == (B, Hq, D) and inp["q"].dtype == torch.bfloat16
    assert inp["k_cache"].shape == (NB, bs, Hkv, D)
    assert inp["k_new"].shape == (B, Hkv, D)
    tables, lens, slots = inp["block_tables"], inp["context_lens"], inp["slot_mapping"]
    assert tables.dtype == torch.int32 and lens.dtype == torch.int32 and slots.dtype == torch.int64
    used = []
    for b in range(B):
        L = int(lens[b])
        n = (L + bs - 1) // bs
        assert 1 <= L <= MB * bs
        row = tables[b].tolist()
        assert all(0 <= x < NB for x in row[:n]) and all(x == -1 for x in row[n:])
        used += row[:n]
        assert int(slots[b]) == row[(L - 1) // bs] * bs + (L - 1) % bs
    assert len(set(used)) == len(used)  # no physical block shared


def test_deterministic_and_seed_dependent():
    w = wl.WORKLOADS["c2"]
    a, b = wl.make_inputs(w), wl.make_inputs(w)
    for key in ("q", "k_cache", "v_cache", "k_new", "v_new", "block_tables", "slot_mapping"):
        assert torch.equal(a[key].view(torch.int16) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.int16) if b[key].dtype == torch.bfloat16 else b[key])
    import dataclasses
    c = wl.make_inputs(dataclasses.replace(w, seed=w.seed + 1))
    assert not torch.equal(a["q"], c["q"])


def test_ragged_lengths_range_and_q_scale():
    w = wl.WORKLOADS["c4"]
    lens = wl.make_inputs(w)["context_lens"]
    assert int(lens.min()) >= 1 and int(lens.max()) <= 4096
    assert (lens % 16 != 0).any()  # partial last blocks occur
    # q drawn with std 3 gives logits of std ~3 against N(0,1) keys at scale 1/sqrt(D)
    w5 = wl.Workload("q3", batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                     num_blocks=64, max_blocks=1, seed=9, context_len=16, q_std=3.0)
    q = wl.make_inputs(w5)["q"].float()
    assert 2.9 < float(q.std()) < 3.1


def test_poison_marks_only_unread_slots():
    w = wl.Workload("p", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                    num_blocks=10, max_blocks=3, seed=3, max_context_len=11)
    clean = wl.make_inputs(w)
    dirty = wl.make_inputs(w, poison=True)
    kb, kd = clean["k_cache"].view(torch.int16), dirty["k_cache"].view(torch.int16)
    tables, lens = clean["block_tables"], clean["context_lens"]
    read = torch.zeros(10, 4, dtype=torch.bool)
    for b in range(3):
        for t in range(int(lens[b])):
            read[int(tables[b, t // 4]), t % 4] = True
    assert torch.equal(kb[read], kd[read])
    assert (kd[~read] == wl.BF16_QNAN_BITS).all()


def test_algorithmic_bytes_formula():
    w = wl.WORKLOADS["c5a"]
    ab = wl.algorithmic_bytes(w, [8192] * 64)
    assert ab["attention"] == 2_149_056_512
    ab = wl.algorithmic_bytes(wl.WORKLOADS["c5b"], [32768] * 2)
    assert ab["attention"] == 268_484_608
