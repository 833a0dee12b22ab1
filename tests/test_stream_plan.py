"""The stream family's work division, on the CPU: the partial slots and least slice the
library plans (paged_decode_plan, host logic) must suffice for every batch the kernel may see.

The kernel (csrc/decode_sk.hip) counts items = 32-token pairs of (sequence, group of 4 KV heads),
sequence-major, gives workgroup w of N the slice [w q, (w + 1) q) with q = max(min_pairs,
ceil(W / N)), and writes the segment of (sequence b, head group) that slice w holds into slot
w - first_item(b, head group) // q; the workgroup closing a (sequence, head group) marks its
later slots empty. This test replays that division with the planned (slots, min_pairs) and
checks, over random ragged batches (empty, partial-block and over-long contexts included), that
every pair is covered exactly once, every slot index is in range and every slot is written
exactly once per call.
"""
import os
import random

import pytest

from paged_kv_decode_write_amd import _binding

HPW, PT = 4, 32


@pytest.fixture()
def plan(monkeypatch):
    if not os.path.exists(_binding.library_path()):
        pytest.skip("libpagedkv.so not built")
    monkeypatch.setenv("PAGEDKV_CU_COUNT", "256")

    def f(B, Hkv, MB, part):
        n, tokens, k = _binding.decode_plan(B, 4 * Hkv, Hkv, 128, MB, 16, part, "mfma_sk",
                                            with_kernel=True)
        assert k == "mfma_sk"
        return n, tokens // PT
    return f


def replay(lens, Hkv, MB, N, slots, min_pairs):
    Lmax = MB * 16
    ngrp = -(-Hkv // HPW)
    cl = [max(0, min(L, Lmax)) for L in lens]
    pairs = [-(-L // PT) for L in cl]
    W = sum(pairs) * ngrp
    q = max(min_pairs, -(-W // N))
    written, covered = {}, set()
    first_of = {}
    S = 0
    for b, p in enumerate(pairs):
        for hg in range(ngrp):
            first_of[(b, hg)] = S + hg * p
        S += p * ngrp
    for b in range(len(lens)):          # empty sequences: every slot marked
        if pairs[b] == 0:
            for g in range(Hkv):
                for s in range(slots):
                    written[(b, g, s)] = written.get((b, g, s), 0) + 1
    for w in range(N):
        lo, hi = w * q, min(w * q + q, W)
        item = lo
        while item < hi:
            # the (sequence, head group) holding `item`
            b, hg = next((b, hg) for (b, hg), f in first_of.items()
                         if pairs[b] and f <= item < f + pairs[b])
            first = first_of[(b, hg)]
            e = min(hi, first + pairs[b])
            slot = w - first // q
            assert 0 <= slot < slots, (slot, slots)
            for g in range(hg * HPW, min(hg * HPW + HPW, Hkv)):
                written[(b, g, slot)] = written.get((b, g, slot), 0) + 1
                for k in range(item - first, e - first):
                    assert (b, g, k) not in covered
                    covered.add((b, g, k))
                if e == first + pairs[b]:
                    for s in range(slot + 1, slots):
                        written[(b, g, s)] = written.get((b, g, s), 0) + 1
            item = e
    for b in range(len(lens)):
        for g in range(Hkv):
            assert all((b, g, k) in covered for k in range(pairs[b]))
            assert all(written.get((b, g, s)) == 1 for s in range(slots)), (b, g)


def test_planned_slots_cover_random_batches(plan):
    rng = random.Random(7)
    for _ in range(300):
        B = rng.randint(1, 80)
        MB = rng.choice([65, 80, 128, 256, 300])
        Hkv = rng.choice([1, 2, 4, 8, 12])
        part = rng.choice([0, 0, 0, 16, 32, 48, 64, 256, 4096])
        slots, min_pairs = plan(B, Hkv, MB, part)
        lens = [rng.choice([0, 1, 15, 16, 17, 31, 32, 33, rng.randint(0, MB * 16), MB * 16,
                            MB * 16 + 5]) for _ in range(B)]
        N = rng.choice([1, 3, 64, 512])
        replay(lens, Hkv, MB, N, slots, min_pairs)


def test_automatic_slots_are_at_most_sixteen(plan):
    for MB in (65, 128, 256, 512, 2048, 8192):
        slots, min_pairs = plan(8, 8, MB, 0)
        assert slots <= 16 and min_pairs >= 8
