"""The stream family's work division, on the CPU: the partial slots and least slice the
library plans (paged_decode_plan, host logic) must suffice for every batch the kernel may see.

The kernel (csrc/decode_sk.hip) counts items = 32-token pairs of (sequence, group of 4 KV heads),
sequence-major, gives workgroup w of N the slice [start(w), start(w + 1)), and writes the
segment of (sequence b, head group) that slice w holds into slot w - (the slice holding
first_item(b, head group)); the workgroup closing a (sequence, head group) marks its later slots
empty. Equal slices: start(w) = min(w q, W), q = max(min_pairs, ceil(W / N)). XCD-weighted
slices (the whole device): weights 507 for even w and 493 for odd w, start(w) = round(W c(w) /
c(N)) with c(w) the weight of workgroups 0 .. w-1, used only when W * 493 >= (min_pairs + 1) *
c(N). This test replays both divisions with the planned (slots, min_pairs) and checks, over
random ragged batches (empty, partial-block and over-long contexts included), that every pair
is covered exactly once, every slot index is in range, every slot is written exactly once per
call and every weighted slice holds at least min_pairs items.
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


EVEN, ODD = 507, 493


def division(W, N, min_pairs, xcd):
    """start(v) of the kernel's slices, and whether the weighted form applies."""
    q = max(min_pairs, -(-W // N))

    def c(v):
        return (v // 2) * (EVEN + ODD) + (v % 2) * EVEN
    weighted = xcd and W * ODD >= (min_pairs + 1) * c(N)
    if weighted:
        return (lambda v: (W * c(v) + c(N) // 2) // c(N)), True
    return (lambda v: min(v * q, W)), False


def replay(lens, Hkv, MB, N, slots, min_pairs, xcd=False):
    Lmax = MB * 16
    ngrp = -(-Hkv // HPW)
    cl = [max(0, min(L, Lmax)) for L in lens]
    pairs = [-(-L // PT) for L in cl]
    W = sum(pairs) * ngrp
    start, weighted = division(W, N, min_pairs, xcd)
    bounds = [start(v) for v in range(N + 1)]
    assert bounds[0] == 0 and bounds[N] == W
    assert all(bounds[v] <= bounds[v + 1] for v in range(N))
    if weighted:
        assert all(bounds[v + 1] - bounds[v] >= min_pairs for v in range(N))

    def slice_of(x):  # the slice holding item x, by search
        return next(v for v in range(N) if bounds[v] <= x < bounds[v + 1])
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
        lo, hi = bounds[w], bounds[w + 1]
        item = lo
        while item < hi:
            # the (sequence, head group) holding `item`
            b, hg = next((b, hg) for (b, hg), f in first_of.items()
                         if pairs[b] and f <= item < f + pairs[b])
            first = first_of[(b, hg)]
            e = min(hi, first + pairs[b])
            slot = w - slice_of(first)
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
        N = rng.choice([1, 3, 64, 256, 512])
        replay(lens, Hkv, MB, N, slots, min_pairs)
        replay(lens, Hkv, MB, N, slots, min_pairs, xcd=True)


def test_automatic_slots_are_at_most_sixteen(plan):
    for MB in (65, 128, 256, 512, 2048, 8192):
        slots, min_pairs = plan(8, 8, MB, 0)
        assert slots <= 16 and min_pairs >= 8


def test_weighted_slices_balance_the_xcds():
    """The weighted division gives every slice its share W * weight / c(N) within one item
    (slices on even XCDs 507/493 of those on odd ones), and applies to the benchmark-sized
    batches: on the 64 x 8192 batch (32768 items) 130 and 126 items."""
    for W in (32768, 6912, 4096):
        start, weighted = division(W, 256, 8, True)
        assert weighted
        cN = 128 * (EVEN + ODD)
        for v in range(256):
            share = W * (EVEN if v % 2 == 0 else ODD) / cN
            assert abs(start(v + 1) - start(v) - share) < 1, (W, v)
    start, _ = division(32768, 256, 8, True)
    assert (start(1), start(2) - start(1)) == (130, 126)
    start, weighted = division(2000, 256, 8, True)  # slices would fall below min_pairs
    assert not weighted and start(1) == 8
