"""The host-side launch plan (kernel family, partitions per sequence, tokens per partition),
without a device: PAGEDKV_CU_COUNT stands in for the device's compute-unit count (256 on
MI355X). Expected values are worked out by hand from the planning rule documented in the
library (comments of make_plan and select_kernel in csrc/api.cpp):
  * contexts over 1024 tokens (max_blocks * block_size) use the one-wave-per-KV-head MFMA
    kernel, or the stream family when batch * kv_heads exceeds a quarter of the CUs, the
    split is left automatic and the head-per-wave plan has more workgroups than CUs; shorter
    ones the split-wave MFMA kernel;
  * target work: 4 workgroups per CU (split-wave), 8 waves per CU (head-wave), or 4 when the
    batch * kv_heads units are at most a quarter of the CUs;
  * n = min(ceil(target / units), ceil(max_len / 256)), tokens per partition rounded up to the
    kernel's granule (128 split-wave, 32 head-wave), n recomputed from it.
"""
import pytest

from paged_kv_decode_write_amd import _binding
from paged_kv_decode_write_amd import workloads as wl

import os


@pytest.fixture()
def plan(monkeypatch):
    if not os.path.exists(_binding.library_path()):
        pytest.skip("libpagedkv.so not built")
    monkeypatch.setenv("PAGEDKV_CU_COUNT", "256")

    def f(w, partition=0, kernel="auto"):
        return _binding.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    w.max_blocks, w.block_size, partition, kernel,
                                    with_kernel=True)
    return f


# (workload, partitions, tokens per partition, kernel), derived per the module docstring:
#  c1: 128 tokens -> mfma; n = min(ceil(1024/8), ceil(128/256)=1) = 1, P = 128
#  c2: 512 -> mfma; n = min(32, 2) = 2, P = roundup(256, 128) = 256
#  c3: 2048 -> mfma_hw; units 128 (x4 > 256): n = min(ceil(2048/128)=16, 8) = 8, P = 256;
#      16 x 2 head groups x 8 = 256 workgroups, not more than the 256 CUs: kept
#  c4: 4096, units 384: head-per-wave n = min(ceil(2048/384)=6, 16) = 6 gives 48 x 2 x 6 = 576
#      workgroups, more than the CUs: the stream family, whose slots and least pairs per
#      workgroup come from pairs_max = max_len / 32 alone:
#      q = max(8, ceil((pairs_max - 1) / 14)) = 10, slots (128 - 1) // 10 + 2 = 14, 320 tokens
#  c5a: 8192, units 512: head-per-wave n = min(4, 32) = 4 gives 64 x 2 x 4 = 512 workgroups:
#      the stream family, q = max(8, ceil(255 / 14)) = 19, slots 255 // 19 + 2 = 15, 608 tokens
#  c5b: 32768 -> mfma_hw; units 16 (x4 <= 256): n = min(ceil(1024/16)=64, 128) = 64, P = 512
EXPECTED = {"c1": (1, 128, "mfma"), "c2": (2, 256, "mfma"), "c3": (8, 256, "mfma_hw"),
            "c4": (14, 320, "mfma_sk"), "c5a": (15, 608, "mfma_sk"),
            "c5b": (64, 512, "mfma_hw")}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_automatic_plan_of_each_workload(plan, name):
    assert plan(wl.WORKLOADS[name]) == EXPECTED[name]


def test_forced_partitions_and_kernels(plan):
    w = wl.WORKLOADS["c5b"]
    assert plan(w, -1) == (1, 32768, "mfma_hw")               # never split
    assert plan(w, 1024) == (32, 1024, "mfma_hw")             # forced size
    # split-wave: target 4 * 256 = 1024 groups over 16 units -> n = 64, P = roundup(512, 128)
    assert plan(w, 0, "mfma") == (64, 512, "mfma")
    assert plan(w, 0, "valu")[2] == "valu"
    with pytest.raises(_binding.PagedKVError):
        plan(w, 24)                                           # not a multiple of block_size
    g5 = wl.Workload("g5", batch=2, num_q_heads=40, num_kv_heads=8, head_dim=128, block_size=16,
                     num_blocks=64, max_blocks=8, seed=1, context_len=128)
    assert plan(g5)[2] == "mfma"                              # the matrix-core kernel takes G = 5
    with pytest.raises(_binding.PagedKVError):
        plan(g5, 0, "valu")                                   # the vector-ALU kernel does not


def test_plan_scales_with_the_compute_units(plan, monkeypatch):
    w = wl.WORKLOADS["c5a"]
    monkeypatch.setenv("PAGEDKV_CU_COUNT", "128")
    # head-per-wave, units 512: target 8 * 128 = 1024 waves -> n = 2, P = 4096
    assert plan(w, 0, "mfma_hw") == (2, 4096, "mfma_hw")
    # c5b's 16 units (x4 <= 128): head-per-wave, 4 * 128 waves -> n = 32, P = 1024
    assert plan(wl.WORKLOADS["c5b"]) == (32, 1024, "mfma_hw")
    # with 24 CUs the 16 units exceed a quarter of them; head-per-wave targets 8 * 24 waves ->
    # n = 12 (P = 2752 -> n = 12), 2 x 2 x 12 = 48 workgroups, more than the 24 CUs: the
    # stream family, pairs_max 1024, q = max(8, ceil(1023 / 14)) = 74, slots 1023 // 74 + 2 =
    # 15, 2368 tokens
    monkeypatch.setenv("PAGEDKV_CU_COUNT", "24")
    assert plan(wl.WORKLOADS["c5b"]) == (15, 2368, "mfma_sk")
    assert plan(wl.WORKLOADS["c5b"], 0, "mfma_hw") == (12, 2752, "mfma_hw")
    # with 64 CUs: 16 units are exactly a quarter: head-per-wave, 4 * 64 waves -> n = 16
    monkeypatch.setenv("PAGEDKV_CU_COUNT", "64")
    assert plan(wl.WORKLOADS["c5b"]) == (16, 2048, "mfma_hw")


def test_stream_family_forced(plan):
    w = wl.WORKLOADS["c4"]
    assert plan(w, 0, "mfma_sk") == (14, 320, "mfma_sk")
    # partition_tokens > 0: the least tokens per workgroup (2 pairs), slots 127 // 2 + 2 = 65
    assert plan(w, 64, "mfma_sk") == (65, 64, "mfma_sk")
    with pytest.raises(_binding.PagedKVError):
        plan(w, -1, "mfma_sk")                                # always splits
    with pytest.raises(_binding.PagedKVError):
        plan(wl.WORKLOADS["c2"], 0, "mfma_sk")                # 512 tokens: too short
    assert plan(w, -1) == (1, 4096, "mfma_hw")                # auto never picks it for -1
    assert plan(w, 256) == (16, 256, "mfma_hw")               # nor for a forced size


# Multi-query (prefill) plans, from the rule documented beside make_prefill_plan: split when
# kv_heads * ceil(num_tokens / tokens per workgroup) < 2 * 2 * CUs and the contexts may exceed
# 2048 keys, into ceil(max_len / P) partitions, P = max(512, roundup(ceil(max_len / 3), 32)).
# row_blocks is passed explicitly (its automatic choice asks the device for occupancy).
#  p1: 8 kv heads * ceil(4096 / 32) = 1024 workgroups, not < 1024: no split
#  p2: 8 * ceil(1438 / 20) = 576 < 1024 and 4096 keys: P = roundup(1366, 32) = 1376, 3 partitions
#  p3: 2048 keys: never split automatically
PREFILL_EXPECTED = {"p1": (2, 1, 4096), "p2": (1, 3, 1376), "p3": (1, 1, 2048)}


def _prefill_plan(w, row_blocks, partition=0):
    return _binding.prefill_plan(sum(w.query_lens), max(w.query_lens), len(w.context_lens),
                                 w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_blocks,
                                 w.block_size, row_blocks, partition)


@pytest.mark.parametrize("name", sorted(PREFILL_EXPECTED))
def test_prefill_plan_of_each_workload(plan, name):
    exp = PREFILL_EXPECTED[name]
    assert _prefill_plan(wl.PREFILL_WORKLOADS[name], exp[0]) == exp


def test_prefill_plan_forced_and_scaled(plan, monkeypatch):
    w = wl.PREFILL_WORKLOADS["p2"]
    assert _prefill_plan(w, 1, 512) == (1, 8, 512)
    assert _prefill_plan(w, 1, -1) == (1, 1, 4096)
    assert _prefill_plan(w, 1, 8192) == (1, 1, 4096 // 32 * 32)   # one partition: no split
    with pytest.raises(_binding.PagedKVError):
        _prefill_plan(w, 1, 48)                                    # not a multiple of 32
    # four times the compute units: p1's 1024 workgroups no longer fill two rounds
    monkeypatch.setenv("PAGEDKV_CU_COUNT", "1024")
    assert _prefill_plan(wl.PREFILL_WORKLOADS["p1"], 2) == (2, 3, 1376)


@pytest.mark.parametrize("name", ["c2", "c4", "c5b"])
@pytest.mark.parametrize("block_size", [32, 64])
def test_larger_blocks_plan_as_their_16_token_view(plan, name, block_size):
    """Blocks of 16k tokens are attended as 16-token blocks: the plan (kernel, partitions,
    tokens per partition) is that of the same context length in 16-token blocks."""
    import dataclasses
    w = wl.WORKLOADS[name]
    k = block_size // 16
    big = dataclasses.replace(w, block_size=block_size, max_blocks=w.max_blocks // k,
                              num_blocks=w.num_blocks // k)
    assert plan(big) == plan(w)
    assert plan(big, -1) == plan(w, -1)
    assert plan(big, 4 * block_size) == plan(w, 4 * block_size)
