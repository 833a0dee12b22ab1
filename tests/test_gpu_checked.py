"""The checked build (libpagedkv_checked.so, PAGEDKV_CHECKED) on the GPU.

Every entry point of the checked library first validates, on the device, the data it reads;
the first violation is kept in a per-device record that paged_kv_check_status reads. These
tests route the Python binding to the checked library and feed it invalid slot ids, block
ids, lengths and query spans of the kinds the kernels are documented to stay memory-safe on
(an out-of-pool slot is not written, an out-of-pool block id is not read, a length is clamped
to the table width, a query row before position 0 sees no key), and expect the record to name
the entry. Valid inputs leave the record empty and give the unchecked library's results bit
for bit: the attention kernels are the same.
"""
import os

import pytest
import torch

from paged_kv_decode_write_amd import _binding as pk
from paged_kv_decode_write_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pk.load_library()
    if not os.path.exists(pk.checked_library_path()):
        raise FileNotFoundError("libpagedkv_checked.so is missing: build it first")
    return torch.device("cuda:0")


@pytest.fixture()
def checked(dev, monkeypatch):
    """The binding's calls go to the checked library for the test's duration; the record
    starts empty."""
    lib = pk.load_checked_library()
    assert lib.paged_kv_checked_build() == 1
    monkeypatch.setattr(pk, "_lib", lib)
    pk.check_status(lib)  # clear
    return lib


def _decode_inputs(dev):
    w = wl.WORKLOADS["c2"]
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
         for k, v in wl.make_inputs(w).items()}
    d["out"] = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    return w, d


def _attend(d, partition=0):
    pk.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                              d["context_lens"], d["scale"], d["out"],
                              partition_tokens=partition)
    return d["out"].clone()


def test_valid_inputs_leave_the_record_empty_and_match_the_default_library(dev, checked,
                                                                           monkeypatch):
    w, d = _decode_inputs(dev)
    kc0, vc0 = d["k_cache"].clone(), d["v_cache"].clone()
    pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])
    outs = [_attend(d, p) for p in (0, -1, 256)]
    pk.paged_decode_step(d["q"], d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"],
                         d["v_cache"], d["block_tables"], d["context_lens"], d["scale"],
                         d["out"])
    outs.append(d["out"].clone())
    assert pk.check_status(checked) == ("none", 0, 0)
    # the same calls on the default library
    monkeypatch.setattr(pk, "_lib", None)
    pk.load_library()
    kc, vc = kc0.clone(), vc0.clone()
    pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], kc, vc)
    assert torch.equal(kc, d["k_cache"]) and torch.equal(vc, d["v_cache"])
    ref = [_attend(d, p) for p in (0, -1, 256)]
    for a, b in zip(outs[:3], ref):
        assert torch.equal(a, b)
    assert torch.equal(outs[3], ref[0])


def test_out_of_pool_slot_is_recorded_and_not_written(dev, checked):
    w, d = _decode_inputs(dev)
    num_slots = w.num_blocks * w.block_size
    slots = d["slot_mapping"].clone()
    slots[3] = num_slots + 5
    kc0 = d["k_cache"].clone()
    pk.paged_kv_write(d["k_new"], d["v_new"], slots, d["k_cache"], d["v_cache"])
    assert pk.check_status(checked) == ("slot", 3, num_slots + 5)
    # the other three rows are written, nothing else changes
    changed = (d["k_cache"] != kc0).flatten(1).any(1).nonzero().flatten().tolist()
    want = sorted({int(s) // w.block_size for s in d["slot_mapping"][:3].tolist()})
    assert sorted(changed) == want
    assert pk.check_status(checked) == ("none", 0, 0)  # the read above cleared it


def test_out_of_pool_block_id_is_recorded(dev, checked):
    w, d = _decode_inputs(dev)
    tables = d["block_tables"].clone()
    tables[2, 1] = w.num_blocks + 7  # covered: sequence 2 spans all of its 32 blocks
    d["block_tables"] = tables
    for p in (0, -1):
        _attend(d, p)
        assert pk.check_status(checked) == ("block", 2 * w.max_blocks + 1, w.num_blocks + 7)


def test_table_entries_past_the_context_are_not_checked(dev, checked):
    w, d = _decode_inputs(dev)
    lens = d["context_lens"].clone()
    lens[0] = 20  # two blocks covered; the rest of row 0 is never read
    tables = d["block_tables"].clone()
    tables[0, 2:] = -1
    tables[0, 5] = w.num_blocks + 100
    d["context_lens"], d["block_tables"] = lens, tables
    _attend(d)
    assert pk.check_status(checked) == ("none", 0, 0)


def test_length_past_the_table_is_recorded(dev, checked):
    w, d = _decode_inputs(dev)
    lens = d["context_lens"].clone()
    lens[1] = w.max_blocks * w.block_size + 3
    d["context_lens"] = lens
    _attend(d)
    assert pk.check_status(checked) == ("length", 1, w.max_blocks * w.block_size + 3)


def test_fused_step_checks_its_slots_and_keeps_the_first_violation(dev, checked):
    w, d = _decode_inputs(dev)
    slots = d["slot_mapping"].clone()
    slots[0] = 1 << 40
    pk.paged_decode_step(d["q"], d["k_new"], d["v_new"], slots, d["k_cache"], d["v_cache"],
                         d["block_tables"], d["context_lens"], d["scale"], d["out"])
    # a second violation before the record is read does not replace the first
    lens = d["context_lens"].clone()
    lens[2] = -4
    d["context_lens"] = lens
    _attend(d)
    assert pk.check_status(checked) == ("slot", 0, 1 << 40)


def _prefill(d, lens=None, max_q_len=None):
    w = wl.PREFILL_WORKLOADS["p3"]
    out = torch.empty_like(d["q"], dtype=torch.float32)
    pk.paged_prefill_attention(d["q"], d["cu_seqlens_q"], d["k_cache"], d["v_cache"],
                               d["block_tables"], d["context_lens"] if lens is None else lens,
                               d["scale"], out,
                               max_q_len=max(w.query_lens) if max_q_len is None else max_q_len)
    return out


def test_prefill_query_spans_are_checked(dev, checked):
    w = wl.PREFILL_WORKLOADS["p3"]
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
         for k, v in wl.make_prefill_inputs(w).items()}
    _prefill(d)
    assert pk.check_status(checked) == ("none", 0, 0)
    lens = d["context_lens"].clone()
    lens[0] = 1024  # 2048 query rows on a 1024-token context: half of them before position 0
    _prefill(d, lens=lens)
    assert pk.check_status(checked) == ("query", 0, 2048)
    _prefill(d, max_q_len=1024)  # spans longer than the grid the call was sized for
    code, index, value = pk.check_status(checked)
    assert code == "query" and index in (0, 1) and value == 2048
