"""paged_decode_step_noalloc (no workspace argument: the split partials and the block-table
view live in the library's static device scratch) against paged_decode_step with a workspace
of its own, through the C ABI. Two calls in a row share the scratch, the second with a
smaller input; each must equal the workspace call bit for bit (same kernels, same plan) and
the oracle within the attention bound, with pools bit-identical to the oracle's write."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_write_amd import _binding as pk
from paged_kv_decode_write_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pk.load_library()
    return torch.device("cuda:0")


def step_pair(w, dev, partition, kernel="auto"):
    """Run both entry points on identical copies of workload w's inputs; compare."""
    inp = wl.make_inputs(w, poison=True)
    host = wl.to_host_numpy(inp)
    ref, kc_ref, vc_ref = oracle.decode_step(host)
    a = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    b = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    shape = (w.batch, w.num_q_heads, w.head_dim)
    out_a = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    out_b = torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
    ws = pk.new_workspace(pk.decode_workspace_bytes(w.batch, w.num_q_heads, w.head_dim,
                                                    w.max_blocks, w.block_size, partition), dev)
    args = lambda d: (d["q"], d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"],
                      d["v_cache"], d["block_tables"], d["context_lens"], d["scale"])
    print(f"[no-alloc] {w.name} bs={w.block_size} partition={partition} kernel={kernel}",
          flush=True)
    pk.paged_decode_step(*args(a), out_a, partition_tokens=partition, kernel=kernel,
                         workspace=ws)
    pk.paged_decode_step_noalloc(*args(b), out_b, partition_tokens=partition, kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), (w.name, partition)
    assert np.array_equal(wl.to_bits(b["k_cache"]), kc_ref)
    assert np.array_equal(wl.to_bits(b["v_cache"]), vc_ref)
    err = np.abs(out_b.cpu().double().numpy() - ref).max()
    assert err <= ATOL, (w.name, partition, err)
    return pk.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_blocks,
                          w.block_size, partition, kernel)[0]


def test_noalloc_matches_workspace_call_twice_second_smaller(dev):
    # ragged 48-sequence batch, split automatically, then a smaller 4 x 512 batch
    assert step_pair(wl.WORKLOADS["c4"], dev, 0) > 1
    assert step_pair(wl.WORKLOADS["c2"], dev, 256) > 1


def test_noalloc_forced_split_then_smaller_and_larger_blocks(dev):
    assert step_pair(wl.WORKLOADS["c3"], dev, 256, "mfma_hw") > 1
    assert step_pair(wl.WORKLOADS["c1"], dev, 32, "mfma") > 1
    # 32-token blocks: the table of 16-token block ids goes into the scratch too
    base = wl.WORKLOADS["c2"]
    w32 = dataclasses.replace(base, name="c2_bs32", block_size=32,
                              max_blocks=base.max_blocks // 2, num_blocks=base.num_blocks // 2)
    step_pair(w32, dev, -1)
    step_pair(w32, dev, 0, "valu")


def test_noalloc_rejects_a_plan_beyond_the_scratch(dev):
    """64 sequences x 8192 tokens cut into 16-token partitions need 64*32*512*130*4 bytes of
    partials, far past the scratch: refused on the host before any launch."""
    B, Hq, Hkv, D, MB = 64, 32, 8, 128, 512
    bf = dict(dtype=torch.bfloat16, device=dev)
    q = torch.zeros(B, Hq, D, **bf)
    kn = torch.zeros(B, Hkv, D, **bf)
    pool = torch.zeros(1, 16, Hkv, D, **bf)
    slots = torch.full((B,), -1, dtype=torch.int64, device=dev)
    tables = torch.zeros(B, MB, dtype=torch.int32, device=dev)
    lens = torch.full((B,), 16, dtype=torch.int32, device=dev)
    out = torch.zeros(B, Hq, D, dtype=torch.float32, device=dev)
    with pytest.raises(pk.PagedKVError) as e:
        pk.paged_decode_step_noalloc(q, kn, kn, slots, pool, pool, tables, lens, 0.1, out,
                                     partition_tokens=16)
    assert e.value.status == 4 and "static scratch" in str(e.value)
