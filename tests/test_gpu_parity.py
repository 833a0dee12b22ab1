"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

KV write: the whole pools must be bit-identical to the oracle's. Attention: max |out - oracle|
must stay within 2e-3 (fp32 output against the float64 oracle), in automatic, forced-split
and never-split modes, for every kernel family built for the shape. Every workload, the
full-size long-context pair (64 x 8192 and 2 x 32768 tokens) and the chunked prefill
included, is compared on every output row; properties that hold at any size (split vs unsplit
agreement, unread slots never matter, determinism) are checked beside it.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_write_amd import _binding as pk
from paged_kv_decode_write_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3
SUMMARY = {}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pk.load_library()  # with a GPU present, a missing library is an error, not a skip
    return torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _write_summary():
    yield
    path = os.environ.get("PAGEDKV_PARITY_SUMMARY")
    if path:
        os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
        with open(path, "w") as f:
            json.dump(SUMMARY, f, indent=1, sort_keys=True)


def kernels_for(w):
    out = []
    for k in ("valu", "mfma", "mfma_hw", "mfma_sk"):
        try:
            pk.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_blocks,
                           w.block_size, 0, k)
            out.append(k)
        except pk.PagedKVError:
            pass
    assert out, f"no kernel for {w}"
    return out


def part_for(kernel, partition):
    """partition_tokens for a kernel family: the stream family always leaves partials, so
    where a test asks for no split (-1) it runs with the family's own automatic slices."""
    return 0 if kernel == "mfma_sk" and partition == -1 else partition


def to_dev(inp, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_write(d):
    pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])


def run_attention(d, kernel="auto", partition=0):
    w = d["workload"]
    out = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32,
                     device=d["q"].device)
    pk.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                              d["context_lens"], d["scale"], out,
                              partition_tokens=part_for(kernel, partition),
                              kernel=kernel)
    return out


def record(key, err):
    SUMMARY[key] = float(err)
    print(f"[parity] {key}: max|err| = {err:.3e}", flush=True)


_CASES = {}


def case(name, dev, poison=False):
    """(host numpy inputs, oracle out, oracle pools after the write, device inputs after the
    GPU write) for a workload; drawn once per session. The write is idempotent, so tests may
    repeat it on the device copy."""
    key = (name, poison)
    if key not in _CASES:
        inp = wl.make_inputs(wl.WORKLOADS[name], poison=poison)
        host = wl.to_host_numpy(inp)
        out, kc, vc = oracle.decode_step(host)
        d = to_dev(inp, dev)
        run_write(d)
        torch.cuda.synchronize()
        _CASES[key] = (host, out, kc, vc, d)
    return _CASES[key]


SMALL = ["c1", "c2", "c3", "c4"]


# ------------------------------------------------------------------------------ KV write
@pytest.mark.parametrize("name", SMALL)
def test_kv_write_bit_exact_full_pool(dev, name):
    host, _, kc_ref, vc_ref, d = case(name, dev)
    assert np.array_equal(wl.to_bits(d["k_cache"]), kc_ref)
    assert np.array_equal(wl.to_bits(d["v_cache"]), vc_ref)


@pytest.mark.parametrize("name", ["c5a", "c5b"])
def test_kv_write_bit_exact_full_size(dev, name):
    w = wl.WORKLOADS[name]
    d = wl.make_inputs(w, device="cuda")
    kc0, vc0 = wl.to_bits(d["k_cache"]), wl.to_bits(d["v_cache"])
    run_write(d)
    torch.cuda.synchronize()
    kc_ref, vc_ref = oracle.kv_write(wl.to_bits(d["k_new"]), wl.to_bits(d["v_new"]),
                                     d["slot_mapping"].cpu().numpy(), kc0, vc0)
    del kc0, vc0
    assert np.array_equal(wl.to_bits(d["k_cache"]), kc_ref)
    assert np.array_equal(wl.to_bits(d["v_cache"]), vc_ref)


def test_kv_write_skips_negative_slots_and_keeps_nan_payloads(dev):
    w = wl.Workload("neg", batch=6, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                    num_blocks=32, max_blocks=4, seed=77, max_context_len=60)
    inp = wl.make_inputs(w)
    inp["slot_mapping"][[1, 4]] = -1
    inp["k_new"].view(torch.int16)[0, 0, 0] = 0x7FA1  # a NaN with a payload
    host = wl.to_host_numpy(inp)
    kc_ref, vc_ref = oracle.kv_write(host["k_new"], host["v_new"], host["slot_mapping"],
                                     host["k_cache"], host["v_cache"])
    d = to_dev(inp, dev)
    run_write(d)
    torch.cuda.synchronize()
    assert np.array_equal(wl.to_bits(d["k_cache"]), kc_ref)
    assert np.array_equal(wl.to_bits(d["v_cache"]), vc_ref)


def test_kv_write_zero_tokens_is_noop(dev):
    kc = torch.randn(4, 16, 2, 64, device=dev).to(torch.bfloat16)
    before = kc.clone()
    e = torch.empty(0, 2, 64, dtype=torch.bfloat16, device=dev)
    pk.paged_kv_write(e, e, torch.empty(0, dtype=torch.int64, device=dev), kc, kc)
    torch.cuda.synchronize()
    assert torch.equal(kc, before)


# ----------------------------------------------------------------------------- attention
@pytest.mark.parametrize("partition", [0, -1, 64, 256])
@pytest.mark.parametrize("name", SMALL)
def test_attention_parity(dev, name, partition):
    host, ref, _, _, d = case(name, dev)
    w = wl.WORKLOADS[name]
    for kernel in kernels_for(w):
        run_write(d)
        out = run_attention(d, kernel, partition).cpu().double().numpy()
        err = np.abs(out - ref).max()
        record(f"{name}/{kernel}/p{partition}", err)
        assert np.isfinite(out).all()
        assert err <= ATOL, (name, kernel, partition, err)


@pytest.mark.parametrize("name", SMALL)
def test_attention_poisoned_pool_matches_clean(dev, name):
    """Quiet-NaN bits in every slot attention must not read leave the output unchanged."""
    w = wl.WORKLOADS[name]
    _, _, _, _, clean = case(name, dev)
    _, ref, _, _, dirty = case(name, dev, poison=True)
    for kernel in kernels_for(w):
        for partition in (0, -1, 64):
            o1 = run_attention(clean, kernel, partition)
            o2 = run_attention(dirty, kernel, partition)
            assert torch.equal(o1, o2), (name, kernel, partition)
            err = np.abs(o2.cpu().double().numpy() - ref).max()
            assert err <= ATOL


def full_size_case(name):
    """A full-size workload drawn on the device (its pools are up to 1 GiB each), and the
    oracle's whole decode step on host copies of it: the pools after the oracle's write, and
    every output row."""
    w = wl.WORKLOADS[name]
    d = wl.make_inputs(w, device="cuda")
    host = wl.to_host_numpy(d)
    ref, kc_ref, vc_ref = oracle.decode_step(host)
    del host
    return d, ref, kc_ref, vc_ref


@pytest.mark.parametrize("name", ["c5a", "c5b"])
def test_full_size_every_row_against_the_oracle(dev, name):
    """The long-context workloads at full size, every (sequence, query head) row against the
    float64 oracle: the fused decode step the benchmark times (pools bit-identical to the
    oracle's write), then separate attention calls of every kernel family, automatic, never
    and forced splits, and the fused step again with every family. Properties: every call
    agrees with the unsplit one."""
    w = wl.WORKLOADS[name]
    d, ref, kc_ref, vc_ref = full_size_case(name)
    out = run_step(d)
    torch.cuda.synchronize()
    assert np.array_equal(wl.to_bits(d["k_cache"]), kc_ref)
    assert np.array_equal(wl.to_bits(d["v_cache"]), vc_ref)
    del kc_ref, vc_ref
    o = out.cpu().double().numpy()
    assert np.isfinite(o).all()
    err = np.abs(o - ref).max()
    record(f"{name}/step/auto/all_rows", err)
    assert err <= ATOL, (name, "step", err)
    forced = {"c5a": 1024, "c5b": 2048}[name]
    outs = {}
    for kernel in kernels_for(w):
        for partition in (0, -1, forced):
            got = run_attention(d, kernel, partition)
            outs[(kernel, partition)] = got
            o = got.cpu().double().numpy()
            assert np.isfinite(o).all()
            err = np.abs(o - ref).max()
            record(f"{name}/{kernel}/p{partition}/all_rows", err)
            assert err <= ATOL, (name, kernel, partition, err)
        got = run_step(d, kernel, 0)  # the rows it writes hold those bits already
        o = got.cpu().double().numpy()
        err = np.abs(o - ref).max()
        record(f"{name}/step/{kernel}/all_rows", err)
        assert err <= ATOL, (name, "step", kernel, err)
    base = outs[(kernels_for(w)[0], -1)]
    for key, o in outs.items():
        diff = (o - base).abs().max().item()
        record(f"{name}/{key[0]}/p{key[1]}/vs_unsplit", diff)
        assert diff <= 1e-4


EDGE_LENGTHS = [1, 15, 16, 17, 256, 257, 4095, 4096, 0, 33]


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 24, 8), (128, 8, 8), (64, 16, 2),
                                      (128, 32, 2), (64, 48, 8), (128, 16, 8), (128, 16, 1),
                                      (64, 4, 1)])
def test_attention_edge_lengths(dev, D, Hq, Hkv):
    """Lengths at block and pair boundaries, an empty context and a long one, for group sizes
    1 to 16 (16 fills the matrix-core tile) and a single KV head: the separate write + attention against the
    oracle, and the fused decode step and the fused RoPE step bit-identical to their separate
    calls (the new row lands at every position of a pair)."""
    w = wl.Workload("edge", batch=len(EDGE_LENGTHS), num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, block_size=16, num_blocks=1200, max_blocks=260, seed=4242,
                    q_std=3.0)
    inp = wl.make_inputs(w, poison=True, lengths=EDGE_LENGTHS)
    host = wl.to_host_numpy(inp)
    ref, _, _ = oracle.decode_step(host)
    pos = (inp["context_lens"].clamp(min=1) - 1).to(dev, torch.int32)
    inv = torch.from_numpy(llama_inv_freq(D)).to(dev)
    for kernel in kernels_for(w):
        for partition in (0, -1, 16, 256, 272):
            d = to_dev(inp, dev)
            run_write(d)
            out_t = run_attention(d, kernel, partition)
            out = out_t.cpu().double().numpy()
            err = np.abs(out - ref).max()
            record(f"edge/D{D}/G{Hq // Hkv}/{kernel}/p{partition}", err)
            assert np.isfinite(out).all()
            assert err <= ATOL, (kernel, partition, err)
            assert not out[EDGE_LENGTHS.index(0)].any()  # empty context -> zeros
            fused = to_dev(inp, dev)
            step_out = run_step(fused, kernel, partition)
            assert torch.equal(step_out, out_t), ("step", kernel, partition)
            for pool in ("k_cache", "v_cache"):
                assert torch.equal(fused[pool].view(torch.int16), d[pool].view(torch.int16))
            fr, sr = to_dev(inp, dev), to_dev(inp, dev)
            q_f, o_f = run_step_rope(fr, pos, inv, False, kernel, partition)
            q_s, o_s = run_rope_separate(sr, pos, inv, False, kernel, partition)
            assert torch.equal(q_f.view(torch.int16), q_s.view(torch.int16)), ("rope", kernel)
            assert torch.equal(o_f, o_s), ("rope", kernel, partition)
            for pool in ("k_cache", "v_cache"):
                assert torch.equal(fr[pool].view(torch.int16), sr[pool].view(torch.int16))


@pytest.mark.parametrize("block_size", [32, 64])
@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 24, 8)])
def test_larger_blocks_edge_lengths(dev, D, Hq, Hkv, block_size):
    """Lengths at 16-token, pair and large-block boundaries with 32- and 64-token blocks, on a
    poisoned pool: the write + attention against the oracle for every kernel family and
    split, an empty context gives zeros, a one-token context gives its value row exactly, and
    the fused step equals the separate calls."""
    lengths = EDGE_LENGTHS + [31, 32, 63, 64, 65, 127, 129]
    w = wl.Workload("edge_big", batch=len(lengths), num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, block_size=block_size, num_blocks=1200 * 16 // block_size,
                    max_blocks=4096 // block_size + 4, seed=4343, q_std=3.0)
    inp = wl.make_inputs(w, poison=True, lengths=lengths)
    ref, _, _ = oracle.decode_step(wl.to_host_numpy(inp))
    G = Hq // Hkv
    for kernel in kernels_for(w):
        for partition in (0, -1, block_size, 4 * block_size):
            d = to_dev(inp, dev)
            run_write(d)
            out_t = run_attention(d, kernel, partition)
            out = out_t.cpu().double().numpy()
            err = np.abs(out - ref).max()
            record(f"edge_bs{block_size}/D{D}/G{G}/{kernel}/p{partition}", err)
            assert np.isfinite(out).all()
            assert err <= ATOL, (kernel, partition, err)
            assert not out[lengths.index(0)].any()
            one = lengths.index(1)
            vrow = d["v_new"][one].float().repeat_interleave(G, dim=0)
            assert torch.equal(out_t[one], vrow), (kernel, partition)
            fused = to_dev(inp, dev)
            assert torch.equal(run_step(fused, kernel, partition), out_t), (kernel, partition)
            for pool in ("k_cache", "v_cache"):
                assert torch.equal(fused[pool].view(torch.int16), d[pool].view(torch.int16))


def test_batch_larger_than_the_pool_slots(dev):
    """96 sequences that all read the same two 16-token blocks (a shared prefix): the batch is
    three times the pool's 32 slots. Every kernel family and split must stay inside the pools
    (the attention-only launch loads no row indexed by the sequence number) and match the
    oracle."""
    B, Hq, Hkv, D, NB = 96, 8, 2, 128, 2
    g = torch.Generator().manual_seed(2024)
    bf = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    q, kc, vc = bf(B, Hq, D), bf(NB, 16, Hkv, D), bf(NB, 16, Hkv, D)
    tables = torch.tensor([[1, 0]] * B, dtype=torch.int32)
    lens = torch.randint(1, 33, (B,), generator=g, dtype=torch.int32)
    scale = D ** -0.5
    ref = oracle.decode_attention(wl.to_bits(q), wl.to_bits(kc), wl.to_bits(vc), tables.numpy(),
                                  lens.numpy(), scale)
    w = wl.Workload("shared", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=16, num_blocks=NB, max_blocks=2, seed=0, max_context_len=32)
    d = {"workload": w, "q": q.to(dev), "k_cache": kc.to(dev), "v_cache": vc.to(dev),
         "block_tables": tables.to(dev), "context_lens": lens.to(dev), "scale": scale}
    for kernel in kernels_for(w):
        for partition in (0, -1, 16):
            out = run_attention(d, kernel, partition)
            torch.cuda.synchronize()
            err = np.abs(out.cpu().double().numpy() - ref).max()
            record(f"shared_blocks/{kernel}/p{partition}", err)
            assert err <= ATOL, (kernel, partition, err)


def test_length_one_returns_value_row_exactly(dev):
    w = wl.Workload("one", batch=5, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                    num_blocks=10, max_blocks=2, seed=99, context_len=1, q_std=3.0)
    for kernel in kernels_for(w):
        for partition in (0, -1, 16):
            d = to_dev(wl.make_inputs(w, poison=True), dev)
            run_write(d)
            out = run_attention(d, kernel, partition)
            vrow = d["v_new"].float().repeat_interleave(4, dim=1)  # [B, Hq, D]
            assert torch.equal(out, vrow), (kernel, partition)


# ------------------------------------------------------- fused decode step (write + attend)
def run_step(d, kernel="auto", partition=0):
    w = d["workload"]
    out = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32,
                     device=d["q"].device)
    pk.paged_decode_step(d["q"], d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"],
                         d["v_cache"], d["block_tables"], d["context_lens"], d["scale"], out,
                         partition_tokens=part_for(kernel, partition), kernel=kernel)
    return out


@pytest.mark.parametrize("name", SMALL)
def test_decode_step_fused_matches_oracle_and_separate_calls(dev, name):
    """One call stores the new rows and attends with them: the pools equal the oracle's bit for
    bit, the output is within the bound, and it is bit-identical to the separate write and
    attention calls, for every kernel family and split."""
    host, ref, kc_ref, vc_ref, _ = case(name, dev, poison=True)
    w = wl.WORKLOADS[name]
    d = to_dev(wl.make_inputs(w, poison=True), dev)  # pools before the write
    first = True
    for kernel in ["auto"] + kernels_for(w):
        for partition in (-1, 0, 256):
            out = run_step(d, kernel, partition)
            torch.cuda.synchronize()
            if first:
                assert np.array_equal(wl.to_bits(d["k_cache"]), kc_ref)
                assert np.array_equal(wl.to_bits(d["v_cache"]), vc_ref)
                first = False
            err = np.abs(out.cpu().double().numpy() - ref).max()
            record(f"{name}/step/{kernel}/p{partition}", err)
            assert np.isfinite(err) and err <= ATOL, (kernel, partition, err)
            assert torch.equal(out, run_attention(d, kernel, partition)), (kernel, partition)


@pytest.mark.parametrize("block_size", [32, 64])
@pytest.mark.parametrize("name", ["c2", "c4"])
def test_larger_blocks_match_oracle(dev, name, block_size):
    """Blocks of 32 and 64 tokens (read as 16-token blocks through a table the call writes
    into its workspace): on a poisoned pool, the fused step's pools equal the oracle's bit for
    bit, the output is within the bound for every kernel family and split, and equals the
    separate attention call on the written pools."""
    import dataclasses
    k = block_size // 16
    base = wl.WORKLOADS[name]
    w = dataclasses.replace(base, name=f"{name}_bs{block_size}", block_size=block_size,
                            max_blocks=base.max_blocks // k, num_blocks=base.num_blocks // k)
    inp = wl.make_inputs(w, poison=True)
    ref, kc_ref, vc_ref = oracle.decode_step(wl.to_host_numpy(inp))
    d = to_dev(inp, dev)
    first = True
    for kernel in ["auto"] + kernels_for(w):
        for partition in (-1, 0, 4 * block_size):
            out = run_step(d, kernel, partition)
            torch.cuda.synchronize()
            if first:
                assert np.array_equal(wl.to_bits(d["k_cache"]), kc_ref)
                assert np.array_equal(wl.to_bits(d["v_cache"]), vc_ref)
                first = False
            err = np.abs(out.cpu().double().numpy() - ref).max()
            record(f"{w.name}/step/{kernel}/p{partition}", err)
            assert np.isfinite(err) and err <= ATOL, (kernel, partition, err)
            assert torch.equal(out, run_attention(d, kernel, partition)), (kernel, partition)


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_prepared_step_matches_the_plain_call(dev, name):
    """A prepared decode step re-reads its bound tensors at every call: after new q / k_new /
    v_new values and lengths are written into them in place, its output and pools equal those
    of paged_decode_step on identical copies, bit for bit, call after call."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, poison=True)
    a = to_dev(inp, dev)
    b = to_dev(inp, dev)
    out_a = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), device=dev)
    step = pk.prepare_decode_step(a["q"], a["k_new"], a["v_new"], a["slot_mapping"],
                                  a["k_cache"], a["v_cache"], a["block_tables"],
                                  a["context_lens"], a["scale"], out_a)
    gen = torch.Generator(device="cpu").manual_seed(7)
    for it in range(3):
        if it:
            for key in ("q", "k_new", "v_new"):
                new = torch.randn(a[key].shape, generator=gen).to(a[key].dtype).to(dev)
                a[key].copy_(new)
                b[key].copy_(new)
            lens = torch.clamp(a["context_lens"] - it, min=1)
            a["context_lens"].copy_(lens)
            b["context_lens"].copy_(lens)
        got = step()
        want = run_step(b)
        torch.cuda.synchronize()
        assert got.data_ptr() == out_a.data_ptr()
        assert torch.equal(got, want), it
        assert torch.equal(a["k_cache"].view(torch.int16), b["k_cache"].view(torch.int16)), it
        assert torch.equal(a["v_cache"].view(torch.int16), b["v_cache"].view(torch.int16)), it


def test_decode_step_negative_slots_and_full_size(dev):
    """Sequences whose slot is -1 store nothing and read their last position from the cache;
    c5b at full size matches the separate calls bit for bit."""
    w = wl.WORKLOADS["c3"]
    inp = wl.make_inputs(w, poison=True)
    inp["slot_mapping"][[0, 5, 11]] = -1
    host = wl.to_host_numpy(inp)
    ref, kc_ref, vc_ref = oracle.decode_step(host)
    d = to_dev(inp, dev)
    for kernel in ["auto"] + kernels_for(w):
        out = run_step(d, kernel, 0)
        torch.cuda.synchronize()
        assert np.array_equal(wl.to_bits(d["k_cache"]), kc_ref)
        assert np.array_equal(wl.to_bits(d["v_cache"]), vc_ref)
        assert np.abs(out.cpu().double().numpy() - ref).max() <= ATOL, kernel
    w = wl.WORKLOADS["c5b"]
    a = wl.make_inputs(w, device="cuda")
    b = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in a.items()}
    fused = run_step(a)
    run_write(b)
    sep = run_attention(b)
    torch.cuda.synchronize()
    assert torch.equal(fused, sep)
    assert torch.equal(a["k_cache"], b["k_cache"]) and torch.equal(a["v_cache"], b["v_cache"])


def test_split_agrees_with_unsplit_and_is_deterministic(dev):
    w = wl.WORKLOADS["c4"]
    d = case("c4", dev)[4]
    for kernel in kernels_for(w):
        base = run_attention(d, kernel, -1)
        again = run_attention(d, kernel, -1)
        assert torch.equal(base, again)
        for partition in (16, 64, 512, 0):
            o = run_attention(d, kernel, partition)
            diff = (o - base).abs().max().item()
            record(f"c4/{kernel}/p{partition}/vs_unsplit", diff)
            assert diff <= 1e-5, (kernel, partition, diff)


def test_kernels_agree(dev):
    w = wl.WORKLOADS["c2"]
    ks = kernels_for(w)
    if len(ks) < 2:
        pytest.skip("one kernel family built for this shape")
    d = case("c2", dev)[4]
    outs = [run_attention(d, k, 0) for k in ks]
    diff = (outs[0] - outs[1]).abs().max().item()
    record("c2/kernels_agree", diff)
    assert diff <= 1e-4


def test_empty_batch_is_noop(dev):
    w = wl.WORKLOADS["c1"]
    d = case("c1", dev)[4]
    out = torch.empty(0, w.num_q_heads, w.head_dim, device=dev)
    pk.paged_decode_attention(d["q"][:0], d["k_cache"], d["v_cache"], d["block_tables"][:0],
                              d["context_lens"][:0], d["scale"], out)
    torch.cuda.synchronize()


def test_one_workspace_across_shapes(dev):
    """One workspace reused by split calls of different batch sizes and partition counts
    (its contents are scratch: nothing carries over from call to call)."""
    w4, w5 = wl.WORKLOADS["c4"], wl.WORKLOADS["c5b"]
    _, ref4, _, _, d4 = case("c4", dev)
    need = max(pk.decode_workspace_bytes(w.batch, w.num_q_heads, w.head_dim, w.max_blocks,
                                         w.block_size, 16) for w in (w4, w5))
    ws = pk.new_workspace(need, dev)
    ws.fill_(0x7F)  # garbage
    d5 = wl.make_inputs(w5, device="cuda")
    run_write(d5)
    for kernel in kernels_for(w5):
        base5 = run_attention(d5, kernel, -1)
        for partition in (16, 256, 0, 48, 1024):
            for d, ref in ((d4, ref4), (d5, None)):
                w = d["workload"]
                out = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), device=dev)
                pk.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                          d["context_lens"], d["scale"], out,
                                          partition_tokens=part_for(kernel, partition),
                                          kernel=kernel, workspace=ws)
                if ref is not None:
                    err = np.abs(out.cpu().double().numpy() - ref).max()
                    assert err <= ATOL, (kernel, partition, err)
                else:
                    diff = (out - base5).abs().max().item()
                    record(f"c5b/{kernel}/p{partition}/vs_unsplit", diff)
                    assert diff <= 1e-4, (kernel, partition, diff)


@pytest.mark.parametrize("mode", ["separate", "fused", "rope"])
@pytest.mark.parametrize("name,partition", [("c2", 0), ("c4", 64)])
def test_graph_capture_replays_match_eager(dev, name, partition, mode):
    """The decode step captured in a HIP graph (no allocation, no memset inside the library
    calls) replays to the eager result, replay after replay, with eager work and
    synchronisations in between: as a write call then an attention call, as the fused step,
    and as the fused step with rotary embedding."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    d = to_dev(inp, dev)
    out = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    q_out = torch.empty_like(d["q"])
    pos = (d["context_lens"] - 1).to(torch.int32)
    inv = torch.from_numpy(llama_inv_freq(w.head_dim)).to(dev)
    ws = pk.new_workspace(pk.decode_workspace_bytes(w.batch, w.num_q_heads, w.head_dim,
                                                    w.max_blocks, w.block_size, partition), dev)

    def step():
        if mode == "separate":
            pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"],
                              d["v_cache"])
            pk.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                      d["context_lens"], d["scale"], out,
                                      partition_tokens=partition, workspace=ws)
        elif mode == "fused":
            pk.paged_decode_step(d["q"], d["k_new"], d["v_new"], d["slot_mapping"],
                                 d["k_cache"], d["v_cache"], d["block_tables"],
                                 d["context_lens"], d["scale"], out,
                                 partition_tokens=partition, workspace=ws)
        else:
            pk.paged_decode_step_rope(d["q"], d["k_new"], d["v_new"], pos, inv,
                                      d["slot_mapping"], q_out, d["k_cache"], d["v_cache"],
                                      d["block_tables"], d["context_lens"], d["scale"], out,
                                      partition_tokens=partition, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager, eager_q = out.clone(), q_out.clone()
    eager_kc, eager_vc = wl.to_bits(d["k_cache"]), wl.to_bits(d["v_cache"])
    if mode != "rope":
        _, ref, kc_ref, vc_ref, _ = case(name, dev)
        assert np.abs(eager.cpu().double().numpy() - ref).max() <= ATOL
        assert np.array_equal(eager_kc, kc_ref) and np.array_equal(eager_vc, vc_ref)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        q_out.fill_(float("nan"))
        d["k_cache"].view(torch.int16)[0, 0, 0, 0] += 0  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        if mode == "rope":
            assert torch.equal(q_out.view(torch.int16), eager_q.view(torch.int16)), f"replay {r}"
    assert np.array_equal(wl.to_bits(d["k_cache"]), eager_kc)
    assert np.array_equal(wl.to_bits(d["v_cache"]), eager_vc)


@pytest.mark.parametrize("name", ["c1", "c2", "c4"])
def test_hip_stream_capture_of_several_steps(dev, name):
    """Eight fused decode steps (as a model captures every layer's step) recorded with the HIP
    runtime's own stream capture, no torch graph wrapper, into one graph; three replays, with
    eager work and synchronisations in between, each leave the output and the pools bit-identical
    to the eager step (the steps are idempotent: each stores the same new rows)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    vp = ctypes.c_void_p
    hip.hipStreamBeginCapture.argtypes = [vp, ctypes.c_int]
    hip.hipStreamEndCapture.argtypes = [vp, ctypes.POINTER(vp)]
    hip.hipGraphInstantiate.argtypes = [ctypes.POINTER(vp), vp, vp, vp, ctypes.c_size_t]
    hip.hipGraphLaunch.argtypes = [vp, vp]
    hip.hipGraphExecDestroy.argtypes = [vp]
    hip.hipGraphDestroy.argtypes = [vp]
    w = wl.WORKLOADS[name]
    d = to_dev(wl.make_inputs(w, poison=True), dev)
    out = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    ws = pk.new_workspace(pk.decode_workspace_bytes(w.batch, w.num_q_heads, w.head_dim,
                                                    w.max_blocks, w.block_size, 0), dev)

    def step():
        pk.paged_decode_step(d["q"], d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"],
                             d["v_cache"], d["block_tables"], d["context_lens"], d["scale"], out,
                             workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    eager_kc, eager_vc = wl.to_bits(d["k_cache"]), wl.to_bits(d["v_cache"])
    _, ref, kc_ref, vc_ref, _ = case(name, dev, poison=True)
    assert np.abs(eager.cpu().double().numpy() - ref).max() <= ATOL
    assert np.array_equal(eager_kc, kc_ref) and np.array_equal(eager_vc, vc_ref)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    graph, exe = vp(), vp()
    with torch.cuda.stream(side):
        assert hip.hipStreamBeginCapture(side.cuda_stream, 2) == 0  # relaxed mode
        for _ in range(8):
            step()
        assert hip.hipStreamEndCapture(side.cuda_stream, ctypes.byref(graph)) == 0
    assert hip.hipGraphInstantiate(ctypes.byref(exe), graph, None, None, 0) == 0
    try:
        for r in range(3):
            out.fill_(float("nan"))
            d["k_cache"].view(torch.int16)[0, 0, 0, 0] += 0  # eager work between replays
            torch.cuda.synchronize()
            assert hip.hipGraphLaunch(exe, side.cuda_stream) == 0
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {r}"
        assert np.array_equal(wl.to_bits(d["k_cache"]), eager_kc)
        assert np.array_equal(wl.to_bits(d["v_cache"]), eager_vc)
    finally:
        hip.hipGraphExecDestroy(exe)
        hip.hipGraphDestroy(graph)


# ------------------------------------------------------- multi-query causal (prefill)
_PCASES = {}


def prefill_case(name, dev, poison=False, rows=None):
    key = (name, poison)
    if key not in _PCASES:
        w = wl.PREFILL_WORKLOADS[name]
        inp = wl.make_prefill_inputs(w, poison=poison)
        host = wl.to_host_numpy(inp)
        kc, vc = oracle.kv_write(host["k_new"], host["v_new"], host["slot_mapping"],
                                 host["k_cache"], host["v_cache"])
        ref = oracle.prefill_attention(host["q"], host["cu_seqlens_q"], kc, vc,
                                       host["block_tables"], host["context_lens"],
                                       host["scale"], rows=rows)
        d = to_dev(inp, dev)
        run_write(d)
        torch.cuda.synchronize()
        assert np.array_equal(wl.to_bits(d["k_cache"]), kc)
        _PCASES[key] = (ref, d)
    return _PCASES[key]


def run_prefill(d, row_blocks=0, partition=0, workspace=None):
    T, Hq, D = d["q"].shape
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device=d["q"].device)
    pk.paged_prefill_attention(d["q"], d["cu_seqlens_q"], d["k_cache"], d["v_cache"],
                               d["block_tables"], d["context_lens"], d["scale"], out,
                               max_q_len=d["max_q_len"], row_blocks=row_blocks,
                               partition_tokens=partition, workspace=workspace)
    return out


@pytest.mark.parametrize("row_blocks", [0, 1, 2, 4])
@pytest.mark.parametrize("name", ["p2", "p3"])
def test_prefill_parity(dev, name, row_blocks):
    ref, d = prefill_case(name, dev)
    out = run_prefill(d, row_blocks).cpu().double().numpy()
    err = np.abs(out - ref).max()
    record(f"{name}/prefill/rb{row_blocks}", err)
    assert np.isfinite(out).all()
    assert err <= ATOL, err


@pytest.mark.parametrize("row_blocks,partition", [(1, 0), (2, 0), (4, 0), (1, 32), (2, 512)])
def test_prefill_first_position_returns_value_row_exactly(dev, row_blocks, partition):
    """In a full prefill the row at position 0 sees only key 0, so its output is that value row
    exactly (one weight of exactly 1), for every query head of the group; with the keys split,
    the merge of that one partial with empty partitions keeps it exact."""
    _, d = prefill_case("p3", dev)
    w = wl.PREFILL_WORKLOADS["p3"]
    out = run_prefill(d, row_blocks, partition)
    G = w.num_q_heads // w.num_kv_heads
    cu = d["cu_seqlens_q"].tolist()
    for b in range(w.batch):
        blk0 = int(d["block_tables"][b, 0])
        v0 = d["v_cache"][blk0, 0].float().repeat_interleave(G, dim=0)  # [Hq, D]
        assert torch.equal(out[cu[b]], v0), (b, row_blocks)


@pytest.mark.parametrize("partition", [0, -1, 32, 96, 512, 1024])
@pytest.mark.parametrize("row_blocks", [1, 2])
@pytest.mark.parametrize("name", ["p2", "p3"])
def test_prefill_key_split_parity(dev, name, row_blocks, partition):
    """Key partitions of 32 keys (one staged pair) up to 1024, the automatic choice and no
    split: every output against the oracle, and the split within fp32 rounding of the unsplit
    call."""
    ref, d = prefill_case(name, dev)
    out = run_prefill(d, row_blocks, partition)
    base = run_prefill(d, row_blocks, -1)
    plan = pk.prefill_plan(d["q"].shape[0], d["max_q_len"], d["context_lens"].shape[0],
                           d["q"].shape[1], d["k_cache"].shape[2], d["q"].shape[2],
                           d["block_tables"].shape[1], d["k_cache"].shape[1], row_blocks,
                           partition)
    err = np.abs(out.cpu().double().numpy() - ref).max()
    record(f"{name}/prefill_split/rb{row_blocks}/p{partition}/n{plan[1]}", err)
    assert torch.isfinite(out).all()
    assert err <= ATOL, err
    assert (out - base).abs().max().item() <= 1e-5
    if partition == -1:
        assert plan[1] == 1
    if partition == 32:
        assert plan[1] > 1


@pytest.mark.parametrize("block_size", [32, 64])
@pytest.mark.parametrize("name", ["p2", "p3"])
def test_prefill_larger_blocks(dev, name, block_size):
    """Multi-query attention over pools of 32- and 64-token blocks (read as 16-token blocks),
    on poisoned pools: every output against the oracle for one and two row blocks per wave,
    unsplit, automatic and with the keys split."""
    import dataclasses
    k = block_size // 16
    base = wl.PREFILL_WORKLOADS[name]
    w = dataclasses.replace(base, name=f"{name}_bs{block_size}", block_size=block_size,
                            num_blocks=base.num_blocks // k + 8,
                            max_blocks=-(-base.max_blocks // k))
    inp = wl.make_prefill_inputs(w, poison=True)
    host = wl.to_host_numpy(inp)
    kc, vc = oracle.kv_write(host["k_new"], host["v_new"], host["slot_mapping"],
                             host["k_cache"], host["v_cache"])
    ref = oracle.prefill_attention(host["q"], host["cu_seqlens_q"], kc, vc,
                                   host["block_tables"], host["context_lens"], host["scale"])
    d = to_dev(inp, dev)
    run_write(d)
    torch.cuda.synchronize()
    assert np.array_equal(wl.to_bits(d["k_cache"]), kc)
    for row_blocks in (1, 2):
        for partition in (-1, 0, 256):
            out = run_prefill(d, row_blocks, partition).cpu().double().numpy()
            err = np.abs(out - ref).max()
            record(f"{w.name}/prefill/rb{row_blocks}/p{partition}", err)
            assert np.isfinite(out).all()
            assert err <= ATOL, (row_blocks, partition, err)


def test_prefill_key_split_ignores_workspace_contents(dev):
    """Every (row, partition) slot the merge reads is written by the call: a workspace full of
    NaN gives the same result as a fresh one, twice in a row."""
    _, d = prefill_case("p2", dev)
    T, Hq, D = d["q"].shape
    need = pk.prefill_workspace_bytes(T, Hq, D, d["block_tables"].shape[1], d["k_cache"].shape[1],
                                      64)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev).view(torch.uint8)
    first = run_prefill(d, 1, 64, workspace=ws)
    second = run_prefill(d, 1, 64, workspace=ws)
    fresh = run_prefill(d, 1, 64, workspace=torch.zeros(need, dtype=torch.uint8, device=dev))
    assert torch.equal(first, fresh) and torch.equal(second, fresh)


def test_prefill_key_split_rejects_a_small_workspace(dev):
    _, d = prefill_case("p2", dev)
    T, Hq, D = d["q"].shape
    need = pk.prefill_workspace_bytes(T, Hq, D, d["block_tables"].shape[1], d["k_cache"].shape[1],
                                      512)
    with pytest.raises(pk.PagedKVError):
        run_prefill(d, 1, 512, workspace=torch.empty(need - 256, dtype=torch.uint8, device=dev))


def test_prefill_chunked_every_row(dev):
    """p1 (8 chunks of 512 queries on 3584 cached tokens): every output row against the
    oracle, unsplit and with 1024-key partitions."""
    ref, d = prefill_case("p1", dev)
    for partition in (0, 1024):
        out = run_prefill(d, 0, partition).cpu().double().numpy()
        assert np.isfinite(out).all()
        err = np.abs(out - ref).max()
        record(f"p1/prefill/all_rows/p{partition}", err)
        assert err <= ATOL, err


def test_prefill_poisoned_pool_matches_clean(dev):
    _, clean = prefill_case("p2", dev)
    ref, dirty = prefill_case("p2", dev, poison=True)
    o1, o2 = run_prefill(clean), run_prefill(dirty)
    assert torch.equal(o1, o2)
    assert np.abs(o2.cpu().double().numpy() - ref).max() <= ATOL


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_prefill_single_query_matches_decode(dev, name):
    """One query row per sequence at its last position is the decode case."""
    w = wl.WORKLOADS[name]
    _, ref, _, _, d = case(name, dev)
    cu = torch.arange(w.batch + 1, dtype=torch.int32, device=dev)
    out = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    pk.paged_prefill_attention(d["q"], cu, d["k_cache"], d["v_cache"], d["block_tables"],
                               d["context_lens"], d["scale"], out, max_q_len=1)
    dec = run_attention(d, "auto", -1)
    diff = (out - dec).abs().max().item()
    record(f"{name}/prefill_q1_vs_decode", diff)
    assert diff <= 1e-4
    assert np.abs(out.cpu().double().numpy() - ref).max() <= ATOL


@pytest.mark.parametrize("row_blocks,partition", [(1, 0), (4, 0), (1, 32), (4, 64)])
@pytest.mark.parametrize("Hq,Hkv,D", [(24, 8, 64), (16, 16, 128), (32, 2, 128)])
def test_prefill_group_sizes_and_edges(dev, Hq, Hkv, D, row_blocks, partition):
    """G = 3, 1 and 16 (5, 16 and 1 query tokens per wave), lengths at block edges, single
    tokens, full prefills and chunks, on a poisoned pool; unsplit and with the keys split into
    partitions of 32 or 64 (rows before a partition, partitions past a tile's keys)."""
    w = wl.PrefillWorkload("edge", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=16,
                           num_blocks=200, max_blocks=80, seed=77,
                           context_lens=(1, 16, 17, 33, 300, 1000),
                           query_lens=(1, 16, 5, 33, 47, 129), q_std=3.0)
    inp = wl.make_prefill_inputs(w, poison=True)
    host = wl.to_host_numpy(inp)
    kc, vc = oracle.kv_write(host["k_new"], host["v_new"], host["slot_mapping"],
                             host["k_cache"], host["v_cache"])
    ref = oracle.prefill_attention(host["q"], host["cu_seqlens_q"], kc, vc, host["block_tables"],
                                   host["context_lens"], host["scale"])
    d = to_dev(inp, dev)
    run_write(d)
    out = run_prefill(d, row_blocks, partition).cpu().double().numpy()
    err = np.abs(out - ref).max()
    record(f"edge_prefill/D{D}/G{Hq // Hkv}/rb{row_blocks}/p{partition}", err)
    assert np.isfinite(out).all() and err <= ATOL, err


# ---------------------------------------------------------- RoPE fused with the KV write
def llama_inv_freq(D, base=500000.0):
    return (base ** (-np.arange(D // 2, dtype=np.float64) * 2 / D)).astype(np.float32)


def bf16_ulp_diff(a_bits, b_bits):
    """|a - b| in units of the larger operand's bf16 spacing (NaN-free inputs)."""
    a = oracle.bf16_bits_to_f64(a_bits)
    b = oracle.bf16_bits_to_f64(b_bits)
    mag = np.maximum(np.abs(a), np.abs(b))
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    ulp = np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))
    return np.abs(a - b) / ulp


@pytest.mark.parametrize("name,interleaved", [("c2", False), ("c4", True), ("c5b", False)])
def test_rope_write_matches_oracle(dev, name, interleaved):
    """Rotated q and the pools after the fused write agree with the oracle's float64 rotation
    rounded to bf16 to within one bf16 unit in the last place (the kernel rounds its fp32
    result, the oracle its float64 result), and almost everywhere exactly."""
    w = wl.WORKLOADS[name]
    if name == "c5b":
        inp = wl.make_inputs(w, device="cuda")
        d = inp
    else:
        inp = wl.make_inputs(w)
        d = to_dev(inp, dev)
    kc0, vc0 = wl.to_bits(d["k_cache"]), wl.to_bits(d["v_cache"])
    pos = (d["context_lens"] - 1).to(torch.int32)
    inv = torch.from_numpy(llama_inv_freq(w.head_dim)).to(dev)
    q_rot = pk.paged_kv_write_rope(d["q"], d["k_new"], d["v_new"], pos, inv, d["slot_mapping"],
                                   d["k_cache"], d["v_cache"], interleaved=interleaved)
    torch.cuda.synchronize()
    q_ref, kc_ref, vc_ref = oracle.kv_write_rope(
        wl.to_bits(d["q"]), wl.to_bits(d["k_new"]), wl.to_bits(d["v_new"]), pos.cpu().numpy(),
        inv.cpu().numpy(), interleaved, d["slot_mapping"].cpu().numpy(), kc0, vc0)
    assert np.array_equal(wl.to_bits(d["v_cache"]), vc_ref)  # v is copied bit for bit
    for got, ref, what in ((wl.to_bits(q_rot), q_ref, "q"), (wl.to_bits(d["k_cache"]), kc_ref, "k")):
        diff = bf16_ulp_diff(got, ref)
        frac = float((got != ref).mean())
        record(f"rope/{name}/{what}/max_ulp", float(diff.max()))
        assert diff.max() <= 1.0, (what, diff.max())
        assert frac <= 0.01, (what, frac)


def test_decode_step_with_rope(dev):
    """Rotate + write the new token at position L-1, then attend with the rotated q."""
    w = wl.WORKLOADS["c4"]
    inp = wl.make_inputs(w)
    host = wl.to_host_numpy(inp)
    d = to_dev(inp, dev)
    pos = (d["context_lens"] - 1).to(torch.int32)
    inv_np = llama_inv_freq(w.head_dim)
    q_rot = pk.paged_kv_write_rope(d["q"], d["k_new"], d["v_new"], pos,
                                   torch.from_numpy(inv_np).to(dev), d["slot_mapping"],
                                   d["k_cache"], d["v_cache"])
    d2 = dict(d)
    d2["q"] = q_rot
    out = run_attention(d2).cpu().double().numpy()
    q_ref, kc, vc = oracle.kv_write_rope(host["q"], host["k_new"], host["v_new"],
                                         pos.cpu().numpy(), inv_np, False, host["slot_mapping"],
                                         host["k_cache"], host["v_cache"])
    ref = oracle.decode_attention(q_ref, kc, vc, host["block_tables"], host["context_lens"],
                                  host["scale"])
    err = np.abs(out - ref).max()
    record("c4/rope_decode_step", err)
    assert err <= ATOL, err


def test_rope_in_place_and_large_positions(dev):
    w = wl.Workload("rope", batch=8, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                    num_blocks=64, max_blocks=8, seed=5, context_len=100)
    inp = wl.make_inputs(w)
    d = to_dev(inp, dev)
    pos = torch.tensor([0, 1, 2, 1000, 8191, 32767, 131071, 65535], dtype=torch.int32, device=dev)
    inv = torch.from_numpy(llama_inv_freq(64, 10000.0)).to(dev)
    q_in = d["q"].clone()
    kc0, vc0 = wl.to_bits(d["k_cache"]), wl.to_bits(d["v_cache"])
    q_out = pk.paged_kv_write_rope(d["q"], d["k_new"], d["v_new"], pos, inv, d["slot_mapping"],
                                   d["k_cache"], d["v_cache"], q_out=d["q"])  # in place
    torch.cuda.synchronize()
    q_ref, kc_ref, _ = oracle.kv_write_rope(wl.to_bits(q_in), wl.to_bits(d["k_new"]),
                                            wl.to_bits(d["v_new"]), pos.cpu().numpy(),
                                            inv.cpu().numpy(), False,
                                            d["slot_mapping"].cpu().numpy(), kc0, vc0)
    assert q_out.data_ptr() == d["q"].data_ptr()
    assert bf16_ulp_diff(wl.to_bits(q_out), q_ref).max() <= 1.0
    assert bf16_ulp_diff(wl.to_bits(d["k_cache"]), kc_ref).max() <= 1.0


# ------------------------------------------------------- decode step with rotary embedding
def run_step_rope(d, pos, inv, interleaved, kernel="auto", partition=0):
    """paged_decode_step_rope into NaN-poisoned q_out and out."""
    w = d["workload"]
    out = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32,
                     device=d["q"].device)
    q_out = torch.full_like(d["q"], float("nan"))
    pk.paged_decode_step_rope(d["q"], d["k_new"], d["v_new"], pos, inv, d["slot_mapping"], q_out,
                              d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                              d["scale"], out, interleaved=interleaved,
                              partition_tokens=part_for(kernel, partition), kernel=kernel)
    return q_out, out


def run_rope_separate(d, pos, inv, interleaved, kernel="auto", partition=0):
    """The same step as two calls: the standalone rotation + write, then attention with the
    rotated q. Modifies d's pools."""
    q_rot = pk.paged_kv_write_rope(d["q"], d["k_new"], d["v_new"], pos, inv, d["slot_mapping"],
                                   d["k_cache"], d["v_cache"], interleaved=interleaved)
    return q_rot, run_attention(dict(d, q=q_rot), kernel, partition)


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("name", SMALL)
def test_decode_step_rope_fused_matches_separate_calls_and_oracle(dev, name, interleaved):
    """One launch rotates q and the new key at position L-1, stores the rotated key and the
    value, and attends: q_out, the pools and the output equal the two separate calls bit for
    bit (every kernel family and split), and the output is within the bound of the oracle's
    rotation + write + attention."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, poison=True)
    host = wl.to_host_numpy(inp)
    pos_np = (host["context_lens"] - 1).astype(np.int32)
    inv_np = llama_inv_freq(w.head_dim)
    q_ref, kc_ref, vc_ref = oracle.kv_write_rope(host["q"], host["k_new"], host["v_new"], pos_np,
                                                 inv_np, interleaved, host["slot_mapping"],
                                                 host["k_cache"], host["v_cache"])
    ref = oracle.decode_attention(q_ref, kc_ref, vc_ref, host["block_tables"],
                                  host["context_lens"], host["scale"])
    pos = torch.from_numpy(pos_np).to(dev)
    inv = torch.from_numpy(inv_np).to(dev)
    fused = to_dev(inp, dev)
    sep = to_dev(inp, dev)
    for kernel in ["auto"] + kernels_for(w):
        for partition in (-1, 0, 256):
            q_f, out_f = run_step_rope(fused, pos, inv, interleaved, kernel, partition)
            q_s, out_s = run_rope_separate(sep, pos, inv, interleaved, kernel, partition)
            torch.cuda.synchronize()
            key = (kernel, partition)
            assert torch.equal(q_f.view(torch.int16), q_s.view(torch.int16)), key
            assert torch.equal(fused["k_cache"].view(torch.int16),
                               sep["k_cache"].view(torch.int16)), key
            assert torch.equal(fused["v_cache"].view(torch.int16),
                               sep["v_cache"].view(torch.int16)), key
            assert torch.equal(out_f, out_s), key
            err = np.abs(out_f.cpu().double().numpy() - ref).max()
            record(f"{name}/step_rope/il{int(interleaved)}/{kernel}/p{partition}", err)
            assert np.isfinite(err) and err <= ATOL, (key, err)
    assert bf16_ulp_diff(wl.to_bits(q_f), q_ref).max() <= 1.0
    kc = wl.to_bits(fused["k_cache"])
    same = kc == kc_ref  # the poisoned (NaN) slots nobody writes compare by their bits
    zero = np.uint16(0)
    diff = bf16_ulp_diff(np.where(same, zero, kc), np.where(same, zero, kc_ref))
    assert (same | (diff <= 1.0)).all()
    assert np.array_equal(wl.to_bits(fused["v_cache"]), vc_ref)


def test_decode_step_rope_larger_blocks(dev):
    """The rotary decode step with 32-token blocks (c4 shape, ragged, poisoned pools): q_out,
    the pools and the output equal the separate rotation + write and attention calls bit for
    bit, for every kernel family and split, and the output is within the bound of the
    oracle's."""
    import dataclasses
    base = wl.WORKLOADS["c4"]
    w = dataclasses.replace(base, name="c4_bs32", block_size=32, max_blocks=base.max_blocks // 2,
                            num_blocks=base.num_blocks // 2)
    inp = wl.make_inputs(w, poison=True)
    host = wl.to_host_numpy(inp)
    pos_np = (host["context_lens"] - 1).astype(np.int32)
    inv_np = llama_inv_freq(w.head_dim)
    q_ref, kc_ref, vc_ref = oracle.kv_write_rope(host["q"], host["k_new"], host["v_new"], pos_np,
                                                 inv_np, False, host["slot_mapping"],
                                                 host["k_cache"], host["v_cache"])
    ref = oracle.decode_attention(q_ref, kc_ref, vc_ref, host["block_tables"],
                                  host["context_lens"], host["scale"])
    pos = torch.from_numpy(pos_np).to(dev)
    inv = torch.from_numpy(inv_np).to(dev)
    fused = to_dev(inp, dev)
    sep = to_dev(inp, dev)
    for kernel in ["auto"] + kernels_for(w):
        for partition in (-1, 0, 128):
            q_f, out_f = run_step_rope(fused, pos, inv, False, kernel, partition)
            q_s, out_s = run_rope_separate(sep, pos, inv, False, kernel, partition)
            torch.cuda.synchronize()
            key = (kernel, partition)
            assert torch.equal(q_f.view(torch.int16), q_s.view(torch.int16)), key
            assert torch.equal(fused["k_cache"].view(torch.int16),
                               sep["k_cache"].view(torch.int16)), key
            assert torch.equal(fused["v_cache"].view(torch.int16),
                               sep["v_cache"].view(torch.int16)), key
            assert torch.equal(out_f, out_s), key
            err = np.abs(out_f.cpu().double().numpy() - ref).max()
            record(f"c4_bs32/step_rope/{kernel}/p{partition}", err)
            assert np.isfinite(err) and err <= ATOL, (key, err)
    assert np.array_equal(wl.to_bits(fused["v_cache"]), vc_ref)


def test_decode_step_rope_large_positions_negative_slots_and_full_size(dev):
    """Positions far beyond the context (the sine and cosine of large angles), sequences with
    no slot (nothing stored, their last position read from the cache), and c5b at full size:
    the fused step equals the separate calls bit for bit."""
    w = wl.WORKLOADS["c3"]
    inp = wl.make_inputs(w, poison=True)
    inp["slot_mapping"][[0, 5, 11]] = -1
    pos = torch.tensor([0, 1, 2, 1000, 8191, 32767, 131071, 65535, 7, 9, 300, 4095, 12, 77,
                        500000, 3], dtype=torch.int32, device=dev)
    for interleaved in (False, True):
        inv = torch.from_numpy(llama_inv_freq(w.head_dim, 10000.0)).to(dev)
        fused, sep = to_dev(inp, dev), to_dev(inp, dev)
        for kernel in ["auto"] + kernels_for(w):
            q_f, out_f = run_step_rope(fused, pos, inv, interleaved, kernel, 0)
            q_s, out_s = run_rope_separate(sep, pos, inv, interleaved, kernel, 0)
            torch.cuda.synchronize()
            assert torch.equal(q_f.view(torch.int16), q_s.view(torch.int16)), kernel
            assert torch.equal(fused["k_cache"].view(torch.int16),
                               sep["k_cache"].view(torch.int16)), kernel
            assert torch.equal(out_f, out_s), kernel
    w = wl.WORKLOADS["c5b"]
    a = wl.make_inputs(w, device="cuda")
    b = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in a.items()}
    pos = (a["context_lens"] - 1).to(torch.int32)
    inv = torch.from_numpy(llama_inv_freq(w.head_dim)).to(dev)
    q_f, out_f = run_step_rope(a, pos, inv, False)
    q_s, out_s = run_rope_separate(b, pos, inv, False)
    torch.cuda.synchronize()
    assert torch.equal(q_f.view(torch.int16), q_s.view(torch.int16))
    assert torch.equal(out_f, out_s)
    assert torch.equal(a["k_cache"], b["k_cache"]) and torch.equal(a["v_cache"], b["v_cache"])


# ------------------------------------------------------- addressing past 4 GiB
def _move_to_big_pool(d, first_block, nb_big, dev):
    """Device copy of input dict d whose pools are [nb_big] blocks, with d's blocks placed
    from block `first_block` on (the rest uninitialised) and the tables and slots shifted to
    match."""
    big = dict(d)
    for pool in ("k_cache", "v_cache"):
        src = d[pool]
        dst = torch.empty((nb_big,) + tuple(src.shape[1:]), dtype=src.dtype, device=dev)
        dst[first_block:first_block + src.shape[0]] = src.to(dev)
        big[pool] = dst
    bt = d["block_tables"].to(dev)
    big["block_tables"] = torch.where(bt >= 0, bt + first_block, bt)
    bs = d["k_cache"].shape[1]
    sm = d["slot_mapping"].to(dev)
    big["slot_mapping"] = torch.where(sm >= 0, sm + first_block * bs, sm)
    for key in ("q", "k_new", "v_new", "context_lens", "cu_seqlens_q"):
        if key in d:
            big[key] = d[key].to(dev)
    return big


def test_pools_past_4gib_every_path(dev):
    """Block ids whose byte offsets lie past 2^32 (blocks from 140000 on, 32 KiB each, in a
    4.6 GiB pool pair): the write, every decode kernel family and split, the fused step, the
    fused RoPE step and prefill give the oracle's results, so no kernel forms a block
    address in 32 bits. The oracle runs on the compact copy of the same data."""
    first, nb_big = 140_000, 150_000
    w = wl.WORKLOADS["c2"]
    inp = wl.make_inputs(w, poison=True)
    host = wl.to_host_numpy(inp)
    ref, kc_ref, vc_ref = oracle.decode_step(host)
    nb = inp["k_cache"].shape[0]
    d = _move_to_big_pool(inp, first, nb_big, dev)
    assert (d["k_cache"].element_size() * d["k_cache"][0].numel() * first) > 2 ** 32
    run_write(d)
    torch.cuda.synchronize()
    assert np.array_equal(wl.to_bits(d["k_cache"][first:first + nb]), kc_ref)
    assert np.array_equal(wl.to_bits(d["v_cache"][first:first + nb]), vc_ref)
    for kernel in kernels_for(w):
        for partition in (-1, 0, 128):
            err = np.abs(run_attention(d, kernel, partition).cpu().double().numpy() - ref).max()
            record(f"big/{kernel}/p{partition}", err)
            assert err <= ATOL, (kernel, partition, err)
    f = _move_to_big_pool(inp, first, nb_big, dev)
    out = run_step(f, "auto", 0)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().double().numpy() - ref).max() <= ATOL
    assert np.array_equal(wl.to_bits(f["k_cache"][first:first + nb]), kc_ref)
    del f
    pos = (inp["context_lens"] - 1).to(dev, torch.int32)
    inv = torch.from_numpy(llama_inv_freq(w.head_dim)).to(dev)
    fr = _move_to_big_pool(inp, first, nb_big, dev)
    q_f, o_f = run_step_rope(fr, pos, inv, False)
    small = to_dev(inp, dev)
    q_s, o_s = run_rope_separate(small, pos, inv, False)
    torch.cuda.synchronize()
    assert torch.equal(q_f.view(torch.int16), q_s.view(torch.int16))
    assert torch.equal(o_f, o_s)
    assert torch.equal(fr["k_cache"][first:first + nb].view(torch.int16),
                       small["k_cache"].view(torch.int16))
    del fr, d
    pw = wl.PREFILL_WORKLOADS["p2"]
    pinp = wl.make_prefill_inputs(pw)
    phost = wl.to_host_numpy(pinp)
    kc, vc = oracle.kv_write(phost["k_new"], phost["v_new"], phost["slot_mapping"],
                             phost["k_cache"], phost["v_cache"])
    pref = oracle.prefill_attention(phost["q"], phost["cu_seqlens_q"], kc, vc,
                                    phost["block_tables"], phost["context_lens"], phost["scale"])
    p = _move_to_big_pool(pinp, first, nb_big, dev)
    run_write(p)
    T, Hq, D = p["q"].shape
    pout = torch.full((T, Hq, D), float("nan"), device=dev)
    pk.paged_prefill_attention(p["q"], p["cu_seqlens_q"], p["k_cache"], p["v_cache"],
                               p["block_tables"], p["context_lens"], p["scale"], pout,
                               max_q_len=p["max_q_len"])
    err = np.abs(pout.cpu().double().numpy() - pref).max()
    record("big/prefill", err)
    assert err <= ATOL, err


def test_many_short_ragged_sequences(dev):
    """1024 sequences of 1..160 tokens (a wide continuous-batching step of short contexts),
    every kernel family and split, against the oracle; the fused step matches the separate
    calls bit for bit."""
    B = 1024
    lengths = [int(x) for x in np.random.default_rng(77).integers(1, 161, size=B)]
    nblocks = sum((L + 15) // 16 for L in lengths)
    w = wl.Workload("wide", batch=B, num_q_heads=32, num_kv_heads=8, head_dim=128,
                    block_size=16, num_blocks=nblocks + 64, max_blocks=10, seed=606,
                    context_len=1)
    inp = wl.make_inputs(w, poison=True, lengths=lengths)
    host = wl.to_host_numpy(inp)
    ref, kc_ref, _ = oracle.decode_step(host)
    for kernel in kernels_for(w):
        for partition in (0, -1, 64):
            d = to_dev(inp, dev)
            run_write(d)
            out = run_attention(d, kernel, partition)
            err = np.abs(out.cpu().double().numpy() - ref).max()
            record(f"wide/{kernel}/p{partition}", err)
            assert err <= ATOL, (kernel, partition, err)
            f = to_dev(inp, dev)
            assert torch.equal(run_step(f, kernel, partition), out), (kernel, partition)
            assert np.array_equal(wl.to_bits(f["k_cache"]), kc_ref)


def test_stream_kernel_many_segments_per_slice(dev):
    """The stream kernel on 600 short sequences (0..160 tokens) with a 1280-token table, so
    that every slice crosses several sequences and closes several segments (each with its
    new-token slot read ahead and its new rows stored from registers). Some slots are
    negative. For five slice settings (both sides of the point where the slices stop being
    weighted by XCD), the plain and the rotary fused step equal their separate calls bit for
    bit, the pools equal the oracle's, and the output is within the bound."""
    B = 600
    rng = np.random.default_rng(4242)
    lengths = [int(x) for x in rng.integers(1, 161, size=B)]
    for b in (0, 17, 301, 599):
        lengths[b] = 0
    nblocks = sum((L + 15) // 16 for L in lengths)
    w = wl.Workload("sk_short", batch=B, num_q_heads=24, num_kv_heads=8, head_dim=128,
                    block_size=16, num_blocks=nblocks + 64, max_blocks=80, seed=4243,
                    context_len=1)
    inp = wl.make_inputs(w, poison=True, lengths=lengths)
    inp["slot_mapping"][[3, 50, 420]] = -1
    host = wl.to_host_numpy(inp)
    ref, kc_ref, vc_ref = oracle.decode_step(host)
    pos_np = np.maximum(host["context_lens"] - 1, 0).astype(np.int32)
    inv_np = llama_inv_freq(w.head_dim)
    q_rr, kc_rr, vc_rr = oracle.kv_write_rope(host["q"], host["k_new"], host["v_new"], pos_np,
                                              inv_np, False, host["slot_mapping"],
                                              host["k_cache"], host["v_cache"])
    ref_r = oracle.decode_attention(q_rr, kc_rr, vc_rr, host["block_tables"],
                                    host["context_lens"], host["scale"])
    pos = torch.from_numpy(pos_np).to(dev)
    inv = torch.from_numpy(inv_np).to(dev)
    # 3564 items: on the whole device (256 CUs) slices of about 14 pairs, XCD-weighted for
    # min_pairs up to 12 (384 tokens) and equal from 13 (416 tokens) on; 1024 tokens: 32 pairs.
    for partition in (0, 64, 384, 416, 1024):
        print(f"[case] sk_short p{partition}", flush=True)
        f, s_ = to_dev(inp, dev), to_dev(inp, dev)
        out_f = run_step(f, "mfma_sk", partition)
        run_write(s_)
        out_s = run_attention(s_, "mfma_sk", partition)
        torch.cuda.synchronize()
        assert torch.equal(out_f, out_s), partition
        assert np.array_equal(wl.to_bits(f["k_cache"]), kc_ref), partition
        assert np.array_equal(wl.to_bits(f["v_cache"]), vc_ref), partition
        err = np.abs(out_f.cpu().double().numpy() - ref).max()
        record(f"sk_short/step/p{partition}", err)
        assert err <= ATOL, (partition, err)
        f, s_ = to_dev(inp, dev), to_dev(inp, dev)
        q_f, out_f = run_step_rope(f, pos, inv, False, "mfma_sk", partition)
        q_s, out_s = run_rope_separate(s_, pos, inv, False, "mfma_sk", partition)
        torch.cuda.synchronize()
        assert torch.equal(q_f.view(torch.int16), q_s.view(torch.int16)), partition
        assert torch.equal(f["k_cache"].view(torch.int16), s_["k_cache"].view(torch.int16))
        assert torch.equal(f["v_cache"].view(torch.int16), s_["v_cache"].view(torch.int16))
        assert torch.equal(out_f, out_s), partition
        assert np.array_equal(wl.to_bits(f["v_cache"]), vc_rr), partition
        err = np.abs(out_f.cpu().double().numpy() - ref_r).max()
        record(f"sk_short/step_rope/p{partition}", err)
        assert np.isfinite(err) and err <= ATOL, (partition, err)


def test_concurrent_calls_on_two_streams(dev):
    """Two split decode calls of different workloads run at the same time on two streams, each
    with the workspace the binding keeps for its stream: both equal their results computed
    alone (the library holds no state a call could share with another)."""
    names = ("c3", "c4")
    alone = {}
    data = {}
    for name in names:
        d = case(name, dev)[4]
        data[name] = d
        alone[name] = run_attention(d, "auto", 256)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in names]
    outs = {}
    for rep in range(3):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream(dev))
        for name, s in zip(names, streams):
            with torch.cuda.stream(s):
                outs[name] = run_attention(data[name], "auto", 256)
        for s in streams:
            torch.cuda.current_stream(dev).wait_stream(s)
        torch.cuda.synchronize()
        for name in names:
            assert torch.equal(outs[name], alone[name]), (rep, name)


def test_concurrent_steps_on_two_streams_match_sequential(dev):
    """Two decode steps with their own pools and workspaces, issued on two streams before
    either is waited for (c4 on the stream kernel, c5b on the split head-per-wave kernel and its
    merge), give the same bits as the same steps run one after the other, three times over."""
    data = {n: to_dev(wl.make_inputs(wl.WORKLOADS[n]), dev) for n in ("c4", "c5b")}
    ref = {}
    for n, d in data.items():
        e = dict(d)
        e["k_cache"], e["v_cache"] = d["k_cache"].clone(), d["v_cache"].clone()
        ref[n] = (run_step(e), e["k_cache"], e["v_cache"])
    torch.cuda.synchronize()
    streams = {"c4": torch.cuda.Stream(dev), "c5b": torch.cuda.Stream(dev)}
    for rep in range(3):
        runs = {}
        for n, d in data.items():
            e = dict(d)
            e["k_cache"], e["v_cache"] = d["k_cache"].clone(), d["v_cache"].clone()
            runs[n] = e
        torch.cuda.synchronize()
        outs = {}
        for n, e in runs.items():
            with torch.cuda.stream(streams[n]):
                outs[n] = run_step(e)
        torch.cuda.synchronize()
        for n, e in runs.items():
            out, kc, vc = ref[n]
            assert torch.equal(outs[n], out), (n, rep)
            assert torch.equal(e["k_cache"].view(torch.int16), kc.view(torch.int16)), (n, rep)
            assert torch.equal(e["v_cache"].view(torch.int16), vc.view(torch.int16)), (n, rep)
