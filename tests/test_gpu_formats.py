"""The fp16-input and 16-bit-output variants of the attention path, against the CPU oracle.

Inputs: the same seeded fp32 draws as the bf16 workloads, rounded to fp16; the oracle reads
them as binary16 and computes in float64. Outputs: an fp32 output must be within 2e-3 of the
oracle, as for bf16 inputs. A 16-bit output is the fp32 result rounded to nearest even, so it
may differ from the oracle by that rounding as well: it must lie within 2e-3 plus one unit in
the last place of the output format, and it must equal the same launch's fp32 output rounded
to nearest even (by the oracle's rounding function) bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_write_amd import _binding as pk
from paged_kv_decode_write_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = 2e-3
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
# (input format, output format) pairs beyond the bf16 -> fp32 default
PAIRS = [("bf16", "bf16"), ("f16", "f32"), ("f16", "f16")]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pk.load_library()
    return torch.device("cuda:0")


def families(w):
    """The kernel families built for workload w's shape (the stream family takes contexts over
    1024 tokens only, the vector-ALU family group sizes 1, 2, 3, 4 and 8)."""
    out = []
    for k in ("valu", "mfma", "mfma_hw", "mfma_sk"):
        try:
            pk.decode_plan(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_blocks,
                           w.block_size, 0, k)
            out.append(k)
        except pk.PagedKVError:
            pass
    return out


def part_for(kernel, partition):
    """partition_tokens for a kernel family: the stream family always leaves partials, so
    where a test asks for no split (-1) it runs with the family's own automatic slices."""
    return 0 if kernel == "mfma_sk" and partition == -1 else partition


def to_dev(inp, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


_CASES = {}


def decode_case(name, kvt, dev):
    key = (name, kvt)
    if key not in _CASES:
        inp = wl.make_inputs(wl.WORKLOADS[name], dtype=kvt)
        host = wl.to_host_numpy(inp)
        kc, vc = oracle.kv_write(host["k_new"], host["v_new"], host["slot_mapping"],
                                 host["k_cache"], host["v_cache"])
        ref = oracle.decode_attention(host["q"], kc, vc, host["block_tables"],
                                      host["context_lens"], host["scale"], dtype=kvt)
        d = to_dev(inp, dev)
        pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])
        torch.cuda.synchronize()
        assert np.array_equal(wl.to_bits(d["k_cache"]), kc)  # the write is format-blind
        assert np.array_equal(wl.to_bits(d["v_cache"]), vc)
        _CASES[key] = (ref, d)
    return _CASES[key]


def ulp16(x, fmt):
    """Spacing of the 16-bit format at |x|: 8 significant bits for bf16 (exponents from
    -126), 11 for fp16 (exponents from -14)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    if fmt == "bf16":
        return np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))
    return np.ldexp(1.0, (np.maximum(e, -14) - 10).astype(np.int64))


def out_values(out, ot):
    """Float64 values of a GPU output tensor of format ot."""
    if ot == "f32":
        return out.cpu().double().numpy()
    return oracle.decode_bits(wl.to_bits(out), ot)


def check_output(out, ref, ot, key, out_f32=None):
    """Compare a GPU output with the float64 oracle under the rules in the module docstring;
    with out_f32 (the same launch's fp32 output) also check that the 16-bit output is that
    fp32 result rounded to nearest even, bit for bit. Returns the max |error|."""
    got = out_values(out, ot)
    assert np.isfinite(got).all(), key
    err = np.abs(got - ref)
    if ot == "f32":
        assert err.max() <= ATOL, (key, err.max())
        return float(err.max())
    assert (err <= ATOL + ulp16(ref, ot)).all(), (key, err.max())
    enc = oracle.f64_to_bf16_bits if ot == "bf16" else oracle.f64_to_f16_bits
    bits = wl.to_bits(out)
    if out_f32 is not None:
        want = enc(out_f32.cpu().double().numpy())
        assert np.array_equal(bits, want), (key, int((bits != want).sum()))
    match = float((bits == enc(ref)).mean())
    print(f"[formats] {key}: max|err| = {err.max():.3e}, equal to the rounded oracle in "
          f"{match:.4f} of places", flush=True)
    return float(err.max())


def run_decode(d, ot, kernel="auto", partition=0):
    w = d["workload"]
    out = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), dtype=TORCH[ot],
                     device=d["q"].device)
    pk.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                              d["context_lens"], d["scale"], out,
                              partition_tokens=part_for(kernel, partition),
                              kernel=kernel)
    return out


@pytest.mark.parametrize("kvt,ot", PAIRS)
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_decode_formats_all_kernels_and_splits(dev, name, kvt, ot):
    ref, d = decode_case(name, kvt, dev)
    w = wl.WORKLOADS[name]
    for kernel in families(w):
        for part in (-1, 0, 256):
            out = run_decode(d, ot, kernel, part)
            full = run_decode(d, "f32", kernel, part) if ot != "f32" else None
            check_output(out, ref, ot, f"{name}/{kvt}->{ot}/{kernel}/p{part}", full)


@pytest.mark.parametrize("kvt,ot", PAIRS)
def test_decode_formats_with_32_token_blocks(dev, kvt, ot):
    """The formats with 32-token blocks (the ragged c4 shape): every kernel family and split
    against the oracle, and the 16-bit output the launch's fp32 result rounded."""
    import dataclasses
    base = wl.WORKLOADS["c4"]
    w = dataclasses.replace(base, name="c4_bs32", block_size=32, max_blocks=base.max_blocks // 2,
                            num_blocks=base.num_blocks // 2)
    inp = wl.make_inputs(w, dtype=kvt)
    host = wl.to_host_numpy(inp)
    kc, vc = oracle.kv_write(host["k_new"], host["v_new"], host["slot_mapping"],
                             host["k_cache"], host["v_cache"])
    ref = oracle.decode_attention(host["q"], kc, vc, host["block_tables"],
                                  host["context_lens"], host["scale"], dtype=kvt)
    d = to_dev(inp, dev)
    pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])
    for kernel in families(w):
        for part in (-1, 0, 256):
            out = run_decode(d, ot, kernel, part)
            full = run_decode(d, "f32", kernel, part) if ot != "f32" else None
            check_output(out, ref, ot, f"c4_bs32/{kvt}->{ot}/{kernel}/p{part}", full)


@pytest.mark.parametrize("kvt,ot", PAIRS)
def test_decode_formats_full_size(dev, kvt, ot):
    """c5b (2 x 32768 tokens, logits std 3) in the launch the benchmark times: every output
    row against the oracle, and a 16-bit output equal to the same launch's fp32 output
    rounded."""
    w = wl.WORKLOADS["c5b"]
    inp = wl.make_inputs(w, dtype=kvt)
    host = wl.to_host_numpy(inp)
    d = to_dev(inp, dev)
    pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])
    kc, vc = oracle.kv_write(host["k_new"], host["v_new"], host["slot_mapping"],
                             host["k_cache"], host["v_cache"])
    ref = oracle.decode_attention(host["q"], kc, vc, host["block_tables"], host["context_lens"],
                                  host["scale"], dtype=kvt)
    out = run_decode(d, ot)
    full = run_decode(d, "f32") if ot != "f32" else None
    check_output(out, ref, ot, f"c5b/{kvt}->{ot}/all_rows", full)


def test_f16_small_weights_still_count(dev):
    """One key outweighs each of the other 32767 by about 2^21 (scores of the others spread a
    little, so their weights are no powers of two), and the others' values average +1 against
    -1 for the large key. Unlifted, a weight of 2^-21 is an fp16 subnormal with three
    significant bits; truncating all of them shifts the output by ~1e-3 (emulated on the CPU
    for the one-wave-per-head kernel without a split). Lifted by 2^7 the shift is below 1e-5.
    The output must match the oracle to 1e-4."""
    L, Hq, Hkv, D, bs = 32768, 4, 1, 128, 16
    NB = L // bs
    g = torch.Generator().manual_seed(5)
    q = torch.randn(1, Hq, D, generator=g).to(torch.float16)
    scale = 1.0 / np.sqrt(D)
    a = 21 * float(np.log(2.0))
    k = torch.randn(L, Hkv, D, generator=g) * 0.05
    qf = q.float()[0, 0]
    k[0, 0] = qf * (a / scale / float(qf @ qf))  # s_0 = a for head 0 (other heads differ)
    v = 1.0 + 0.1 * torch.randn(L, Hkv, D, generator=g)
    v[0] = -1.0
    perm = torch.randperm(NB, generator=g)
    kc = torch.empty(NB, bs, Hkv, D, dtype=torch.float16)
    vc = torch.empty(NB, bs, Hkv, D, dtype=torch.float16)
    kc[perm] = k.to(torch.float16).view(NB, bs, Hkv, D)
    vc[perm] = v.to(torch.float16).view(NB, bs, Hkv, D)
    tables = perm.to(torch.int32)[None]
    lens = torch.tensor([L], dtype=torch.int32)
    ref = oracle.decode_attention(wl.to_bits(q), wl.to_bits(kc), wl.to_bits(vc), tables.numpy(),
                                  lens.numpy(), scale, dtype="f16")
    dq, dkc, dvc = q.to(dev), kc.to(dev), vc.to(dev)
    for kernel in ("mfma", "mfma_hw", "mfma_sk", "valu"):
        for part in (-1, 0):
            out = torch.empty(1, Hq, D, dtype=torch.float32, device=dev)
            pk.paged_decode_attention(dq, dkc, dvc, tables.to(dev), lens.to(dev), scale, out,
                                      partition_tokens=part_for(kernel, part), kernel=kernel)
            err = np.abs(out.cpu().double().numpy() - ref).max()
            print(f"[formats] f16 small weights {kernel}/p{part}: {err:.3e}", flush=True)
            assert err <= 1e-4, (kernel, part, err)


_PCASES = {}


def prefill_case(name, kvt, dev):
    key = (name, kvt)
    if key not in _PCASES:
        w = wl.PREFILL_WORKLOADS[name]
        inp = wl.make_prefill_inputs(w, dtype=kvt)
        host = wl.to_host_numpy(inp)
        kc, vc = oracle.kv_write(host["k_new"], host["v_new"], host["slot_mapping"],
                                 host["k_cache"], host["v_cache"])
        ref = oracle.prefill_attention(host["q"], host["cu_seqlens_q"], kc, vc,
                                       host["block_tables"], host["context_lens"],
                                       host["scale"], dtype=kvt)
        d = to_dev(inp, dev)
        pk.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])
        _PCASES[key] = (ref, d)
    return _PCASES[key]


@pytest.mark.parametrize("row_blocks", [0, 1, 4])
@pytest.mark.parametrize("kvt,ot", PAIRS)
@pytest.mark.parametrize("name", ["p2", "p3"])
def test_prefill_formats(dev, name, kvt, ot, row_blocks):
    ref, d = prefill_case(name, kvt, dev)
    T, Hq, D = d["q"].shape

    def run(fmt):
        out = torch.full((T, Hq, D), float("nan"), dtype=TORCH[fmt], device=dev)
        pk.paged_prefill_attention(d["q"], d["cu_seqlens_q"], d["k_cache"], d["v_cache"],
                                   d["block_tables"], d["context_lens"], d["scale"], out,
                                   max_q_len=d["max_q_len"], row_blocks=row_blocks)
        return out

    full = run("f32") if ot != "f32" else None
    check_output(run(ot), ref, ot, f"{name}/prefill/{kvt}->{ot}/rb{row_blocks}", full)


def test_binding_rejects_mixed_formats(dev):
    d = decode_case("c1", "f16", dev)[1]
    w = d["workload"]
    out = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):  # fp16 inputs, bf16 output
        pk.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                  d["context_lens"], d["scale"], out)
    with pytest.raises(ValueError):  # bf16 q with fp16 caches
        pk.paged_decode_attention(d["q"].to(torch.bfloat16), d["k_cache"], d["v_cache"],
                                  d["block_tables"], d["context_lens"], d["scale"],
                                  out.float())


@pytest.mark.parametrize("kvt,ot", PAIRS)
@pytest.mark.parametrize("name", ["c2", "c4"])
def test_decode_step_formats_match_separate_calls(dev, name, kvt, ot):
    """The fused decode step (write + attention in one launch) with fp16 inputs or a 16-bit
    output equals the separate write and attention calls bit for bit, pools included, for
    every kernel family and split."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, dtype=kvt, poison=True)
    for kernel in ["auto"] + families(w):
        for part in (-1, 0, 256):
            fused, sep = to_dev(inp, dev), to_dev(inp, dev)
            out_f = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"),
                               dtype=TORCH[ot], device=dev)
            pk.paged_decode_step(fused["q"], fused["k_new"], fused["v_new"],
                                 fused["slot_mapping"], fused["k_cache"], fused["v_cache"],
                                 fused["block_tables"], fused["context_lens"], fused["scale"],
                                 out_f, partition_tokens=part_for(kernel, part), kernel=kernel)
            pk.paged_kv_write(sep["k_new"], sep["v_new"], sep["slot_mapping"], sep["k_cache"],
                              sep["v_cache"])
            out_s = run_decode(sep, ot, kernel, part)
            torch.cuda.synchronize()
            key = (name, kvt, ot, kernel, part)
            if ot == "f32":
                assert torch.equal(out_f, out_s), key
            else:
                assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16)), key
            for pool in ("k_cache", "v_cache"):
                assert torch.equal(fused[pool].view(torch.int16), sep[pool].view(torch.int16))
