"""The C-ABI library without a GPU: it loads, exports every declared symbol, and rejects bad
arguments on the host with the documented status codes before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_decode_write_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_kv.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_ALIGN = range(7)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.library_path()):
        pytest.skip("libpagedkv.so not built")
    return _binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("paged_kv_write", "paged_decode_attention", "paged_decode_attention_ex",
                 "paged_decode_attention_typed", "paged_prefill_attention",
                 "paged_prefill_attention_ex", "paged_kv_write_rope", "paged_decode_step", "paged_decode_step_rope",
                 "paged_decode_workspace_bytes", "paged_kv_status_string", "paged_kv_abi_version",
                 "paged_kv_last_error", "paged_decode_plan", "paged_prefill_attention_split",
                 "paged_prefill_workspace_bytes", "paged_prefill_plan", "paged_kv_checked_build",
                 "paged_kv_check_status"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (paged_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings(lib):
    assert lib.paged_kv_abi_version() == 6
    assert lib.paged_kv_status_string(OK) == b"PAGEDKV_OK"
    assert lib.paged_kv_status_string(ERR_WORKSPACE) == b"PAGEDKV_ERR_WORKSPACE"
    assert lib.paged_kv_status_string(99) == b"PAGEDKV_UNKNOWN_STATUS"


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced: the host rejects first


def _write(lib, k=FAKE, v=FAKE, slots=FAKE, T=4, kc=FAKE, vc=FAKE, NB=8, bs=16, Hkv=8, D=128):
    return lib.paged_kv_write(k, v, slots, T, kc, vc, NB, bs, Hkv, D, None)


def test_write_argument_errors(lib):
    assert _write(lib, T=-1) == ERR_SHAPE
    assert _write(lib, NB=0) == ERR_SHAPE
    assert _write(lib, bs=0) == ERR_SHAPE
    assert _write(lib, Hkv=1, D=6) == ERR_UNSUPPORTED
    assert _write(lib, k=None) == ERR_NULL
    assert _write(lib, vc=None) == ERR_NULL
    assert _write(lib, k=FAKE + 2) == ERR_ALIGN
    assert _write(lib, slots=FAKE + 4) == ERR_ALIGN
    assert _write(lib, T=0, k=None, v=None) == OK  # nothing to do, nothing touched
    assert b"non-NULL" in (_write(lib, k=None) and lib.paged_kv_last_error())


BF16, F16, F32 = 0, 1, 2


def _attn(lib, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, MB=8, lens=FAKE, B=2, Hq=32, Hkv=8, D=128,
          bs=16, NB=64, out=FAKE, ws=None, wsb=0, part=-1, kernel=0, kvt=BF16, ot=F32,
          scale=0.1):
    return lib.paged_decode_attention_ex(q, kc, vc, bt, MB, lens, B, Hq, Hkv, D, bs, NB, scale,
                                         kvt, out, ot, ws, wsb, part, kernel, None, None, None)


def test_attention_argument_errors(lib):
    assert _attn(lib, B=-1) == ERR_SHAPE
    assert _attn(lib, Hq=30) == ERR_SHAPE           # not a multiple of Hkv
    assert _attn(lib, NB=0) == ERR_SHAPE
    assert _attn(lib, D=96) == ERR_UNSUPPORTED
    assert _attn(lib, bs=8) == ERR_UNSUPPORTED
    assert _attn(lib, bs=24) == ERR_UNSUPPORTED      # blocks: multiples of 16 only
    assert _attn(lib, bs=2048, MB=2) == ERR_UNSUPPORTED
    assert _attn(lib, bs=32, part=48) == ERR_SHAPE   # partitions: multiples of block_size
    assert _attn(lib, kernel=7) == ERR_UNSUPPORTED
    assert _attn(lib, kernel=1, Hq=40) == ERR_UNSUPPORTED  # G=5 has no VALU build
    assert _attn(lib, q=None) == ERR_NULL
    assert _attn(lib, out=None) == ERR_NULL
    assert _attn(lib, q=FAKE + 8) == ERR_ALIGN
    assert _attn(lib, B=0, q=None, out=None) == OK  # empty batch: no-op


def test_format_pairs(lib):
    # bf16 or fp16 inputs; fp32 output or the input's own format (checked before any sizes)
    for kvt, ot in ((BF16, F32), (BF16, BF16), (F16, F32), (F16, F16)):
        assert _attn(lib, B=0, q=None, out=None, kvt=kvt, ot=ot) == OK
        assert _prefill(lib, T=0, q=None, out=None, kvt=kvt, ot=ot) == OK
    for kvt, ot in ((BF16, F16), (F16, BF16), (F32, F32), (3, F32), (BF16, 7), (-1, F32)):
        assert _attn(lib, kvt=kvt, ot=ot) == ERR_UNSUPPORTED
        assert _prefill(lib, kvt=kvt, ot=ot) == ERR_UNSUPPORTED
    assert b"format" in lib.paged_kv_last_error()
    st = lib.paged_decode_attention_typed(FAKE, FAKE, FAKE, FAKE, 8, FAKE, 0, 32, 8, 128, 16, 64,
                                          0.1, F16, None, F16, None, 0, 0, None)
    assert st == OK
    st = lib.paged_decode_attention_typed(FAKE, FAKE, FAKE, FAKE, 8, FAKE, 2, 32, 8, 128, 16, 64,
                                          0.1, F16, FAKE, BF16, None, 0, 0, None)
    assert st == ERR_UNSUPPORTED


def _step(lib, q=FAKE, kn=FAKE, vn=FAKE, sl=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, MB=8, lens=FAKE,
          B=2, Hq=32, Hkv=8, D=128, bs=16, NB=64, out=FAKE):
    return lib.paged_decode_step(q, kn, vn, sl, kc, vc, bt, MB, lens, B, Hq, Hkv, D, bs, NB, 0.1,
                                 BF16, out, F32, None, 0, -1, 0, None, None, None)


def test_decode_step_argument_errors(lib):
    assert _step(lib, kn=None) == ERR_NULL
    assert _step(lib, sl=None) == ERR_NULL
    assert _step(lib, vn=FAKE + 8) == ERR_ALIGN
    assert _step(lib, sl=FAKE + 4) == ERR_ALIGN
    assert _step(lib, D=96) == ERR_UNSUPPORTED
    assert _step(lib, B=0, q=None, kn=None, out=None) == OK  # empty batch: no-op


def _prefill(lib, q=FAKE, cu=FAKE, T=8, maxq=4, kc=FAKE, vc=FAKE, bt=FAKE, MB=8, lens=FAKE,
             B=2, Hq=32, Hkv=8, D=128, bs=16, NB=64, out=FAKE, rb=0, kvt=BF16, ot=F32,
             scale=0.1):
    return lib.paged_prefill_attention_ex(q, cu, T, maxq, kc, vc, bt, MB, lens, B, Hq, Hkv, D,
                                          bs, NB, scale, kvt, out, ot, rb, None)


def test_prefill_argument_errors(lib):
    assert _prefill(lib, rb=3) == ERR_SHAPE
    assert _prefill(lib, rb=8) == ERR_SHAPE
    assert _prefill(lib, T=-1) == ERR_SHAPE
    assert _prefill(lib, maxq=-1) == ERR_SHAPE
    assert _prefill(lib, Hq=30) == ERR_SHAPE
    assert _prefill(lib, D=96) == ERR_UNSUPPORTED
    assert _prefill(lib, Hq=34, Hkv=2) == ERR_UNSUPPORTED  # group of 17 query heads
    assert _prefill(lib, bs=8) == ERR_UNSUPPORTED     # blocks: 16 << k tokens only
    assert _prefill(lib, bs=48) == ERR_UNSUPPORTED
    assert _prefill(lib, bs=2048, MB=2) == ERR_UNSUPPORTED
    assert _prefill(lib, bs=64, T=0, q=None, out=None) == OK  # 64-token blocks are taken
    assert _prefill(lib, q=None) == ERR_NULL
    assert _prefill(lib, cu=None) == ERR_NULL
    assert _prefill(lib, out=FAKE + 4) == ERR_ALIGN
    assert _prefill(lib, T=0, q=None, out=None) == OK  # no query rows: no-op


def _prefill_split(lib, ws=None, ws_bytes=0, part=0, T=8, maxq=4, MB=8, q=FAKE, rb=0):
    return lib.paged_prefill_attention_split(q, FAKE, T, maxq, FAKE, FAKE, FAKE, MB, FAKE, 2, 32,
                                             8, 128, 16, 64, 0.1, BF16, FAKE, F32, rb, ws,
                                             ws_bytes, part, None)


def test_prefill_split_argument_errors(lib):
    assert _prefill_split(lib, part=-2) == ERR_SHAPE
    assert _prefill_split(lib, part=48) == ERR_SHAPE       # not a multiple of 32 keys
    assert _prefill_split(lib, rb=3) == ERR_SHAPE
    assert _prefill_split(lib, q=None) == ERR_NULL
    assert _prefill_split(lib, T=0, q=None) == OK           # no query rows: no-op


def test_prefill_workspace_bytes(lib):
    f = lib.paged_prefill_workspace_bytes
    assert f(100, 24, 128, 256, 16, -1) == 0                # never split
    assert f(100, 24, 128, 128, 16, 0) == 0                 # 2048 keys: auto never splits
    # auto over 4096 keys: at most 3 partitions (of 1376 keys)
    acc = 100 * 24 * 128 * 4
    ml = 100 * 24 * 2 * 4
    r = lambda x: (x + 255) // 256 * 256
    assert f(100, 24, 128, 256, 16, 0) == r(3 * acc) + r(3 * ml)
    assert f(100, 24, 128, 256, 16, 1376) == r(3 * acc) + r(3 * ml)
    assert f(100, 24, 128, 256, 16, 1024) == r(4 * acc) + r(4 * ml)
    # forced 512-key partitions: 8 of them
    assert f(100, 24, 128, 256, 16, 512) == r(8 * acc) + r(8 * ml)
    assert f(100, 24, 128, 256, 16, 48) == 0                # not a multiple of 32
    assert f(0, 24, 128, 256, 16, 0) == 0


def test_workspace_bytes(lib):
    f = lib.paged_decode_workspace_bytes
    assert f(64, 32, 128, 512, 16, -1) == 0              # never split
    assert f(1, 32, 64, 8, 16, 0) == 0                   # 128 tokens: auto never splits
    def split(n):  # n partial slots of D + 2 floats per (sequence, query head)
        return 2 * 32 * n * 128 * 4 + 2 * 32 * n * 2 * 4
    # forced 256-token partitions over 32768 tokens: 128 partitions; the stream family, with
    # at least 8 pairs of 32 tokens per workgroup, can need (1024 - 1) // 8 + 2 = 129 slots
    assert f(2, 32, 128, 2048, 16, 256) == split(129)
    # auto bound: partitions of at least 256 tokens (128), or the stream family's 16 at most
    assert f(2, 32, 128, 2048, 16, 0) == split(128)
    assert f(2, 32, 128, 2048, 16, 24) == 0               # not a multiple of block_size
    assert f(0, 32, 128, 2048, 16, 0) == 0
    # 2048 tokens: 8 partitions of 256, or the stream family's (64 - 1) // 8 + 2 = 9 slots
    assert f(2, 32, 128, 128, 16, 0) == split(9)
    # blocks of 32 or 64 tokens: the same split region, then the table of 16-token block ids
    # (batch x max_blocks x block_size/16 int32, rounded up to 256 bytes)
    assert f(2, 32, 128, 1024, 32, 256) == split(129) + 2 * 1024 * 2 * 4
    assert f(2, 32, 128, 512, 64, 0) == split(128) + 2 * 512 * 4 * 4
    assert f(3, 8, 64, 5, 32, -1) == 256                 # 3 x 10 ids, one 256-byte granule


def test_binding_rejects_cpu_tensors():
    import torch
    k = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _binding.paged_kv_write(k, k, torch.zeros(2, dtype=torch.int64),
                                torch.zeros(4, 16, 8, 128, dtype=torch.bfloat16),
                                torch.zeros(4, 16, 8, 128, dtype=torch.bfloat16))


def _step_rope(lib, q=FAKE, kn=FAKE, vn=FAKE, pos=FAKE, freq=FAKE, il=0, sl=FAKE, qo=FAKE + 4096,
               kc=FAKE, vc=FAKE, bt=FAKE, MB=8, lens=FAKE, B=2, Hq=32, Hkv=8, D=128, bs=16,
               NB=64, out=FAKE, kvt=BF16, kernel=0):
    return lib.paged_decode_step_rope(q, kn, vn, pos, freq, il, sl, qo, kc, vc, bt, MB, lens, B,
                                      Hq, Hkv, D, bs, NB, 0.1, kvt, out, F32, None, 0, -1,
                                      kernel, None, None, None)


def test_decode_step_rope_argument_errors(lib):
    # q is 2 x 32 x 128 bf16 = 16 KiB from FAKE: q_out at FAKE + 4096 overlaps it
    assert _step_rope(lib, pos=None) == ERR_NULL
    assert _step_rope(lib, freq=None) == ERR_NULL
    assert _step_rope(lib, qo=None) == ERR_NULL
    assert _step_rope(lib, kn=None) == ERR_NULL
    assert _step_rope(lib, il=2, qo=FAKE + 16384) == ERR_SHAPE
    assert b"interleaved" in lib.paged_kv_last_error()
    assert _step_rope(lib, kvt=F16) == ERR_UNSUPPORTED
    assert _step_rope(lib, freq=FAKE + 8) == ERR_ALIGN
    assert _step_rope(lib, qo=FAKE + 4104) == ERR_ALIGN
    assert _step_rope(lib, pos=FAKE + 2) == ERR_ALIGN
    assert _step_rope(lib) == ERR_SHAPE  # q_out overlaps q
    assert b"overlap" in lib.paged_kv_last_error()
    assert _step_rope(lib, D=96) == ERR_UNSUPPORTED
    assert _step_rope(lib, B=0, q=None, kn=None, out=None, qo=None) == OK  # empty batch: no-op


def test_larger_blocks_need_the_table_workspace(lib, monkeypatch):
    """A call with blocks of 32 tokens writes its table of 16-token block ids into the
    workspace, so it needs one even when it does not split; the check comes before any
    launch."""
    monkeypatch.setenv("PAGEDKV_CU_COUNT", "256")
    assert _attn(lib, bs=32, part=-1) == ERR_WORKSPACE
    assert b"workspace" in lib.paged_kv_last_error()



def _step_noalloc(lib, q=FAKE, kn=FAKE, vn=FAKE, sl=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, MB=8,
                  lens=FAKE, B=2, Hq=32, Hkv=8, D=128, bs=16, NB=64, out=FAKE, part=-1):
    return lib.paged_decode_step_noalloc(q, kn, vn, sl, kc, vc, bt, MB, lens, B, Hq, Hkv, D, bs,
                                         NB, 0.1, BF16, out, F32, part, 0, None, None, None)


def test_decode_step_noalloc_host_checks(lib, monkeypatch):
    """The no-workspace step validates like paged_decode_step, and refuses on the host, before
    any device call, a plan whose partials exceed its static scratch: 64 x 8192 tokens in
    16-token partitions need 64*32*512*130*4 bytes."""
    monkeypatch.setenv("PAGEDKV_CU_COUNT", "256")
    assert _step_noalloc(lib, kn=None) == ERR_NULL
    assert _step_noalloc(lib, vn=FAKE + 8) == ERR_ALIGN
    assert _step_noalloc(lib, D=96) == ERR_UNSUPPORTED
    assert _step_noalloc(lib, B=0, q=None, kn=None, out=None) == OK
    assert _step_noalloc(lib, B=64, MB=512, NB=32768, part=16) == ERR_WORKSPACE
    msg = lib.paged_kv_last_error()
    assert b"static scratch" in msg and str(64 * 32 * 512 * 130 * 4).encode() in msg


def test_unchecked_build_has_no_check_record(lib):
    """The default library validates nothing on the device: it says so, and the status call
    refuses before touching the device."""
    assert lib.paged_kv_checked_build() == 0
    code = ctypes.c_int32(-1)
    assert lib.paged_kv_check_status(ctypes.byref(code), None, None, 1) == ERR_UNSUPPORTED
    assert code.value == -1


def test_checked_build_loads_and_exports_everything():
    """libpagedkv_checked.so (PAGEDKV_CHECKED) is built beside the default library, exports
    every declared symbol, reports itself checked, and checks its arguments on the host."""
    path = _binding.checked_library_path()
    if not os.path.exists(path):
        pytest.skip("libpagedkv_checked.so not built")
    ck = _binding.load_checked_library()
    assert ck.paged_kv_checked_build() == 1
    assert ck.paged_kv_abi_version() == 6
    for name in declared_functions():
        assert hasattr(ck, name), name
    assert ck.paged_kv_check_status(None, None, None, 1) == ERR_NULL
    # host-side argument checks are the same as in the default build
    assert _write(ck, T=-1) == ERR_SHAPE
    assert _write(ck, k=None) == ERR_NULL


def test_probe_library_exports_its_declared_symbols():
    """The measurement utility libpagedkv_probe.so exports every call paged_kv_probe.h
    declares (the benchmark's read probe loads them by name)."""
    path = os.path.join(os.path.dirname(_binding.library_path()), "libpagedkv_probe.so")
    if not os.path.exists(path):
        pytest.skip("libpagedkv_probe.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "paged_kv_probe.h")).read(),
                  flags=re.S)
    declared = set(re.findall(r"\b(pagedkv_\w+)\s*\(", text))
    assert {"pagedkv_read_probe", "pagedkv_read_probe_nt", "pagedkv_read_probe_chunked_nt"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    assert declared <= set(re.findall(r"\bT (pagedkv_\w+)", out))
