"""Paged KV decode attention and slot-mapping KV write for AMD Instinct MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI (``libpagedkv.so``, declared in
``include/paged_kv.h``). This package is the thin Python binding over it: it marshals torch
tensors into pointers and the current stream, and nothing else. The library is loaded on
first use; if it is missing the call raises, there is no fallback.
"""
from ._binding import (paged_kv_write, paged_decode_attention, paged_decode_step,
                       paged_decode_step_noalloc, prepare_decode_step, PreparedDecodeStep, paged_decode_step_rope,
                       paged_prefill_attention,
                       paged_kv_write_rope,
                       decode_workspace_bytes, decode_plan,
                       prefill_workspace_bytes, prefill_plan,
                       library_path, load_library, abi_version, PagedKVError)

__all__ = ["paged_kv_write", "paged_decode_attention", "paged_decode_step",
           "paged_decode_step_noalloc", "prepare_decode_step", "PreparedDecodeStep", "paged_decode_step_rope",
           "paged_prefill_attention",
           "paged_kv_write_rope",
           "decode_workspace_bytes", "decode_plan",
           "prefill_workspace_bytes", "prefill_plan",
           "library_path", "load_library", "abi_version", "PagedKVError"]
