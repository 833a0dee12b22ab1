"""ctypes binding of libpagedkv (declared in include/paged_kv.h).

Argument marshalling only: shape/dtype/device checks, torch tensors to device pointers, the
current HIP stream. Every step of the computation runs in the library's HIP kernels. There
is no fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libpagedkv.so"
CHECKED_LIB_NAME = "libpagedkv_checked.so"

STATUS_NAMES = {0: "PAGEDKV_OK", 1: "PAGEDKV_ERR_NULL", 2: "PAGEDKV_ERR_SHAPE",
                3: "PAGEDKV_ERR_UNSUPPORTED", 4: "PAGEDKV_ERR_WORKSPACE", 5: "PAGEDKV_ERR_HIP",
                6: "PAGEDKV_ERR_ALIGN"}
KERNELS = {"auto": 0, "valu": 1, "mfma": 2, "mfma_hw": 3, "mfma_sk": 4}
# pagedkv_dtype values of the tensor element types the library takes.
DTYPES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}
INPUT_TYPES = (torch.bfloat16, torch.float16)

_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None
# One workspace per (device, stream), grown on demand and reused, so steady-state calls
# allocate nothing.
_workspaces = {}


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def library_path() -> str:
    return os.environ.get("PAGEDKV_LIBRARY", os.path.join(_HERE, LIB_NAME))


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C signatures of every entry point on a loaded library."""
    P, I32, I64, SZ, F32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_size_t, ctypes.c_float)
    lib.paged_kv_abi_version.restype = ctypes.c_int
    lib.paged_kv_abi_version.argtypes = []
    lib.paged_kv_status_string.restype = ctypes.c_char_p
    lib.paged_kv_status_string.argtypes = [ctypes.c_int]
    lib.paged_kv_last_error.restype = ctypes.c_char_p
    lib.paged_kv_last_error.argtypes = []
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_kv_write.argtypes = [P, P, P, I64, P, P, I64, I32, I32, I32, P]
    lib.paged_decode_workspace_bytes.restype = SZ
    lib.paged_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    attn = [P, P, P, P, I32, P, I32, I32, I32, I32, I32, I64, F32, P, P, SZ, I32]
    lib.paged_decode_attention.restype = ctypes.c_int
    lib.paged_decode_attention.argtypes = attn + [P]
    typed = attn[:13] + [I32, P, I32, P, SZ, I32]
    lib.paged_decode_attention_typed.restype = ctypes.c_int
    lib.paged_decode_attention_typed.argtypes = typed + [P]
    lib.paged_decode_attention_ex.restype = ctypes.c_int
    lib.paged_decode_attention_ex.argtypes = typed + [I32, P, P, P]
    lib.paged_decode_step.restype = ctypes.c_int
    lib.paged_decode_step.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32,
                                      I64, F32, I32, P, I32, P, SZ, I32, I32, P, P, P]
    lib.paged_decode_step_noalloc.restype = ctypes.c_int
    lib.paged_decode_step_noalloc.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I32, I32,
                                              I32, I32, I64, F32, I32, P, I32, I32, I32, P,
                                              P, P]
    lib.paged_decode_step_rope.restype = ctypes.c_int
    lib.paged_decode_step_rope.argtypes = [P, P, P, P, P, I32, P, P, P, P, P, I32, P, I32,
                                           I32, I32, I32, I32, I64, F32, I32, P, I32, P, SZ,
                                           I32, I32, P, P, P]
    lib.paged_kv_write_rope.restype = ctypes.c_int
    lib.paged_kv_write_rope.argtypes = [P, P, P, P, P, I32, P, I64, P, P, P, I64, I32, I32,
                                        I32, I32, P]
    lib.paged_prefill_attention.restype = ctypes.c_int
    lib.paged_prefill_attention.argtypes = [P, P, I64, I32, P, P, P, I32, P, I32, I32, I32,
                                            I32, I32, I64, F32, P, P]
    lib.paged_prefill_attention_ex.restype = ctypes.c_int
    lib.paged_prefill_attention_ex.argtypes = [P, P, I64, I32, P, P, P, I32, P, I32, I32,
                                               I32, I32, I32, I64, F32, I32, P, I32, I32,
                                               P]
    lib.paged_decode_plan.restype = ctypes.c_int
    lib.paged_decode_plan.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32,
                                      ctypes.POINTER(I32), ctypes.POINTER(I32),
                                      ctypes.POINTER(I32)]
    lib.paged_prefill_attention_split.restype = ctypes.c_int
    lib.paged_prefill_attention_split.argtypes = [P, P, I64, I32, P, P, P, I32, P, I32, I32,
                                                  I32, I32, I32, I64, F32, I32, P, I32, I32,
                                                  P, SZ, I32, P]
    lib.paged_prefill_workspace_bytes.restype = SZ
    lib.paged_prefill_workspace_bytes.argtypes = [I64, I32, I32, I32, I32, I32]
    lib.paged_prefill_plan.restype = ctypes.c_int
    lib.paged_prefill_plan.argtypes = [I64, I32, I32, I32, I32, I32, I32, I32, I32, I32,
                                       ctypes.POINTER(I32), ctypes.POINTER(I32),
                                       ctypes.POINTER(I32)]
    lib.paged_kv_checked_build.restype = ctypes.c_int
    lib.paged_kv_checked_build.argtypes = []
    lib.paged_kv_check_status.restype = ctypes.c_int
    lib.paged_kv_check_status.argtypes = [ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int64), ctypes.c_int32]
    return lib


def load_library() -> ctypes.CDLL:
    """Load libpagedkv.so (after torch, so both share one HIP runtime) and declare the
    C signatures. Raises FileNotFoundError if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it first (python -m paged_kv_decode_write_amd.build)")
        _lib = _declare(ctypes.CDLL(path))
        return _lib


_checked_lib: Optional[ctypes.CDLL] = None


def checked_library_path() -> str:
    return os.path.join(_HERE, CHECKED_LIB_NAME)


def load_checked_library() -> ctypes.CDLL:
    """Load the checked build, libpagedkv_checked.so (the same entry points, each call
    validating its slot ids, block ids, lengths and query spans on the device first), as a
    library of its own: call its entry points directly and read the result with
    check_status(lib)."""
    global _checked_lib
    with _lock:
        if _checked_lib is not None:
            return _checked_lib
        path = checked_library_path()
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it first (python -m paged_kv_decode_write_amd.build)")
        _checked_lib = _declare(ctypes.CDLL(path, mode=os.RTLD_LOCAL))
        return _checked_lib


CHECK_CODES = {0: "none", 1: "slot", 2: "length", 3: "block", 4: "query"}


def check_status(lib: Optional[ctypes.CDLL] = None, clear: bool = True):
    """Synchronise the current device and return the checked build's record as
    (code name, index, value); `clear` resets it."""
    lib = lib or load_checked_library()
    code, index, value = ctypes.c_int32(0), ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib.paged_kv_check_status(ctypes.byref(code), ctypes.byref(index), ctypes.byref(value),
                                   1 if clear else 0)
    if st != 0:
        raise PagedKVError(st, lib.paged_kv_last_error().decode(errors="replace"))
    return CHECK_CODES.get(code.value, code.value), index.value, value.value


def abi_version() -> int:
    return load_library().paged_kv_abi_version()


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().paged_kv_last_error().decode(errors="replace")
        raise PagedKVError(status, msg)


# torch's raw current-stream query (an int handle, no Stream object built); the public
# torch.cuda.current_stream(...).cuda_stream gives the same value at several times the cost,
# which matters for the launch-bound small calls.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device: torch.device) -> int:
    if _raw_stream is not None and device.index is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _device(dev: torch.device):
    """Context making dev the current device for a library call; a no-op when it already is."""
    if dev.index is not None and torch.cuda.current_device() == dev.index:
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _require(t: torch.Tensor, name: str, dtype, ndim: int,
             device: Optional[torch.device] = None) -> None:
    """dtype: one torch dtype, or a tuple of accepted ones."""
    # Fast path: every check passes (cheap attribute reads only).
    if (isinstance(t, torch.Tensor) and t.is_cuda and t.dim() == ndim and
            (t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype) and
            (device is None or t.get_device() == device.index) and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    accepted = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in accepted:
        raise ValueError(f"{name} must be {' or '.join(map(str, accepted))}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def paged_kv_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Store token t's K/V rows (k[t], v[t]: [Hkv, D]) at slot slot_mapping[t] of the pools
    k_cache / v_cache ([NB, block_size, Hkv, D], updated in place), all bf16 or all fp16
    (bit patterns are copied). Negative slots are skipped."""
    _require(k_cache, "k_cache", INPUT_TYPES, 4)
    dev, dt = k_cache.device, k_cache.dtype
    _require(v_cache, "v_cache", dt, 4, dev)
    _require(k, "k", dt, 3, dev)
    _require(v, "v", dt, 3, dev)
    _require(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    NB, bs, Hkv, D = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    T = k.shape[0]
    if k.shape != (T, Hkv, D) or v.shape != (T, Hkv, D) or slot_mapping.shape != (T,):
        raise ValueError(f"k/v must be [T, {Hkv}, {D}] and slot_mapping [T]")
    lib = load_library()
    with _device(dev):
        _check(lib.paged_kv_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), T,
                                  k_cache.data_ptr(), v_cache.data_ptr(), NB, bs, Hkv, D,
                                  _stream_handle(dev)))


def decode_workspace_bytes(batch: int, num_q_heads: int, head_dim: int,
                           max_blocks_per_seq: int, block_size: int,
                           partition_tokens: int = 0) -> int:
    return int(load_library().paged_decode_workspace_bytes(
        batch, num_q_heads, head_dim, max_blocks_per_seq, block_size, partition_tokens))


KERNEL_NAMES = {v: k for k, v in KERNELS.items()}


def prefill_workspace_bytes(num_tokens: int, num_q_heads: int, head_dim: int,
                            max_blocks_per_seq: int, block_size: int,
                            partition_tokens: int = 0) -> int:
    return int(load_library().paged_prefill_workspace_bytes(
        num_tokens, num_q_heads, head_dim, max_blocks_per_seq, block_size, partition_tokens))


def prefill_plan(num_tokens, max_q_len, batch, num_q_heads, num_kv_heads, head_dim,
                 max_blocks_per_seq, block_size, row_blocks=0, partition_tokens=0):
    """(row_blocks, num_partitions, keys_per_partition) the multi-query call would use on
    the current device."""
    nb = ctypes.c_int32(0)
    n = ctypes.c_int32(0)
    p = ctypes.c_int32(0)
    _check(load_library().paged_prefill_plan(num_tokens, max_q_len, batch, num_q_heads,
                                             num_kv_heads, head_dim, max_blocks_per_seq,
                                             block_size, row_blocks, partition_tokens,
                                             ctypes.byref(nb), ctypes.byref(n), ctypes.byref(p)))
    return nb.value, n.value, p.value


def decode_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                partition_tokens=0, kernel="auto", with_kernel=False):
    """(num_partitions, tokens_per_partition[, kernel name]) the call would use on the
    current device."""
    n = ctypes.c_int32(0)
    p = ctypes.c_int32(0)
    k = ctypes.c_int32(0)
    _check(load_library().paged_decode_plan(batch, num_q_heads, num_kv_heads, head_dim,
                                            max_blocks_per_seq, block_size, partition_tokens,
                                            KERNELS[kernel], ctypes.byref(n), ctypes.byref(p),
                                            ctypes.byref(k)))
    if with_kernel:
        return n.value, p.value, KERNEL_NAMES[k.value]
    return n.value, p.value


def _cached_workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    key = (dev.index, _stream_handle(dev))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of nbytes for explicit reuse across calls on one stream."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def paged_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           scale: float, out: torch.Tensor, *, partition_tokens: int = 0,
                           kernel: str = "auto", workspace: Optional[torch.Tensor] = None,
                           events: Optional[tuple] = None) -> torch.Tensor:
    """out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the context_lens[b] cached
    positions of sequence b, read through block_tables[b] (KV head h // (Hq/Hkv)).

    q [B, Hq, D] and k_cache/v_cache [NB, block_size, Hkv, D]: all bf16 or all fp16;
    block_tables [B, MB] int32; context_lens [B] int32; out [B, Hq, D] fp32 or the input
    type (written and returned).
    partition_tokens: 0 automatic, -1 never split, >0 split size in tokens (tests).
    kernel: "auto", "valu", "mfma" or "mfma_hw". workspace: optional uint8 device buffer (see
    new_workspace); when omitted, a cached per-stream workspace is used.
    events: optional (begin, end) raw hipEvent_t handles recorded around the main kernel.
    """
    _require(k_cache, "k_cache", INPUT_TYPES, 4)
    dev, dt = k_cache.device, k_cache.dtype
    _require(v_cache, "v_cache", dt, 4, dev)
    _require(q, "q", dt, 3, dev)
    _require(block_tables, "block_tables", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    _require(out, "out", (torch.float32, dt), 3, dev)
    NB, bs, Hkv, D = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    B, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError(f"q head_dim {Dq} != cache head_dim {D}")
    if out.shape != (B, Hq, D):
        raise ValueError(f"out must be [{B}, {Hq}, {D}]")
    MB = block_tables.shape[1]
    if block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    lib = load_library()
    need = int(lib.paged_decode_workspace_bytes(B, Hq, D, MB, bs, partition_tokens))
    if workspace is None:
        workspace = _cached_workspace(dev, need)
    elif workspace.device != dev or workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor on the cache's device")
    ws_bytes = workspace.numel()
    ev_b, ev_e = events if events is not None else (None, None)
    with _device(dev):
        _check(lib.paged_decode_attention_ex(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), MB,
            context_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, float(scale), DTYPES[dt],
            out.data_ptr(), DTYPES[out.dtype], workspace.data_ptr() if need else None,
            ws_bytes if need else 0, partition_tokens, KERNELS[kernel], ev_b, ev_e,
            _stream_handle(dev)))
    return out


def _check_step(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                out, kernel):
    """Validate the tensors of a decode step; returns (dev, dtype, NB, bs, Hkv, D, B, Hq, MB)."""
    _require(k_cache, "k_cache", INPUT_TYPES, 4)
    dev, dt = k_cache.device, k_cache.dtype
    _require(v_cache, "v_cache", dt, 4, dev)
    _require(q, "q", dt, 3, dev)
    _require(k_new, "k_new", dt, 3, dev)
    _require(v_new, "v_new", dt, 3, dev)
    _require(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    _require(block_tables, "block_tables", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    _require(out, "out", (torch.float32, dt), 3, dev)
    NB, bs, Hkv, D = k_cache.shape
    B, Hq, Dq = q.shape
    if v_cache.shape != k_cache.shape or Dq != D or out.shape != (B, Hq, D):
        raise ValueError("shape mismatch between q, out and the caches")
    if k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D) or slot_mapping.shape != (B,):
        raise ValueError(f"k_new/v_new must be [{B}, {Hkv}, {D}] and slot_mapping [{B}]")
    MB = block_tables.shape[1]
    if block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    return dev, dt, NB, bs, Hkv, D, B, Hq, MB


def _step_workspace(lib, dev, B, Hq, D, MB, bs, partition_tokens, workspace):
    need = int(lib.paged_decode_workspace_bytes(B, Hq, D, MB, bs, partition_tokens))
    if workspace is None:
        workspace = _cached_workspace(dev, need)
    elif workspace.device != dev or workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor on the cache's device")
    return (workspace.data_ptr(), workspace.numel()) if need else (None, 0)


def paged_decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      slot_mapping: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      out: torch.Tensor, *, partition_tokens: int = 0, kernel: str = "auto",
                      workspace: Optional[torch.Tensor] = None,
                      events: Optional[tuple] = None) -> torch.Tensor:
    """The decode step in one call: store k_new[b] / v_new[b] ([B, Hkv, D]) at slot
    slot_mapping[b] ([B] int64) of the pools, then attend as paged_decode_attention does.
    Equals paged_kv_write followed by paged_decode_attention when slot_mapping[b] is the slot
    of position context_lens[b] - 1 of sequence b (or negative); the matrix-core kernels do both
    in one launch."""
    dev, dt, NB, bs, Hkv, D, B, Hq, MB = _check_step(
        q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens, out, kernel)
    lib = load_library()
    ws, wsb = _step_workspace(lib, dev, B, Hq, D, MB, bs, partition_tokens, workspace)
    ev_b, ev_e = events if events is not None else (None, None)
    with _device(dev):
        _check(lib.paged_decode_step(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
            k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), MB,
            context_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, float(scale), DTYPES[dt],
            out.data_ptr(), DTYPES[out.dtype], ws, wsb, partition_tokens, KERNELS[kernel], ev_b,
            ev_e, _stream_handle(dev)))
    return out


def paged_decode_step_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                              slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                              v_cache: torch.Tensor, block_tables: torch.Tensor,
                              context_lens: torch.Tensor, scale: float, out: torch.Tensor, *,
                              partition_tokens: int = 0, kernel: str = "auto",
                              events: Optional[tuple] = None) -> torch.Tensor:
    """paged_decode_step with no workspace: the library keeps the split partials in a static
    device array of its own (PAGEDKV_STATIC_SCRATCH_BYTES per device), so the call allocates
    nothing. Calls that may overlap on one device race on that array."""
    dev, dt, NB, bs, Hkv, D, B, Hq, MB = _check_step(
        q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens, out, kernel)
    lib = load_library()
    ev_b, ev_e = events if events is not None else (None, None)
    with _device(dev):
        _check(lib.paged_decode_step_noalloc(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
            k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), MB,
            context_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, float(scale), DTYPES[dt],
            out.data_ptr(), DTYPES[out.dtype], partition_tokens, KERNELS[kernel], ev_b, ev_e,
            _stream_handle(dev)))
    return out


class PreparedDecodeStep:
    """paged_decode_step bound once to its tensors, for a serving loop that launches the same
    step again and again while updating the tensors in place (new q, k_new, v_new, slots,
    tables and lengths written into the same storage). The checks, the workspace and the
    argument conversion happen once, here; a call reads the current stream and calls the
    library. The object holds references to every bound tensor and to a workspace of its own
    (a shared per-stream workspace could be regrown under it). Calls that may run at the same
    time must not share one prepared step (they share its workspace and output)."""

    __slots__ = ("_fn", "_args", "_dev_index", "_refs", "out")

    def __init__(self, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                 context_lens, scale, out, *, partition_tokens=0, kernel="auto",
                 workspace=None):
        dev, dt, NB, bs, Hkv, D, B, Hq, MB = _check_step(
            q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens, out,
            kernel)
        lib = load_library()
        need = int(lib.paged_decode_workspace_bytes(B, Hq, D, MB, bs, partition_tokens))
        if workspace is None:
            workspace = new_workspace(need, dev) if need else None
        elif (workspace.device != dev or workspace.dtype != torch.uint8 or
              workspace.numel() < need):
            raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on the "
                             "cache's device")
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        ws = P(workspace.data_ptr()) if need else None
        wsb = ctypes.c_size_t(workspace.numel() if need else 0)
        self._args = (
            P(q.data_ptr()), P(k_new.data_ptr()), P(v_new.data_ptr()), P(slot_mapping.data_ptr()),
            P(k_cache.data_ptr()), P(v_cache.data_ptr()), P(block_tables.data_ptr()), I32(MB),
            P(context_lens.data_ptr()), I32(B), I32(Hq), I32(Hkv), I32(D), I32(bs), I64(NB),
            ctypes.c_float(scale), I32(DTYPES[dt]), P(out.data_ptr()), I32(DTYPES[out.dtype]),
            ws, wsb, I32(partition_tokens), I32(KERNELS[kernel]), None, None)
        self._refs = (q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                      context_lens, out, workspace)
        self._fn = lib.paged_decode_step
        self._dev_index = dev.index
        self.out = out

    def __call__(self) -> torch.Tensor:
        idx = self._dev_index
        if torch.cuda.current_device() != idx:
            with torch.cuda.device(idx):
                return self()
        stream = (_raw_stream(idx) if _raw_stream is not None
                  else torch.cuda.current_stream(idx).cuda_stream)
        status = self._fn(*self._args, stream)
        if status:
            _check(status)
        return self.out


def prepare_decode_step(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                        context_lens, scale, out, **kw) -> PreparedDecodeStep:
    """A PreparedDecodeStep for these tensors (arguments as in paged_decode_step)."""
    return PreparedDecodeStep(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                              context_lens, scale, out, **kw)


def paged_decode_step_rope(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                           positions: torch.Tensor, inv_freq: torch.Tensor,
                           slot_mapping: torch.Tensor, q_out: torch.Tensor,
                           k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                           out: torch.Tensor, *, interleaved: bool = False,
                           partition_tokens: int = 0, kernel: str = "auto",
                           workspace: Optional[torch.Tensor] = None,
                           events: Optional[tuple] = None) -> torch.Tensor:
    """paged_decode_step with rotary embedding in front: q and k_new (bf16, not rotated) are
    rotated at positions[b] ([B] int32) by inv_freq ([D/2] fp32); the rotated q goes to q_out
    ([B, Hq, D], separate from q), the rotated key into the cache, and attention uses both.
    Equals paged_kv_write_rope followed by paged_decode_attention(q_out, ...) bit for bit."""
    dev, dt, NB, bs, Hkv, D, B, Hq, MB = _check_step(
        q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens, out, kernel)
    _require(positions, "positions", torch.int32, 1, dev)
    _require(inv_freq, "inv_freq", torch.float32, 1, dev)
    _require(q_out, "q_out", dt, 3, dev)
    if positions.shape != (B,) or inv_freq.shape != (D // 2,) or q_out.shape != q.shape:
        raise ValueError(f"positions must be [{B}], inv_freq [{D // 2}] and q_out like q")
    lib = load_library()
    ws, wsb = _step_workspace(lib, dev, B, Hq, D, MB, bs, partition_tokens, workspace)
    ev_b, ev_e = events if events is not None else (None, None)
    with _device(dev):
        _check(lib.paged_decode_step_rope(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), positions.data_ptr(),
            inv_freq.data_ptr(), int(bool(interleaved)), slot_mapping.data_ptr(),
            q_out.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), MB,
            context_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, float(scale), DTYPES[dt],
            out.data_ptr(), DTYPES[out.dtype], ws, wsb, partition_tokens, KERNELS[kernel], ev_b,
            ev_e, _stream_handle(dev)))
    return out


def paged_prefill_attention(q: torch.Tensor, cu_seqlens_q: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, scale: float, out: torch.Tensor, *,
                            max_q_len: Optional[int] = None, row_blocks: int = 0,
                            partition_tokens: int = 0,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Multi-query causal attention over the paged cache (prefill / chunked prefill).

    Sequence b's query rows are q[cu_seqlens_q[b]:cu_seqlens_q[b+1]], its last Q_b positions;
    row i attends to positions 0 .. context_lens[b] - Q_b + i. q [T, Hq, D] and the caches
    bf16 or fp16 alike, cu_seqlens_q [B+1] int32, out [T, Hq, D] fp32 or the input type.
    max_q_len (the largest Q_b) sizes the launch; when
    omitted it is read from cu_seqlens_q, which synchronises with the device. row_blocks
    (1, 2 or 4; 0 = chosen by the library) is the number of 16-row query blocks per wave.
    partition_tokens splits each query tile's keys (0 = the library's choice, -1 = never, > 0
    = that many keys, a multiple of 32); a split uses `workspace` (uint8, reused per stream
    when not given).
    """
    _require(k_cache, "k_cache", INPUT_TYPES, 4)
    dev, dt = k_cache.device, k_cache.dtype
    _require(v_cache, "v_cache", dt, 4, dev)
    _require(q, "q", dt, 3, dev)
    _require(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, dev)
    _require(block_tables, "block_tables", torch.int32, 2, dev)
    _require(context_lens, "context_lens", torch.int32, 1, dev)
    _require(out, "out", (torch.float32, dt), 3, dev)
    NB, bs, Hkv, D = k_cache.shape
    T, Hq, Dq = q.shape
    B = context_lens.shape[0]
    if v_cache.shape != k_cache.shape or Dq != D or out.shape != q.shape:
        raise ValueError("shape mismatch between q, out and the caches")
    if cu_seqlens_q.shape != (B + 1,) or block_tables.shape[0] != B:
        raise ValueError("cu_seqlens_q must be [B+1] and block_tables [B, MB]")
    if max_q_len is None:
        max_q_len = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if B else 0
    lib = load_library()
    MB = block_tables.shape[1]
    need = int(lib.paged_prefill_workspace_bytes(T, Hq, D, MB, bs, int(partition_tokens)))
    if workspace is None:
        if need:
            workspace = _cached_workspace(dev, need)
    elif workspace.device != dev or workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor on the cache's device")
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel()) if workspace is not None \
        else (None, 0)
    with _device(dev):
        _check(lib.paged_prefill_attention_split(
            q.data_ptr(), cu_seqlens_q.data_ptr(), T, int(max_q_len), k_cache.data_ptr(),
            v_cache.data_ptr(), block_tables.data_ptr(), MB, context_lens.data_ptr(), B, Hq,
            Hkv, D, bs, NB, float(scale), DTYPES[dt], out.data_ptr(), DTYPES[out.dtype],
            int(row_blocks), ws_ptr, ws_bytes, int(partition_tokens), _stream_handle(dev)))
    return out


def paged_kv_write_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        positions: torch.Tensor, inv_freq: torch.Tensor,
                        slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, *, q_out: Optional[torch.Tensor] = None,
                        interleaved: bool = False) -> torch.Tensor:
    """Rotate q and k of token t at positions[t] (pair i by positions[t] * inv_freq[i]), store
    the rotated k and the raw v at slot slot_mapping[t], return the rotated q (q_out, or a new
    tensor). q [T, Hq, D], k/v [T, Hkv, D] bf16; positions [T] int32; inv_freq [D/2] fp32."""
    _require(k_cache, "k_cache", torch.bfloat16, 4)
    dev = k_cache.device
    _require(v_cache, "v_cache", torch.bfloat16, 4, dev)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, torch.bfloat16, 3, dev)
    _require(positions, "positions", torch.int32, 1, dev)
    _require(inv_freq, "inv_freq", torch.float32, 1, dev)
    _require(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    NB, bs, Hkv, D = k_cache.shape
    T, Hq, _ = q.shape
    if (k.shape != (T, Hkv, D) or v.shape != (T, Hkv, D) or q.shape[2] != D or
            positions.shape != (T,) or slot_mapping.shape != (T,) or inv_freq.shape != (D // 2,)
            or v_cache.shape != k_cache.shape):
        raise ValueError("shape mismatch in paged_kv_write_rope arguments")
    if q_out is None:
        q_out = torch.empty_like(q)
    _require(q_out, "q_out", torch.bfloat16, 3, dev)
    if q_out.shape != q.shape:
        raise ValueError("q_out must have q's shape")
    lib = load_library()
    with _device(dev):
        _check(lib.paged_kv_write_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       positions.data_ptr(), inv_freq.data_ptr(),
                                       int(bool(interleaved)), slot_mapping.data_ptr(), T,
                                       q_out.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       NB, bs, Hq, Hkv, D, _stream_handle(dev)))
    return q_out
