"""ctypes binding of libpa_decode.so: argument marshalling only.

Every step of the decode path runs in the HIP library; this module checks
tensor dtypes, shapes, devices and contiguity, passes raw device pointers and
torch's current HIP stream, and turns a non-zero status into an exception.
PyTorch provides the device memory and the stream, nothing else.  If the
library is missing the functions raise: there is no other implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

_lock = threading.Lock()
_lib = None

PA_OUT_F32, PA_OUT_BF16 = 0, 1
HQ, HKV, D, PAGE = 32, 8, 64, 16

# names declared in include/pa_decode.h, include/pa_decode_q8.h, include/pa_decode_q4.h,
# include/pa_measure.h and include/pa_kvpool.h
EXPORTS = ("pa_append_kv", "pa_decode_workspace_bytes", "pa_decode_plan", "pa_decode_plan_lengths",
           "pa_decode_attention", "pa_append_decode_attention", "pa_decode_attention_profiled",
           "pa_append_kv_rope", "pa_append_decode_attention_rope", "pa_fill_kv",
           "pa_validate_metadata", "pa_status_string", "pa_abi_version",
           "pa_decode_worklist", "pa_append_decode_attention_worklist",
           "pa_append_decode_attention_noalloc",
           # include/pa_decode_balanced.h
           "pa_balance_plan", "pa_decode_balanced",
           # include/pa_decode_q8.h
           "pa_append_kv_q8", "pa_append_kv_rope_q8", "pa_fill_kv_q8", "pa_decode_attention_q8",
           "pa_append_decode_attention_q8", "pa_append_decode_attention_rope_q8",
           "pa_decode_plan_lengths_q8", "pa_append_decode_attention_worklist_q8",
           # include/pa_decode_q4.h
           "pa_append_kv_q4", "pa_append_kv_rope_q4", "pa_fill_kv_q4", "pa_decode_attention_q4",
           "pa_append_decode_attention_q4", "pa_append_decode_attention_rope_q4",
           "pa_decode_plan_lengths_q4", "pa_append_decode_attention_worklist_q4",
           # include/pa_measure.h
           "pa_stream_read", "pa_page_stream", "pa_decode_balanced_timeline",
           "pa_wall_clock_khz",
           # include/pa_kvpool.h
           "pa_kvpool_create", "pa_kvpool_destroy", "pa_kvpool_credit", "pa_kvpool_submit",
           "pa_kvpool_admit", "pa_kvpool_grow", "pa_kvpool_step", "pa_kvpool_finish",
           "pa_kvpool_block_table", "pa_kvpool_request_info", "pa_kvpool_get_stats")


class PaShape(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32)]


class KVPoolStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("pool_pages", "peak_active", "max_batch",
                                              "peak_allocated", "admission_waits", "free_pages")]


class PaRope(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("positions", ctypes.c_int32)]


def make_shape(num_pages: int, max_blocks: int, num_q_heads: int = HQ,
               num_kv_heads: int = HKV, head_dim: int = D, page_size: int = PAGE) -> PaShape:
    return PaShape(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, max_blocks)


def load_library(path: str | None = None):
    """Open the built library (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        path = path or _build.LIB
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library not built: {path} is missing "
                "(run `python -m paged_kv_decode_07_amd.build`)")
        lib = ctypes.CDLL(path)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        SP = ctypes.POINTER(PaShape)
        lib.pa_append_kv.argtypes = [SP, I32, P, P, P, P, P, P, P]
        lib.pa_decode_workspace_bytes.argtypes = [SP, I32, I32, I32, ctypes.POINTER(SZ)]
        lib.pa_decode_plan.argtypes = [SP, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]
        lib.pa_decode_plan_lengths.argtypes = [SP, I32, P, I32, I32, ctypes.POINTER(I32),
                                               ctypes.POINTER(I32)]
        lib.pa_decode_attention.argtypes = [SP, I32, P, P, P, P, P, I32, ctypes.c_float,
                                            P, I32, I32, P, SZ, P]
        lib.pa_decode_attention_profiled.argtypes = [SP, I32, P, P, P, P, P, P, P, I32,
                                                     ctypes.c_float, P, I32, I32, P, SZ, P, P, P]
        lib.pa_append_decode_attention.argtypes = [SP, I32, P, P, P, P, P, P, P, I32,
                                                   ctypes.c_float, P, I32, I32, P, SZ, P]
        lib.pa_append_decode_attention_noalloc.argtypes = [SP, I32, P, P, P, P, P, P, P, I32,
                                                           ctypes.c_float, P, I32, I32, P]
        RP = ctypes.POINTER(PaRope)
        lib.pa_append_kv_rope.argtypes = [SP, I32, P, P, P, RP, P, P, P, P, P, P]
        lib.pa_append_decode_attention_rope.argtypes = [SP, I32, P, P, P, RP, P, P, P, P, I32,
                                                        ctypes.c_float, P, I32, I32, P, SZ, P]
        lib.pa_fill_kv.argtypes = [SP, P, P, I32, I32, P, P, P, P]
        for sfx in ("_q8", "_q4"):
            getattr(lib, "pa_append_kv" + sfx).argtypes = [SP, I32, P, P, P, P, P, P, P, P]
            getattr(lib, "pa_append_kv_rope" + sfx).argtypes = [SP, I32, P, P, P, RP, P, P, P, P,
                                                                P, P, P]
            getattr(lib, "pa_fill_kv" + sfx).argtypes = [SP, P, P, I32, I32, P, P, P, P, P]
            getattr(lib, "pa_decode_attention" + sfx).argtypes = [
                SP, I32, P, P, P, P, P, P, I32, ctypes.c_float, P, I32, I32, P, SZ, P]
            getattr(lib, "pa_append_decode_attention" + sfx).argtypes = [
                SP, I32, P, P, P, P, P, P, P, P, I32, ctypes.c_float, P, I32, I32, P, SZ, P]
            getattr(lib, "pa_append_decode_attention_rope" + sfx).argtypes = [
                SP, I32, P, P, P, RP, P, P, P, P, P, I32, ctypes.c_float, P, I32, I32, P, SZ, P]
            getattr(lib, "pa_decode_plan_lengths" + sfx).argtypes = [
                SP, I32, P, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]
            getattr(lib, "pa_append_decode_attention_worklist" + sfx).argtypes = [
                SP, I32, P, P, P, P, P, P, P, P, I32, ctypes.c_float, P, I32, I32, P, I32, P, SZ,
                P]
        I64_ = ctypes.c_int64
        lib.pa_balance_plan.argtypes = [SP, I32, P, I32, I32, I32, P, I64_,
                                        ctypes.POINTER(I64_), ctypes.POINTER(I32)]
        lib.pa_decode_balanced.argtypes = [SP, I32, P, P, P, RP, P, P, P, I32, P, P, I32,
                                           ctypes.c_float, P, I32, P, I64_, I32, P]
        lib.pa_stream_read.argtypes = [P, SZ, P, I32, P]
        lib.pa_page_stream.argtypes = [SP, I32, P, P, P, I32, P, P, I32, I32, P, P]
        lib.pa_decode_balanced_timeline.argtypes = [SP, I32, P, P, P, P, P, P, I32, P, P, I32,
                                                    ctypes.c_float, P, P, I64_, I32, P, I64_, P]
        lib.pa_wall_clock_khz.argtypes = [ctypes.POINTER(I32)]
        lib.pa_decode_worklist.argtypes = [SP, I32, P, I32, I32, I32, I32, P, I32,
                                           ctypes.POINTER(I32), ctypes.POINTER(I32),
                                           ctypes.POINTER(I32)]
        lib.pa_append_decode_attention_worklist.argtypes = [SP, I32, P, P, P, P, P, P, P, I32,
                                                            ctypes.c_float, P, I32, I32, P, I32,
                                                            P, SZ, P]
        I64 = ctypes.c_int64
        PP = ctypes.POINTER(ctypes.c_void_p)
        lib.pa_kvpool_create.argtypes = [I32, I32, I32, I32, I32, PP]
        lib.pa_kvpool_destroy.argtypes = [P]
        lib.pa_kvpool_credit.argtypes = [P, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I64)]
        lib.pa_kvpool_submit.argtypes = [P, I64, I32, I32, ctypes.POINTER(I32)]
        lib.pa_kvpool_admit.argtypes = [P, ctypes.POINTER(I64), I32, ctypes.POINTER(I32)]
        lib.pa_kvpool_grow.argtypes = [P, I64, I32]
        lib.pa_kvpool_step.argtypes = [P]
        lib.pa_kvpool_finish.argtypes = [P, I64]
        lib.pa_kvpool_block_table.argtypes = [P, I64, I32, ctypes.POINTER(I32), I32,
                                              ctypes.POINTER(I32)]
        lib.pa_kvpool_request_info.argtypes = [P, I64, ctypes.POINTER(I32), ctypes.POINTER(I32),
                                               ctypes.POINTER(I32), ctypes.POINTER(I32)]
        lib.pa_kvpool_get_stats.argtypes = [P, ctypes.POINTER(KVPoolStats)]
        lib.pa_validate_metadata.argtypes = [SP, I32, P, P, I32, P, ctypes.POINTER(ctypes.c_int64)]
        lib.pa_status_string.argtypes = [ctypes.c_int]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_abi_version.argtypes = []
        for name in EXPORTS:
            if name != "pa_status_string":
                getattr(lib, name).restype = ctypes.c_int
        if path == _build.LIB:
            _lib = lib
        return lib


def status_string(rc: int) -> str:
    return load_library().pa_status_string(int(rc)).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what}: {status_string(rc)} (status {rc})")


def _stream_ptr(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _event_handles(*events):
    """HIP event handles of torch.cuda.Event objects (None passes NULL).

    A torch event owns a HIP event only once it has been recorded.
    """
    handles = []
    for ev in events:
        h = ev.cuda_event if ev is not None else 0
        if ev is not None and not h:
            raise ValueError("record each timing event once before passing it")
        handles.append(ctypes.c_void_p(h or None))
    return handles


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _is_device(t: torch.Tensor) -> bool:
    """Whether ``t`` lives in device memory (the library takes device pointers only)."""
    return t.is_cuda


def _bits16(t: torch.Tensor, name: str, shape_tail) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: expected bfloat16 (or its 16-bit patterns), got {t.dtype}")
    if not _is_device(t):
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if tuple(t.shape[-len(shape_tail):]) != tuple(shape_tail):
        raise ValueError(f"{name}: trailing shape {tuple(t.shape)} != {tuple(shape_tail)}")
    return t


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not _is_device(t) or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous int32 device tensor")
    return t


def _same_batch(B: int, **tensors) -> None:
    """Every given tensor's first dimension is the batch."""
    for name, t in tensors.items():
        if t is not None and (t.dim() < 1 or int(t.shape[0]) != B):
            raise ValueError(f"batch dimension mismatch: {name} has {tuple(t.shape)}, batch {B}")


def _out_code(out_dtype) -> int:
    code = {torch.float32: PA_OUT_F32, torch.bfloat16: PA_OUT_BF16}.get(out_dtype)
    if code is None:
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    return code


def _out(out, B: int, out_dtype, device) -> torch.Tensor:
    """The caller's output tensor, checked, or a new one: contiguous [B][32][64] of out_dtype."""
    if out is None:
        return torch.empty((B, HQ, D), dtype=out_dtype, device=device)
    if out.dtype != out_dtype or tuple(out.shape) != (B, HQ, D) or not out.is_contiguous() \
            or not _is_device(out):
        raise ValueError("out must be a contiguous [B][32][64] device tensor of out_dtype")
    return out


def _same_pools(k_pool, v_pool) -> None:
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")


def append_kv(k_new, v_new, k_pool, v_pool, block_tables, seq_lens, stream=None) -> None:
    """Write each sequence's new K/V row (``[B][8][64]``) into its page slot."""
    B = int(seq_lens.shape[0])
    _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, k_new=k_new, v_new=v_new, block_tables=block_tables)
    _same_pools(k_pool, v_pool)
    shape = make_shape(int(k_pool.shape[0]), int(block_tables.shape[1]))
    rc = load_library().pa_append_kv(ctypes.byref(shape), B, _ptr(k_new), _ptr(v_new),
                                     _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                     _ptr(seq_lens), _stream_ptr(stream))
    _check(rc, "pa_append_kv")


def decode_plan(batch: int, max_seq_len: int, num_pages: int, max_blocks: int = 128,
                pages_per_split: int = 0):
    """(pages per split, splits of the longest sequence) the library uses."""
    shape = make_shape(num_pages, max_blocks)
    ps, ns = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = load_library().pa_decode_plan(ctypes.byref(shape), batch, max_seq_len,
                                       pages_per_split, ctypes.byref(ps), ctypes.byref(ns))
    _check(rc, "pa_decode_plan")
    return ps.value, ns.value


def decode_plan_lengths(seq_lens_host, num_pages: int, max_blocks: int = 128,
                        max_seq_len: int | None = None, num_cus: int = 0):
    """Split plan for lengths known on the host: (pages per split, splits).

    ``num_cus`` 0 plans for the current device; a positive count plans
    without touching any device.
    """
    import numpy as np
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    msl = int(lens.max()) if max_seq_len is None and lens.size else int(max_seq_len or 0)
    shape = make_shape(num_pages, max_blocks)
    ps, ns = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = load_library().pa_decode_plan_lengths(ctypes.byref(shape), int(lens.size),
                                               lens.ctypes.data_as(ctypes.c_void_p), msl,
                                               int(num_cus), ctypes.byref(ps), ctypes.byref(ns))
    _check(rc, "pa_decode_plan_lengths")
    return ps.value, ns.value


def decode_workspace_bytes(batch: int, max_seq_len: int, num_pages: int,
                           max_blocks: int = 128, pages_per_split: int = 0) -> int:
    shape = make_shape(num_pages, max_blocks)
    n = ctypes.c_size_t(0)
    rc = load_library().pa_decode_workspace_bytes(ctypes.byref(shape), batch, max_seq_len,
                                                  pages_per_split, ctypes.byref(n))
    _check(rc, "pa_decode_workspace_bytes")
    return n.value


def decode_attention(q, k_pool, v_pool, block_tables, seq_lens, max_seq_len: int,
                     scale: float = 0.125, out=None, out_dtype=torch.float32,
                     pages_per_split: int = 0, workspace=None, stream=None,
                     event_before_main=None, event_after_main=None):
    """Paged GQA decode attention; returns ``out`` ``[B][32][64]``.

    ``workspace`` may be passed (a uint8 device tensor of at least
    ``decode_workspace_bytes(...)`` bytes) to keep the call free of torch
    allocations; otherwise one is allocated here when the plan needs it.
    """
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, block_tables=block_tables)
    _same_pools(k_pool, v_pool)
    code = _out_code(out_dtype)
    num_pages, max_blocks = int(k_pool.shape[0]), int(block_tables.shape[1])
    out = _out(out, B, out_dtype, q.device)
    need = decode_workspace_bytes(B, max_seq_len, num_pages, max_blocks, pages_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    shape = make_shape(num_pages, max_blocks)
    args = [ctypes.byref(shape), B, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
            _ptr(seq_lens), int(max_seq_len), float(scale), _ptr(out), code,
            int(pages_per_split), _ptr(workspace), ws_bytes, _stream_ptr(stream)]
    lib = load_library()
    if event_before_main is None and event_after_main is None:
        rc = lib.pa_decode_attention(*args)
    else:
        rc = lib.pa_decode_attention_profiled(*args[:3], None, None, *args[3:],
                                              *_event_handles(event_before_main,
                                                              event_after_main))
    _check(rc, "pa_decode_attention")
    return out


def append_decode_attention(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens,
                            max_seq_len: int, scale: float = 0.125, out=None,
                            out_dtype=torch.float32, pages_per_split: int = 0, workspace=None,
                            stream=None, event_before_main=None, event_after_main=None):
    """One decode step in one launch: append each sequence's new K/V row, then attend.

    Same result as ``append_kv`` followed by ``decode_attention``; returns ``out``.
    """
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, k_new=k_new, v_new=v_new, block_tables=block_tables)
    _same_pools(k_pool, v_pool)
    code = _out_code(out_dtype)
    num_pages, max_blocks = int(k_pool.shape[0]), int(block_tables.shape[1])
    out = _out(out, B, out_dtype, q.device)
    need = decode_workspace_bytes(B, max_seq_len, num_pages, max_blocks, pages_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    shape = make_shape(num_pages, max_blocks)
    args = [ctypes.byref(shape), B, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
            _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens), int(max_seq_len), float(scale),
            _ptr(out), code, int(pages_per_split), _ptr(workspace), ws_bytes,
            _stream_ptr(stream)]
    lib = load_library()
    if event_before_main is None and event_after_main is None:
        rc = lib.pa_append_decode_attention(*args)
    else:
        rc = lib.pa_decode_attention_profiled(*args, *_event_handles(event_before_main,
                                                                      event_after_main))
    _check(rc, "pa_append_decode_attention")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20      # PA_NOALLOC_SCRATCH_BYTES of include/pa_decode.h


def append_decode_attention_noalloc(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens,
                                    max_seq_len: int, out, scale: float = 0.125,
                                    out_dtype=torch.float32, pages_per_split: int = 0,
                                    stream=None):
    """The fused step of ``append_decode_attention`` with the split partials in the
    library's own device scratch: the call allocates nothing, so ``out`` must be
    given.  Calls that overlap in time on one GPU share that scratch and race."""
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, k_new=k_new, v_new=v_new, block_tables=block_tables)
    _same_pools(k_pool, v_pool)
    code = _out_code(out_dtype)
    if out is None:
        raise ValueError("out is required: this call allocates nothing")
    out = _out(out, B, out_dtype, q.device)
    shape = make_shape(int(k_pool.shape[0]), int(block_tables.shape[1]))
    rc = load_library().pa_append_decode_attention_noalloc(
        ctypes.byref(shape), B, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), _ptr(seq_lens), int(max_seq_len), float(scale), _ptr(out), code,
        int(pages_per_split), _stream_ptr(stream))
    _check(rc, "pa_append_decode_attention_noalloc")
    return out


def _rope(cos, sin) -> PaRope:
    for name, t in (("rope_cos", cos), ("rope_sin", sin)):
        if t.dtype != torch.float32 or not _is_device(t) or not t.is_contiguous() or t.dim() != 2 \
                or t.shape[1] != D // 2:
            raise ValueError(f"{name}: must be a contiguous float32 [positions][32] device tensor")
    if cos.shape != sin.shape:
        raise ValueError("rope_cos and rope_sin differ in shape")
    return PaRope(cos.data_ptr(), sin.data_ptr(), int(cos.shape[0]))


def append_kv_rope(q, k_new, v_new, rope_cos, rope_sin, k_pool, v_pool, block_tables,
                   seq_lens, q_out=None, stream=None):
    """Rotate the new q/k at position L-1 (RoPE), append K/V; returns ``q_out``."""
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, k_new=k_new, v_new=v_new, block_tables=block_tables)
    _same_pools(k_pool, v_pool)
    if q_out is None:
        q_out = torch.empty_like(q)
    _bits16(q_out, "q_out", (HQ, D))
    _same_batch(B, q_out=q_out)
    rope = _rope(rope_cos, rope_sin)
    shape = make_shape(int(k_pool.shape[0]), int(block_tables.shape[1]))
    rc = load_library().pa_append_kv_rope(
        ctypes.byref(shape), B, _ptr(q), _ptr(k_new), _ptr(v_new), ctypes.byref(rope),
        _ptr(q_out), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens),
        _stream_ptr(stream))
    _check(rc, "pa_append_kv_rope")
    return q_out


def append_decode_attention_rope(q, k_new, v_new, rope_cos, rope_sin, k_pool, v_pool,
                                 block_tables, seq_lens, max_seq_len: int, scale: float = 0.125,
                                 out=None, out_dtype=torch.float32, pages_per_split: int = 0,
                                 workspace=None, stream=None):
    """Fused step with RoPE: rotate q/k at L-1, append, attend; returns ``out``."""
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, k_new=k_new, v_new=v_new, block_tables=block_tables)
    _same_pools(k_pool, v_pool)
    code = _out_code(out_dtype)
    num_pages, max_blocks = int(k_pool.shape[0]), int(block_tables.shape[1])
    out = _out(out, B, out_dtype, q.device)
    need = decode_workspace_bytes(B, max_seq_len, num_pages, max_blocks, pages_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rope = _rope(rope_cos, rope_sin)
    shape = make_shape(num_pages, max_blocks)
    rc = load_library().pa_append_decode_attention_rope(
        ctypes.byref(shape), B, _ptr(q), _ptr(k_new), _ptr(v_new), ctypes.byref(rope),
        _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens), int(max_seq_len),
        float(scale), _ptr(out), code, int(pages_per_split), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    _check(rc, "pa_append_decode_attention_rope")
    return out


def fill_kv(k_rows, v_rows, block_table_row, start: int, k_pool, v_pool, stream=None) -> None:
    """Prefill page fill: tokens ``start .. start+T-1`` of one sequence into its pages."""
    _bits16(k_rows, "k_rows", (HKV, D)); _bits16(v_rows, "v_rows", (HKV, D))
    _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
    _i32(block_table_row, "block_table_row")
    if k_rows.shape != v_rows.shape:
        raise ValueError("k_rows and v_rows differ in shape")
    _same_pools(k_pool, v_pool)
    shape = make_shape(int(k_pool.shape[0]), int(block_table_row.shape[-1]))
    rc = load_library().pa_fill_kv(ctypes.byref(shape), _ptr(k_rows), _ptr(v_rows),
                                   int(k_rows.shape[0]), int(start), _ptr(block_table_row),
                                   _ptr(k_pool), _ptr(v_pool), _stream_ptr(stream))
    _check(rc, "pa_fill_kv")


# ---------------------------------------------------------------------------
# INT8 and INT4 K/V pages (include/pa_decode_q8.h, include/pa_decode_q4.h).
# The INT4 functions take the same arguments as their INT8 namesakes.
# ---------------------------------------------------------------------------
_SUFFIX = {8: "_q8", 4: "_q4"}


def new_q8_pools(num_pages: int, device="cuda"):
    """Zeroed INT8 pools: K codes, V codes (int8 ``[pages][8][16][64]``, head-major
    within a page) and scales (float32 ``[pages][8][2][16]``)."""
    codes = (num_pages, HKV, PAGE, D)
    return (torch.zeros(codes, dtype=torch.int8, device=device),
            torch.zeros(codes, dtype=torch.int8, device=device),
            torch.zeros((num_pages, HKV, 2, PAGE), dtype=torch.float32, device=device))


def new_q4_pools(num_pages: int, device="cuda"):
    """Zeroed INT4 pools: K codes, V codes (uint8 ``[pages][8][16][32]``, two codes
    per byte) and scales (float32 ``[pages][8][2][16]``)."""
    codes = (num_pages, HKV, PAGE, D // 2)
    return (torch.zeros(codes, dtype=torch.uint8, device=device),
            torch.zeros(codes, dtype=torch.uint8, device=device),
            torch.zeros((num_pages, HKV, 2, PAGE), dtype=torch.float32, device=device))


def _q8_pools(k_codes, v_codes, kv_scales, nbits: int = 8) -> int:
    dtype, width = (torch.int8, D) if nbits == 8 else (torch.uint8, D // 2)
    for name, t in (("k_codes", k_codes), ("v_codes", v_codes)):
        if t.dtype != dtype or not _is_device(t) or not t.is_contiguous() or \
                tuple(t.shape[1:]) != (HKV, PAGE, width):
            raise ValueError(f"{name}: must be a contiguous {str(dtype)[6:]} "
                             f"[pages][8][16][{width}] device tensor")
    if k_codes.shape != v_codes.shape:
        raise ValueError("k_codes and v_codes differ in shape")
    n = int(k_codes.shape[0])
    if kv_scales.dtype != torch.float32 or not _is_device(kv_scales) or \
            not kv_scales.is_contiguous() or tuple(kv_scales.shape) != (n, HKV, 2, PAGE):
        raise ValueError("kv_scales: must be a contiguous float32 [pages][8][2][16] device tensor")
    return n


def append_kv_q8(k_new, v_new, k_codes, v_codes, kv_scales, block_tables, seq_lens,
                 stream=None, nbits: int = 8) -> None:
    """Quantise each sequence's new K/V row (``[B][8][64]`` BF16) into its page slot."""
    B = int(seq_lens.shape[0])
    _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, k_new=k_new, v_new=v_new, block_tables=block_tables)
    shape = make_shape(_q8_pools(k_codes, v_codes, kv_scales, nbits), int(block_tables.shape[1]))
    fn = "pa_append_kv" + _SUFFIX[nbits]
    rc = getattr(load_library(), fn)(
        ctypes.byref(shape), B, _ptr(k_new), _ptr(v_new), _ptr(k_codes), _ptr(v_codes),
        _ptr(kv_scales), _ptr(block_tables), _ptr(seq_lens), _stream_ptr(stream))
    _check(rc, fn)


def append_kv_rope_q8(q, k_new, v_new, rope_cos, rope_sin, k_codes, v_codes, kv_scales,
                      block_tables, seq_lens, q_out=None, stream=None, nbits: int = 8):
    """Rotate the new q/k at position L-1, quantise K/V into the slot; returns ``q_out``."""
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, k_new=k_new, v_new=v_new, block_tables=block_tables)
    if q_out is None:
        q_out = torch.empty_like(q)
    _bits16(q_out, "q_out", (HQ, D))
    _same_batch(B, q_out=q_out)
    rope = _rope(rope_cos, rope_sin)
    shape = make_shape(_q8_pools(k_codes, v_codes, kv_scales, nbits), int(block_tables.shape[1]))
    fn = "pa_append_kv_rope" + _SUFFIX[nbits]
    rc = getattr(load_library(), fn)(
        ctypes.byref(shape), B, _ptr(q), _ptr(k_new), _ptr(v_new), ctypes.byref(rope),
        _ptr(q_out), _ptr(k_codes), _ptr(v_codes), _ptr(kv_scales), _ptr(block_tables),
        _ptr(seq_lens), _stream_ptr(stream))
    _check(rc, fn)
    return q_out


def fill_kv_q8(k_rows, v_rows, block_table_row, start: int, k_codes, v_codes, kv_scales,
               stream=None, nbits: int = 8) -> None:
    """Quantised prefill fill: tokens ``start .. start+T-1`` of one sequence."""
    _bits16(k_rows, "k_rows", (HKV, D)); _bits16(v_rows, "v_rows", (HKV, D))
    _i32(block_table_row, "block_table_row")
    if k_rows.shape != v_rows.shape:
        raise ValueError("k_rows and v_rows differ in shape")
    shape = make_shape(_q8_pools(k_codes, v_codes, kv_scales, nbits),
                       int(block_table_row.shape[-1]))
    fn = "pa_fill_kv" + _SUFFIX[nbits]
    rc = getattr(load_library(), fn)(ctypes.byref(shape), _ptr(k_rows), _ptr(v_rows),
                                     int(k_rows.shape[0]), int(start), _ptr(block_table_row),
                                     _ptr(k_codes), _ptr(v_codes), _ptr(kv_scales),
                                     _stream_ptr(stream))
    _check(rc, fn)


def decode_plan_lengths_q8(seq_lens_host, num_pages: int, max_blocks: int = 128,
                           max_seq_len: int | None = None, num_cus: int = 0, nbits: int = 8):
    """(pages_per_split, splits) for INT8 pages from host sequence lengths."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    if max_seq_len is None:
        max_seq_len = int(lens.max()) if lens.size else 0
    shape = make_shape(num_pages, max_blocks)
    ps, ns = ctypes.c_int32(), ctypes.c_int32()
    fn = "pa_decode_plan_lengths" + _SUFFIX[nbits]
    rc = getattr(load_library(), fn)(
        ctypes.byref(shape), int(lens.size), lens.ctypes.data_as(ctypes.c_void_p),
        int(max_seq_len), int(num_cus), ctypes.byref(ps), ctypes.byref(ns))
    _check(rc, fn)
    return ps.value, ns.value


def _decode_q8(fn, q, k_new, v_new, rope, k_codes, v_codes, kv_scales, block_tables, seq_lens,
               max_seq_len, scale, out, out_dtype, pages_per_split, workspace, stream, nbits=8):
    fn += _SUFFIX[nbits]
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    if k_new is not None:
        _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, k_new=k_new, v_new=v_new, block_tables=block_tables)
    num_pages = _q8_pools(k_codes, v_codes, kv_scales, nbits)
    code = _out_code(out_dtype)
    max_blocks = int(block_tables.shape[1])
    out = _out(out, B, out_dtype, q.device)
    need = decode_workspace_bytes(B, max_seq_len, num_pages, max_blocks, pages_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    shape = make_shape(num_pages, max_blocks)
    args = [ctypes.byref(shape), B, _ptr(q)]
    if k_new is not None:
        args += [_ptr(k_new), _ptr(v_new)]
    if rope is not None:
        args += [ctypes.byref(rope)]
    args += [_ptr(k_codes), _ptr(v_codes), _ptr(kv_scales), _ptr(block_tables), _ptr(seq_lens),
             int(max_seq_len), float(scale), _ptr(out), code, int(pages_per_split),
             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_ptr(stream)]
    _check(getattr(load_library(), fn)(*args), fn)
    return out


def decode_attention_q8(q, k_codes, v_codes, kv_scales, block_tables, seq_lens, max_seq_len: int,
                        scale: float = 0.125, out=None, out_dtype=torch.float32,
                        pages_per_split: int = 0, workspace=None, stream=None, nbits: int = 8):
    """Decode attention over INT8 (or ``nbits=4``: INT4) pages; returns ``out`` ``[B][32][64]``."""
    return _decode_q8("pa_decode_attention", q, None, None, None, k_codes, v_codes, kv_scales,
                      block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                      pages_per_split, workspace, stream, nbits)


def append_decode_attention_q8(q, k_new, v_new, k_codes, v_codes, kv_scales, block_tables,
                               seq_lens, max_seq_len: int, scale: float = 0.125, out=None,
                               out_dtype=torch.float32, pages_per_split: int = 0,
                               workspace=None, stream=None, rope_cos=None, rope_sin=None,
                               nbits: int = 8):
    """Fused quantised decode step (optionally with RoPE of the new q/k); returns ``out``."""
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("give both rope_cos and rope_sin, or neither")
    if rope_cos is None:
        return _decode_q8("pa_append_decode_attention", q, k_new, v_new, None, k_codes,
                          v_codes, kv_scales, block_tables, seq_lens, max_seq_len, scale, out,
                          out_dtype, pages_per_split, workspace, stream, nbits)
    return _decode_q8("pa_append_decode_attention_rope", q, k_new, v_new,
                      _rope(rope_cos, rope_sin), k_codes, v_codes, kv_scales, block_tables,
                      seq_lens, max_seq_len, scale, out, out_dtype, pages_per_split, workspace,
                      stream, nbits)


def append_kv_q4(*args, **kw) -> None:
    """INT4 pages: ``append_kv_q8`` with ``[pages][8][16][32]`` uint8 code pools."""
    return append_kv_q8(*args, nbits=4, **kw)


def append_kv_rope_q4(*args, **kw):
    """INT4 pages: ``append_kv_rope_q8`` with INT4 code pools."""
    return append_kv_rope_q8(*args, nbits=4, **kw)


def fill_kv_q4(*args, **kw) -> None:
    """INT4 pages: ``fill_kv_q8`` with INT4 code pools."""
    return fill_kv_q8(*args, nbits=4, **kw)


def decode_plan_lengths_q4(*args, **kw):
    """INT4 pages: ``decode_plan_lengths_q8`` with the INT4 cost model."""
    return decode_plan_lengths_q8(*args, nbits=4, **kw)


def decode_attention_q4(*args, **kw):
    """INT4 pages: ``decode_attention_q8`` with INT4 code pools."""
    return decode_attention_q8(*args, nbits=4, **kw)


def append_decode_attention_q4(*args, **kw):
    """INT4 pages: ``append_decode_attention_q8`` with INT4 code pools."""
    return append_decode_attention_q8(*args, nbits=4, **kw)


def decode_worklist(seq_lens_host, num_pages: int, max_blocks: int = 128,
                    max_seq_len: int | None = None, pages_per_split: int = 0,
                    int8: bool = False, num_cus: int = 0, int4: bool = False):
    """Longest-first work list for host lengths: (work int32 [n][2], pages_per_split, splits).
    ``int8`` / ``int4`` pick the planner's cost model for those page formats."""
    if int8 and int4:
        raise ValueError("int8 and int4 are exclusive")
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    if max_seq_len is None:
        max_seq_len = int(lens.max()) if lens.size else 0
    shape = make_shape(num_pages, max_blocks)
    cap = max(1, int(lens.size) * max(1, -(-max_seq_len // PAGE)))
    work = np.zeros((cap, 2), dtype=np.int32)
    count, ps, ns = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = load_library().pa_decode_worklist(
        ctypes.byref(shape), int(lens.size), lens.ctypes.data_as(ctypes.c_void_p),
        int(max_seq_len), int(pages_per_split), 2 if int4 else (1 if int8 else 0), int(num_cus),
        work.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(count), ctypes.byref(ps),
        ctypes.byref(ns))
    _check(rc, "pa_decode_worklist")
    return work[:count.value].copy(), ps.value, ns.value


def append_decode_attention_worklist(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens,
                                     max_seq_len: int, work, pages_per_split: int,
                                     scale: float = 0.125, out=None, out_dtype=torch.float32,
                                     workspace=None, stream=None, kv_scales=None):
    """Decode step over a device work list (``decode_worklist``); k_new/v_new may be None
    (decode only).  With ``kv_scales`` the pools are INT8 (int8) or INT4 (uint8) code pools."""
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, k_new=k_new, v_new=v_new, block_tables=block_tables)
    _i32(work, "work")
    if work.dim() != 2 or work.shape[1] != 2 or work.shape[0] < 1:
        raise ValueError("work: int32 [n][2] device tensor with n >= 1")
    q8 = kv_scales is not None
    nbits = 4 if q8 and k_pool.dtype == torch.uint8 else 8
    num_pages = _q8_pools(k_pool, v_pool, kv_scales, nbits) if q8 else int(k_pool.shape[0])
    if not q8:
        _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
        _same_pools(k_pool, v_pool)
    code = _out_code(out_dtype)
    max_blocks = int(block_tables.shape[1])
    out = _out(out, B, out_dtype, q.device)
    need = decode_workspace_bytes(B, max_seq_len, num_pages, max_blocks, pages_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    shape = make_shape(num_pages, max_blocks)
    nk = _ptr(k_new) if k_new is not None else None
    nv = _ptr(v_new) if v_new is not None else None
    pools = [_ptr(k_pool), _ptr(v_pool)] + ([_ptr(kv_scales)] if q8 else [])
    fn = "pa_append_decode_attention_worklist" + (_SUFFIX[nbits] if q8 else "")
    rc = getattr(load_library(), fn)(
        ctypes.byref(shape), B, _ptr(q), nk, nv, *pools, _ptr(block_tables), _ptr(seq_lens),
        int(max_seq_len), float(scale), _ptr(out), code, int(pages_per_split), _ptr(work),
        int(work.shape[0]), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream))
    _check(rc, fn)
    return out


# int32 words of a balanced plan's header and of one wavefront's descriptor
# (include/pa_decode_balanced.h)
BAL_HEADER, BAL_DESC = 64, 64


class BalancedPlan:
    """A plan of ``pa_balance_plan`` on the device: ``plan`` (int32 device tensor),
    ``groups`` (work-groups to launch) and the host lengths it was built for."""

    def __init__(self, plan, groups: int, seq_lens_host):
        self.plan, self.groups, self.seq_lens_host = plan, int(groups), seq_lens_host

    @property
    def words(self) -> int:
        return int(self.plan.numel())


# Pinned host buffers that plans are built in and uploaded from, per device:
# idle [buffer, event recorded after its last upload] pairs.  A caller takes a
# buffer out while it plans into it and queues its upload, and gives it back
# with the event recorded; a buffer is written again only once that event has
# completed, so an upload never waits for the work queued before it.
_STAGING_SLOTS = 4
_staging: dict = {}


def _staging_take(device: torch.device, words: int):
    with _lock:
        pool = _staging.setdefault(str(device), [])
        for i, slot in enumerate(pool):
            if slot[0].numel() >= words and slot[1].query():
                return pool.pop(i)
        if len(pool) < _STAGING_SLOTS:
            return [torch.empty(words, dtype=torch.int32, pin_memory=True), torch.cuda.Event()]
        slot = pool.pop(0)                     # the least recently given back
    slot[1].synchronize()
    if slot[0].numel() < words:
        slot[0] = torch.empty(words, dtype=torch.int32, pin_memory=True)
    return slot


def _staging_give(device: torch.device, slot) -> None:
    with _lock:
        _staging.setdefault(str(device), []).append(slot)


def balance_plan(seq_lens_host, num_pages: int, max_blocks: int = 128,
                 max_seq_len: int | None = None, num_cus: int = 0, heads_together: int = 8,
                 device="cuda", host_only: bool = False, stream=None):
    """Plan of the balanced launch for host lengths (``include/pa_decode_balanced.h``).

    Returns a ``BalancedPlan`` whose plan is uploaded to ``device`` on ``stream``
    (default: the device's current stream) without waiting for the work queued
    there: the plan is built in a pinned buffer and copied asynchronously, so a
    serving loop can plan its next step while the GPU runs this one.  With
    ``host_only``: the host int32 array and the work-group count."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    if max_seq_len is None:
        max_seq_len = int(lens.max()) if lens.size else 0
    shape = make_shape(num_pages, max_blocks)
    lib = load_library()
    words, groups = ctypes.c_int64(), ctypes.c_int32()
    args = (ctypes.byref(shape), int(lens.size), lens.ctypes.data_as(ctypes.c_void_p),
            int(max_seq_len), int(num_cus), int(heads_together))
    # one call into room for as many work-groups as compute units (the usual
    # plan; the library writes every word of it), a second when it needs more
    guess = BAL_HEADER + max(int(num_cus) if num_cus > 0 else 256, 1) * 8 * BAL_DESC
    if host_only:
        host = np.empty(guess, dtype=np.int32)
        rc = lib.pa_balance_plan(*args, host.ctypes.data_as(ctypes.c_void_p), host.size,
                                 ctypes.byref(words), ctypes.byref(groups))
        if rc != 0 and words.value > host.size:
            host = np.empty(words.value, dtype=np.int32)
            rc = lib.pa_balance_plan(*args, host.ctypes.data_as(ctypes.c_void_p), host.size,
                                     ctypes.byref(words), ctypes.byref(groups))
        _check(rc, "pa_balance_plan")
        return host[:words.value], groups.value
    device = torch.device(device)
    if device.type == "cuda" and device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    slot = _staging_take(device, guess)
    try:
        rc = lib.pa_balance_plan(*args, ctypes.c_void_p(slot[0].data_ptr()), slot[0].numel(),
                                 ctypes.byref(words), ctypes.byref(groups))
        if rc != 0 and words.value > slot[0].numel():
            _staging_give(device, slot)
            slot = _staging_take(device, words.value)
            rc = lib.pa_balance_plan(*args, ctypes.c_void_p(slot[0].data_ptr()),
                                     slot[0].numel(), ctypes.byref(words), ctypes.byref(groups))
        _check(rc, "pa_balance_plan")
        st = stream if stream is not None else torch.cuda.current_stream(device)
        with torch.cuda.stream(st):
            plan = torch.empty(words.value, dtype=torch.int32, device=device)
            plan.copy_(slot[0][:words.value], non_blocking=True)
            slot[1].record(st)
    finally:
        _staging_give(device, slot)
    return BalancedPlan(plan, groups.value, lens)


def _balanced_checks(q, k_pool, v_pool, block_tables, seq_lens, plan, k_new, v_new, kv_scales):
    """Argument checks of the balanced launches: (batch, page format, shape)."""
    B = int(seq_lens.shape[0])
    _bits16(q, "q", (HQ, D))
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _bits16(k_new, "k_new", (HKV, D)); _bits16(v_new, "v_new", (HKV, D))
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, q=q, k_new=k_new, v_new=v_new, block_tables=block_tables)
    if not isinstance(plan, BalancedPlan):
        raise TypeError("plan must come from balance_plan")
    _i32(plan.plan, "plan")
    if plan.seq_lens_host is not None and len(plan.seq_lens_host) != B:
        raise ValueError("the plan was built for another batch")
    fmt = 0
    if kv_scales is not None:
        fmt = 2 if k_pool.dtype == torch.uint8 else 1
        num_pages = _q8_pools(k_pool, v_pool, kv_scales, 4 if fmt == 2 else 8)
    else:
        _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
        _same_pools(k_pool, v_pool)
        num_pages = int(k_pool.shape[0])
    return B, fmt, make_shape(num_pages, int(block_tables.shape[1]))


def decode_balanced(q, k_pool, v_pool, block_tables, seq_lens, max_seq_len: int, plan,
                    k_new=None, v_new=None, kv_scales=None, scale: float = 0.125, out=None,
                    out_dtype=torch.float32, rope_cos=None, rope_sin=None, stream=None):
    """Decode step over a ``BalancedPlan`` (optionally with the fused append and RoPE).

    BF16 pools as ``decode_attention``; with ``kv_scales`` the pools are INT8
    (int8) or INT4 (uint8) code pools.  Returns ``out``; no workspace."""
    B, fmt, shape = _balanced_checks(q, k_pool, v_pool, block_tables, seq_lens, plan, k_new,
                                     v_new, kv_scales)
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("give both rope_cos and rope_sin, or neither")
    rope = _rope(rope_cos, rope_sin) if rope_cos is not None else None
    code = _out_code(out_dtype)
    out = _out(out, B, out_dtype, q.device)
    rc = load_library().pa_decode_balanced(
        ctypes.byref(shape), B, _ptr(q), _ptr(k_new) if k_new is not None else None,
        _ptr(v_new) if v_new is not None else None,
        ctypes.byref(rope) if rope is not None else None, _ptr(k_pool), _ptr(v_pool),
        _ptr(kv_scales) if kv_scales is not None else None, fmt, _ptr(block_tables),
        _ptr(seq_lens), int(max_seq_len), float(scale), _ptr(out), code, _ptr(plan.plan),
        plan.words, plan.groups, _stream_ptr(stream))
    _check(rc, "pa_decode_balanced")
    return out


# words per wavefront of the timeline launch (include/pa_measure.h)
STAMP_WORDS = 8


def decode_balanced_timeline(q, k_pool, v_pool, block_tables, seq_lens, max_seq_len: int, plan,
                             k_new=None, v_new=None, kv_scales=None, scale: float = 0.125,
                             out=None, stamps=None, stream=None):
    """``decode_balanced`` (FP32 output, no RoPE) that also records each
    wavefront's real-time counter at seven points of its work
    (``include/pa_measure.h``).  Returns ``(out, stamps)``; ``stamps`` is int64
    ``[groups][8][8]`` (words 0..6 counter ticks, word 7 hardware ids and the
    wavefront's page count)."""
    B, fmt, shape = _balanced_checks(q, k_pool, v_pool, block_tables, seq_lens, plan, k_new,
                                     v_new, kv_scales)
    out = _out(out, B, torch.float32, q.device)
    words = plan.groups * 8 * STAMP_WORDS
    if stamps is None:
        stamps = torch.zeros((plan.groups, 8, STAMP_WORDS), dtype=torch.int64, device=q.device)
    elif stamps.dtype != torch.int64 or not _is_device(stamps) or not stamps.is_contiguous() or \
            stamps.numel() < words:
        raise ValueError("decode_balanced_timeline: stamps must be a contiguous int64 device "
                         "tensor of groups x 8 x 8 words")
    rc = load_library().pa_decode_balanced_timeline(
        ctypes.byref(shape), B, _ptr(q), _ptr(k_new) if k_new is not None else None,
        _ptr(v_new) if v_new is not None else None, _ptr(k_pool), _ptr(v_pool),
        _ptr(kv_scales) if kv_scales is not None else None, fmt, _ptr(block_tables),
        _ptr(seq_lens), int(max_seq_len), float(scale), _ptr(out), _ptr(plan.plan), plan.words,
        plan.groups, _ptr(stamps), int(stamps.numel()), _stream_ptr(stream))
    _check(rc, "pa_decode_balanced_timeline")
    return out, stamps


def wall_clock_khz() -> int:
    """Rate of the counter ``decode_balanced_timeline`` reads, in kHz."""
    khz = ctypes.c_int32(0)
    _check(load_library().pa_wall_clock_khz(ctypes.byref(khz)), "pa_wall_clock_khz")
    return int(khz.value)


def stream_read(buf, sink, groups: int = 0, stream=None) -> None:
    """Read every byte of ``buf`` once (``include/pa_measure.h``); ``sink`` holds a
    uint32 word per work-group."""
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda or sink.dtype != torch.int32:
        raise ValueError("stream_read: contiguous device buffer and int32 device sink required")
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < (groups if groups > 0 else 65536):
        raise ValueError("stream_read: sink smaller than the number of work-groups")
    _check(load_library().pa_stream_read(_ptr(buf), nbytes, _ptr(sink), int(groups),
                                         _stream_ptr(stream)), "pa_stream_read")


def page_stream(k_pool, v_pool, kv_scales, block_tables, seq_lens, waves_per_head: int = 1,
                ring: int = 2, sink=None, stream=None) -> torch.Tensor:
    """The decode kernels' page reads without their arithmetic (``include/pa_measure.h``).

    The page format follows the pools: BF16 ``[pages][16][8][64]`` (``kv_scales``
    None), INT8 ``[pages][8][16][64]`` or INT4 ``[pages][8][16][32]`` codes with
    their scales.  Returns ``sink``: int32 ``[B][8 * waves_per_head]``, the XOR of
    every word each wavefront read."""
    B = int(seq_lens.shape[0])
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    _same_batch(B, block_tables=block_tables)
    if kv_scales is None:
        _bits16(k_pool, "k_pool", (PAGE, HKV, D)); _bits16(v_pool, "v_pool", (PAGE, HKV, D))
        _same_pools(k_pool, v_pool)
        num_pages, fmt = int(k_pool.shape[0]), 0
    else:
        nbits = 8 if k_pool.dtype == torch.int8 else 4     # _q8_pools refuses anything else
        num_pages, fmt = _q8_pools(k_pool, v_pool, kv_scales, nbits), 1 if nbits == 8 else 2
    if waves_per_head not in (1, 2) or ring not in (1, 2, 3):
        raise ValueError("page_stream: waves_per_head must be 1 or 2 and ring 1, 2 or 3")
    words = B * HKV * waves_per_head
    if sink is None:
        sink = torch.empty((B, HKV * waves_per_head), dtype=torch.int32, device=seq_lens.device)
    elif sink.dtype != torch.int32 or not _is_device(sink) or not sink.is_contiguous() or \
            sink.numel() < words:
        raise ValueError("page_stream: sink must be a contiguous int32 device tensor of "
                         "batch x 8 x waves_per_head words")
    shape = make_shape(num_pages, int(block_tables.shape[1]))
    _check(load_library().pa_page_stream(
        ctypes.byref(shape), B, _ptr(k_pool), _ptr(v_pool),
        _ptr(kv_scales) if kv_scales is not None else None, fmt, _ptr(block_tables),
        _ptr(seq_lens), int(waves_per_head), int(ring), _ptr(sink), _stream_ptr(stream)),
        "pa_page_stream")
    return sink


class KVPool:
    """Host page allocator and admission control (``include/pa_kvpool.h``)."""

    WAIT, REJECT = "wait", "reject"

    def __init__(self, num_pages: int, num_layers: int = 16, page_tokens: int = PAGE,
                 context: int = 2048, static: bool = False):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_kvpool_create(num_pages, num_layers, page_tokens, context,
                                          int(static), ctypes.byref(h)), "pa_kvpool_create")
        self._h = h
        self.num_pages, self.layers = num_pages, num_layers

    def close(self):
        if self._h:
            self._lib.pa_kvpool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def credit_for(self, prompt: int, max_new: int):
        a, c = ctypes.c_int32(), ctypes.c_int64()
        _check(self._lib.pa_kvpool_credit(self._h, prompt, max_new, ctypes.byref(a),
                                          ctypes.byref(c)), "pa_kvpool_credit")
        return a.value, c.value

    def submit(self, rid: int, prompt: int, max_new: int) -> str:
        r = ctypes.c_int32()
        _check(self._lib.pa_kvpool_submit(self._h, rid, prompt, max_new, ctypes.byref(r)),
               "pa_kvpool_submit")
        return self.WAIT if r.value == 1 else self.REJECT

    def admit(self, capacity: int = 65536):
        arr = (ctypes.c_int64 * capacity)()
        n = ctypes.c_int32()
        _check(self._lib.pa_kvpool_admit(self._h, arr, capacity, ctypes.byref(n)),
               "pa_kvpool_admit")
        return [arr[i] for i in range(n.value)]

    def grow(self, rid: int, length: int) -> None:
        _check(self._lib.pa_kvpool_grow(self._h, rid, length), "pa_kvpool_grow")

    def step(self) -> None:
        _check(self._lib.pa_kvpool_step(self._h), "pa_kvpool_step")

    def finish(self, rid: int) -> None:
        _check(self._lib.pa_kvpool_finish(self._h, rid), "pa_kvpool_finish")

    def block_table(self, rid: int, layer: int, capacity: int = 128):
        row = (ctypes.c_int32 * capacity)()
        n = ctypes.c_int32()
        _check(self._lib.pa_kvpool_block_table(self._h, rid, layer, row, capacity,
                                               ctypes.byref(n)), "pa_kvpool_block_table")
        return [row[i] for i in range(n.value)]

    def info(self, rid: int):
        a, c, L, act = (ctypes.c_int32() for _ in range(4))
        _check(self._lib.pa_kvpool_request_info(self._h, rid, ctypes.byref(a), ctypes.byref(c),
                                                ctypes.byref(L), ctypes.byref(act)),
               "pa_kvpool_request_info")
        return {"allowed_new": a.value, "credit": c.value, "length": L.value,
                "active": bool(act.value)}

    @property
    def stats(self):
        st = KVPoolStats()
        _check(self._lib.pa_kvpool_get_stats(self._h, ctypes.byref(st)), "pa_kvpool_get_stats")
        return {n: getattr(st, n) for n, _ in KVPoolStats._fields_}


def validate_metadata(block_tables, seq_lens, max_seq_len: int, num_pages: int, stream=None):
    """Host check of device metadata; returns (ok, first bad batch index or -1)."""
    B = int(seq_lens.shape[0])
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    shape = make_shape(num_pages, int(block_tables.shape[1]))
    bad = ctypes.c_int64(-1)
    rc = load_library().pa_validate_metadata(ctypes.byref(shape), B, _ptr(block_tables),
                                             _ptr(seq_lens), int(max_seq_len),
                                             _stream_ptr(stream), ctypes.byref(bad))
    if rc not in (0, -7):
        _check(rc, "pa_validate_metadata")
    return rc == 0, bad.value
