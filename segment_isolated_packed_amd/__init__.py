"""Segment-isolated packed attention for MI355X (gfx950): Python binding of ``libkev.so``.

The functions carry the names of the C entry points in ``include/kev.h`` and
only marshal arguments: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: if the library cannot be loaded, calls raise.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkev.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "kev.h")

KEV_BF16, KEV_F32 = 0, 1
KEV_OK = 0
KEV_ERR_INVALID_ARG = -1
KEV_ERR_UNSUPPORTED = -2
KEV_ERR_BAD_SEQLENS = -3
KEV_ERR_SLOT_OVERFLOW = -4
KEV_ERR_BAD_SLOT = -5
KEV_ERR_DEVICE = -6
KEV_ERR_NO_MEMORY = -7
KEV_ERR_SCRATCH_LIMIT = -8
KEV_DEVERR_SEQLENS, KEV_DEVERR_SLOT, KEV_DEVERR_CACHE_LEN, KEV_DEVERR_BLOCK = 1, 2, 4, 8
KEV_PAGED_MAX_BLOCKS = 2048
KEV_ORDER_QUESTION, KEV_ORDER_LEVEL = 0, 1


class KevError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


class KvPool(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("n_slots", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PagedPool(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("n_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkev.so (building it first only if it does not exist yet).

    torch is imported first so that the process has one HIP runtime: the
    library then binds to the runtime torch already loaded.
    """
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (one HIP runtime per process: torch's)
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
    P, I = ctypes.c_void_p, ctypes.c_int32
    L.kev_packed_attn_prefill.argtypes = [P, P, P, P, I, I, I, I, P, I, I, P]
    L.kev_packed_attn_prefill_noalloc.argtypes = [P, P, P, P, I, I, I, I, P, I, I, P]
    L.kev_slot_attn_decode.argtypes = [P, ctypes.POINTER(KvPool), P, P, P, P, P, I, I, P]
    L.kev_packed_attn_prefill_slots.argtypes = [P, P, P, P, I, I, I, I, P, I, ctypes.POINTER(KvPool), P, P]
    L.kev_chunked_prefill_slots.argtypes = [P, P, P, P, I, I, I, I, P, I, ctypes.POINTER(KvPool), P, P, P]
    L.kev_paged_attn_decode.argtypes = [P, ctypes.POINTER(PagedPool), P, I, P, P, P, P, I, I, P]
    L.kev_status_string.argtypes = [ctypes.c_int]
    L.kev_status_string.restype = ctypes.c_char_p
    L.kev_get_device_errors.argtypes = [P, ctypes.POINTER(I)]
    L.kev_set_kernel_events.argtypes = [P, P]
    L.kev_prefill_block_rows.argtypes = [I, I, I, I]
    L.kev_prefill_order.argtypes = [I, I, I]
    L.kev_schedule_host.argtypes = [P, I, I, I, P, I, ctypes.POINTER(I)]
    L.kev_schedule_device.argtypes = [P, I, I, I, I, P, I, ctypes.POINTER(I), P]
    for f in (L.kev_packed_attn_prefill, L.kev_packed_attn_prefill_noalloc, L.kev_slot_attn_decode, L.kev_packed_attn_prefill_slots,
              L.kev_chunked_prefill_slots, L.kev_paged_attn_decode, L.kev_get_device_errors,
              L.kev_set_kernel_events,
              L.kev_prefill_block_rows, L.kev_prefill_order, L.kev_schedule_host,
              L.kev_schedule_device):
        f.restype = ctypes.c_int
    _lib = L
    return L


def status_string(code: int) -> str:
    return load_library().kev_status_string(code).decode()


def _check(rc: int, where: str):
    if rc != KEV_OK:
        raise KevError(rc, where)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KEV_BF16
    if t.dtype == torch.float32:
        return KEV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev_ptr(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _out_like(q, out):
    """A new output shaped like q, or the caller's after checking that it is one: the kernels
    write q.shape elements of q.dtype through the pointer, which the C ABI cannot check."""
    import torch
    if out is None:
        return torch.empty_like(q)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError(f"out must be {tuple(q.shape)} {q.dtype}, got {tuple(out.shape)} {out.dtype}")
    return out


def _total_tokens(T: int, total_tokens):
    """total_tokens bounds every row the kernels touch, so it may not exceed the tensors' T."""
    if total_tokens is None:
        return T
    if not 0 <= int(total_tokens) <= T:
        raise ValueError(f"total_tokens must be in [0, {T}] (the rows of q, k, v), got {total_tokens}")
    return int(total_tokens)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def kev_packed_attn_prefill(q, k, v, cu_seqlens, out=None, total_tokens: int | None = None,
                            stream=None):
    """Packed segment-isolated causal prefill on the device.

    q [T, heads, d], k/v [T, kv_heads, d] (bf16 or fp32), cu_seqlens int32 [n_seg+1]
    on the device.  Returns out [T, heads, d] (allocated if not given).
    """
    import torch
    L = load_library()
    T, heads, d = q.shape
    kv_heads = k.shape[1]
    if k.shape != (T, kv_heads, d) or v.shape != k.shape:
        raise ValueError("k and v must be [T, kv_heads, head_dim] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    out = _out_like(q, out)
    total_tokens = _total_tokens(T, total_tokens)
    rc = L.kev_packed_attn_prefill(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                   _dev_ptr(cu_seqlens, "cu_seqlens"), cu_seqlens.numel() - 1,
                                   heads, kv_heads, d, _dev_ptr(out, "out"), total_tokens,
                                   _dtype_code(q), _stream(stream))
    _check(rc, "kev_packed_attn_prefill")
    return out


def kev_packed_attn_prefill_noalloc(q, k, v, cu_seqlens, out, total_tokens: int | None = None, stream=None):
    """kev_packed_attn_prefill with no allocation: the work list lives in the library's
    per-GPU device scratch (4 MiB), and `out` must be given (nothing is allocated here
    either).  Calls that overlap on one GPU race on that scratch."""
    import torch
    L = load_library()
    T, heads, d = q.shape
    kv_heads = k.shape[1]
    if k.shape != (T, kv_heads, d) or v.shape != k.shape:
        raise ValueError("k and v must be [T, kv_heads, head_dim] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    out = _out_like(q, out)
    total_tokens = _total_tokens(T, total_tokens)
    rc = L.kev_packed_attn_prefill_noalloc(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                           _dev_ptr(cu_seqlens, "cu_seqlens"), cu_seqlens.numel() - 1,
                                           heads, kv_heads, d, _dev_ptr(out, "out"), total_tokens,
                                           _dtype_code(q), _stream(stream))
    _check(rc, "kev_packed_attn_prefill_noalloc")
    return out


def kev_slot_attn_decode(q, kv_pool, slot_ids, cache_lens, k_new, v_new, out=None, stream=None):
    """Single-token decode with in-kernel append into the slot pool.

    q [n_req, heads, d]; kv_pool [n_slots, 2, kv_heads, capacity, d] (bf16, updated in
    place); slot_ids / cache_lens int32 [n_req] on the device; k_new / v_new
    [n_req, kv_heads, d].  Returns out [n_req, heads, d].
    """
    import torch
    L = load_library()
    n_req, heads, d = q.shape
    n_slots, two, kv_heads, capacity, pd = kv_pool.shape
    if two != 2 or pd != d:
        raise ValueError("kv_pool must be [n_slots, 2, kv_heads, capacity, head_dim]")
    if k_new.shape != (n_req, kv_heads, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [n_req, kv_heads, head_dim]")
    for name, t in (("slot_ids", slot_ids), ("cache_lens", cache_lens)):
        if t.dtype != torch.int32 or t.numel() != n_req:
            raise ValueError(f"{name} must be int32 [n_req]")
    for t in (kv_pool, k_new, v_new):
        if t.dtype != q.dtype:
            raise TypeError("q, kv_pool, k_new, v_new must share one dtype")
    out = _out_like(q, out)
    pool = KvPool(_dev_ptr(kv_pool, "kv_pool").value, n_slots, capacity, kv_heads, d,
                  _dtype_code(kv_pool))
    rc = L.kev_slot_attn_decode(_dev_ptr(q, "q"), ctypes.byref(pool),
                                _dev_ptr(slot_ids, "slot_ids"), _dev_ptr(cache_lens, "cache_lens"),
                                _dev_ptr(out, "out"), _dev_ptr(k_new, "k_new"),
                                _dev_ptr(v_new, "v_new"), n_req, heads, _stream(stream))
    _check(rc, "kev_slot_attn_decode")
    return out


def kev_paged_attn_decode(q, kv_pool, block_tables, cache_lens, k_new, v_new, out=None, stream=None):
    """Single-token decode with in-kernel append into a paged pool.

    q [n_req, heads, d]; kv_pool [n_blocks, 2, kv_heads, block_size, d] (bf16, updated in
    place); block_tables int32 [n_req, max_blocks] and cache_lens int32 [n_req] on the
    device; k_new / v_new [n_req, kv_heads, d].  Returns out [n_req, heads, d].
    """
    import torch
    L = load_library()
    n_req, heads, d = q.shape
    n_blocks, two, kv_heads, block_size, pd = kv_pool.shape
    if two != 2 or pd != d:
        raise ValueError("kv_pool must be [n_blocks, 2, kv_heads, block_size, head_dim]")
    if k_new.shape != (n_req, kv_heads, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [n_req, kv_heads, head_dim]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != n_req:
        raise ValueError("block_tables must be int32 [n_req, max_blocks]")
    if cache_lens.dtype != torch.int32 or cache_lens.numel() != n_req:
        raise ValueError("cache_lens must be int32 [n_req]")
    for t in (kv_pool, k_new, v_new):
        if t.dtype != q.dtype:
            raise TypeError("q, kv_pool, k_new, v_new must share one dtype")
    out = _out_like(q, out)
    pool = PagedPool(_dev_ptr(kv_pool, "kv_pool").value, n_blocks, block_size, kv_heads, d,
                     _dtype_code(kv_pool))
    rc = L.kev_paged_attn_decode(_dev_ptr(q, "q"), ctypes.byref(pool), _dev_ptr(block_tables, "block_tables"),
                                 block_tables.shape[1], _dev_ptr(cache_lens, "cache_lens"), _dev_ptr(out, "out"),
                                 _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"), n_req, heads, _stream(stream))
    _check(rc, "kev_paged_attn_decode")
    return out


def _slot_prefill(name, q, k, v, cu_seqlens, kv_pool, slot_ids, prefix_lens, out, total_tokens, stream):
    import torch
    L = load_library()
    T, heads, d = q.shape
    kv_heads = k.shape[1]
    if k.shape != (T, kv_heads, d) or v.shape != k.shape:
        raise ValueError("k and v must be [T, kv_heads, head_dim] matching q")
    n_slots, two, pkvh, capacity, pd = kv_pool.shape
    if two != 2 or pd != d or pkvh != kv_heads:
        raise ValueError("kv_pool must be [n_slots, 2, kv_heads, capacity, head_dim] matching k")
    for t in (k, v, kv_pool):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, kv_pool must share one dtype")
    ints = [("cu_seqlens", cu_seqlens), ("slot_ids", slot_ids)]
    if prefix_lens is not None:
        ints.append(("prefix_lens", prefix_lens))
    for nm, t in ints:
        if t.dtype != torch.int32:
            raise TypeError(f"{nm} must be int32")
    n_seg = cu_seqlens.numel() - 1
    for nm, t in ints[1:]:
        if t.numel() != n_seg:
            raise ValueError(f"{nm} must have one entry per question")
    out = _out_like(q, out)
    total_tokens = _total_tokens(T, total_tokens)
    pool = KvPool(_dev_ptr(kv_pool, "kv_pool").value, n_slots, capacity, kv_heads, d,
                  _dtype_code(kv_pool))
    args = [_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(cu_seqlens, "cu_seqlens"), n_seg,
            heads, kv_heads, d, _dev_ptr(out, "out"), total_tokens,
            ctypes.byref(pool), _dev_ptr(slot_ids, "slot_ids")]
    if prefix_lens is not None:
        args.append(_dev_ptr(prefix_lens, "prefix_lens"))
    _check(getattr(L, name)(*args, _stream(stream)), name)
    return out


def kev_packed_attn_prefill_slots(q, k, v, cu_seqlens, kv_pool, slot_ids, out=None,
                                  total_tokens: int | None = None, stream=None):
    """Packed prefill that also stores question s's K/V rows as rows 0..len-1 of slot
    slot_ids[s] of kv_pool (bf16, [n_slots, 2, kv_heads, capacity, d], updated in place).

    q [T, heads, d], k/v [T, kv_heads, d] (bf16), cu_seqlens / slot_ids int32 on the device.
    Returns out [T, heads, d].
    """
    return _slot_prefill("kev_packed_attn_prefill_slots", q, k, v, cu_seqlens, kv_pool, slot_ids, None,
                         out, total_tokens, stream)


def kev_chunked_prefill_slots(q, k, v, cu_seqlens, kv_pool, slot_ids, prefix_lens, out=None,
                              total_tokens: int | None = None, stream=None):
    """Chunked prefill: question s of the packed stream continues the prefix_lens[s] rows
    cached in slot slot_ids[s] of kv_pool; its rows attend to those and to their own causal
    block, and its K/V rows are appended to the slot (rows prefix..prefix+len-1, in place).

    q [T, heads, d], k/v [T, kv_heads, d] (bf16); cu_seqlens, slot_ids, prefix_lens int32 on
    the device.  Returns out [T, heads, d].
    """
    return _slot_prefill("kev_chunked_prefill_slots", q, k, v, cu_seqlens, kv_pool, slot_ids, prefix_lens,
                         out, total_tokens, stream)


def kev_set_kernel_events(start=None, end=None):
    """Time the main kernel of the following calls on this thread: `start` / `end` are
    torch.cuda.Event objects (recorded once already, so that they exist) or None to clear."""
    L = load_library()
    ptr = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)
    _check(L.kev_set_kernel_events(ptr(start), ptr(end)), "kev_set_kernel_events")


def kev_get_device_errors(stream=None) -> int:
    """Synchronise the stream and read-and-clear the device error word (KEV_DEVERR_* bits)."""
    L = load_library()
    flags = ctypes.c_int32(0)
    _check(L.kev_get_device_errors(_stream(stream), ctypes.byref(flags)), "kev_get_device_errors")
    return int(flags.value)


def kev_prefill_block_rows(heads: int, kv_heads: int, head_dim: int, dtype: int) -> int:
    return int(load_library().kev_prefill_block_rows(heads, kv_heads, head_dim, dtype))


def kev_prefill_order(total_tokens: int, head_dim: int, dtype: int) -> int:
    return int(load_library().kev_prefill_order(total_tokens, head_dim, dtype))


def kev_schedule_host(cu_seqlens, block_rows: int, order: int = 0):
    """Work list (question, query block) computed on the host from a host copy of cu_seqlens."""
    import numpy as np
    L = load_library()
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n_seg = len(cu) - 1
    cap = int(cu[-1]) // block_rows + n_seg + 1 if n_seg > 0 else 1
    items = np.zeros(2 * cap, dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(L.kev_schedule_host(cu.ctypes.data_as(ctypes.c_void_p), n_seg, block_rows, order,
                               items.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(n)),
           "kev_schedule_host")
    return items[: 2 * n.value].reshape(-1, 2)


def kev_schedule_device(cu_seqlens, total_tokens: int, block_rows: int, order: int = 0, stream=None):
    """Work list produced by the device scheduler kernel (copied back; synchronises)."""
    import numpy as np
    L = load_library()
    n_seg = cu_seqlens.numel() - 1
    cap = total_tokens // block_rows + n_seg + 1
    items = np.zeros(2 * cap, dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(L.kev_schedule_device(_dev_ptr(cu_seqlens, "cu_seqlens"), n_seg, total_tokens,
                                 block_rows, order, items.ctypes.data_as(ctypes.c_void_p), cap,
                                 ctypes.byref(n), _stream(stream)), "kev_schedule_device")
    return items[: 2 * n.value].reshape(-1, 2)
