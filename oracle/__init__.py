"""CPU oracle for segment-isolated packed attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It never imports the HIP library or
its binding, and the HIP path never imports it.

``kev_oracle.c`` holds the plain fp64 loops (full prefill, sampled prefill
rows, slot-pool decode), the prefill-to-slot K/V store, chunked prefill
against a slot prefix and decode against a paged (block-table) pool; ``dense.py`` holds the explicit dense-mask brute
force for tiny inputs.  Each function cites the passage of the pages it
follows in its own header comment or docstring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kev_oracle.c")
LIB = os.path.join(HERE, "libkev_oracle.so")

BF16, F32 = 0, 1
_STATUS = {0: "ok", -1: "invalid argument", -3: "bad cu_seqlens", -4: "slot overflow",
           -5: "bad slot id", -7: "out of memory"}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(_STATUS.get(code, f"status {code}"))
        self.code = code


def compile_oracle(src: str = SRC, out: str = LIB) -> str:
    """gcc -O2, no fast-math, OpenMP across (segment, head) units."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _code(dtype: str) -> int:
    return BF16 if dtype == "bf16" else F32


def _input(a: np.ndarray, dtype: str) -> np.ndarray:
    want = np.uint16 if dtype == "bf16" else np.float32
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"expected {want} array for dtype {dtype}, got {a.dtype}")
    return a


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """The input bits as float64 (bf16 bits are widened exactly)."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


class Oracle:
    """ctypes view of one build of ``kev_oracle.c``."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        P, I, C = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
        L.kev_oracle_prefill.argtypes = [P, P, P, C, P, I, I, I, I, P, C]
        L.kev_oracle_prefill_rows.argtypes = [P, P, P, C, P, I, I, I, I, P, P, I, P, C]
        L.kev_oracle_decode.argtypes = [P, P, I, I, I, I, P, P, P, P, I, I, C, P, P, C]
        L.kev_oracle_store_kv.argtypes = [P, P, C, P, I, I, I, P, P, I, I, P]
        L.kev_oracle_chunked_prefill.argtypes = [P, P, P, C, P, I, I, I, I, P, P, P, I, I, P, P, C]
        L.kev_oracle_paged_decode.argtypes = [P, P, I, I, I, I, P, I, P, P, P, I, I, C, P, P, C]
        L.kev_oracle_max_threads.argtypes = []
        for f in (L.kev_oracle_prefill, L.kev_oracle_prefill_rows, L.kev_oracle_decode,
                  L.kev_oracle_store_kv, L.kev_oracle_chunked_prefill, L.kev_oracle_paged_decode,
                  L.kev_oracle_max_threads):
            f.restype = C
        self._L = L
        self.path = path

    @staticmethod
    def _check(rc: int):
        if rc != 0:
            raise OracleError(rc)

    def max_threads(self) -> int:
        return int(self._L.kev_oracle_max_threads())

    def prefill(self, q, k, v, cu_seqlens, heads: int, kv_heads: int, head_dim: int,
                dtype: str, n_threads: int = 0) -> np.ndarray:
        """Packed, segment-isolated causal attention; returns out[T, heads, d] in fp64."""
        q, k, v = (_input(x, dtype) for x in (q, k, v))
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        T = int(cu[-1]) if len(cu) else 0
        out = np.zeros((T, heads, head_dim), dtype=np.float64)
        self._check(self._L.kev_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _code(dtype), _ptr(cu),
                                               len(cu) - 1, heads, kv_heads, head_dim, _ptr(out),
                                               n_threads))
        return out

    def prefill_rows(self, q, k, v, cu_seqlens, heads: int, kv_heads: int, head_dim: int,
                     dtype: str, rows, row_heads, n_threads: int = 0) -> np.ndarray:
        """Outputs of selected (token row, query head) pairs; returns [n, d] in fp64."""
        q, k, v = (_input(x, dtype) for x in (q, k, v))
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        row_heads = np.ascontiguousarray(row_heads, dtype=np.int32)
        out = np.zeros((len(rows), head_dim), dtype=np.float64)
        self._check(self._L.kev_oracle_prefill_rows(
            _ptr(q), _ptr(k), _ptr(v), _code(dtype), _ptr(cu), len(cu) - 1, heads, kv_heads,
            head_dim, _ptr(rows), _ptr(row_heads), len(rows), _ptr(out), n_threads))
        return out

    def prefill_case(self, case, n_threads: int = 0) -> np.ndarray:
        return self.prefill(case.q, case.k, case.v, case.cu_seqlens, case.heads, case.kv_heads,
                            case.head_dim, case.dtype, n_threads)

    def decode(self, q, pool, slot_ids, cache_lens, k_new, v_new, heads: int, dtype: str,
               want_pool: bool = False, n_threads: int = 0):
        """Slot-pool decode with in-place append; returns out[n_req, heads, d] (fp64)
        and, if ``want_pool``, the expected pool after the append."""
        q, pool, k_new, v_new = (_input(x, dtype) for x in (q, pool, k_new, v_new))
        n_slots, two, kv_heads, capacity, d = pool.shape
        if two != 2:
            raise ValueError("pool must be [n_slots, 2, kv_heads, capacity, d]")
        slot_ids = np.ascontiguousarray(slot_ids, dtype=np.int32)
        cache_lens = np.ascontiguousarray(cache_lens, dtype=np.int32)
        n_req = len(slot_ids)
        out = np.zeros((n_req, heads, d), dtype=np.float64)
        after = np.empty_like(pool) if want_pool else None
        self._check(self._L.kev_oracle_decode(
            _ptr(q), _ptr(pool), n_slots, capacity, kv_heads, d, _ptr(slot_ids),
            _ptr(cache_lens), _ptr(k_new), _ptr(v_new), n_req, heads, _code(dtype), _ptr(out),
            _ptr(after), n_threads))
        return (out, after) if want_pool else out

    def paged_decode(self, q, pool, block_tables, cache_lens, k_new, v_new, heads: int, dtype: str,
                     want_pool: bool = False, n_threads: int = 0):
        """Decode against a paged pool [n_blocks, 2, kv_heads, block_size, d] read through
        block_tables [n_req, max_blocks]; returns out[n_req, heads, d] (fp64) and, if
        ``want_pool``, the pool after the in-place append."""
        q, pool, k_new, v_new = (_input(x, dtype) for x in (q, pool, k_new, v_new))
        n_blocks, two, kv_heads, block_size, d = pool.shape
        if two != 2:
            raise ValueError("pool must be [n_blocks, 2, kv_heads, block_size, d]")
        tables = np.ascontiguousarray(block_tables, dtype=np.int32)
        cache_lens = np.ascontiguousarray(cache_lens, dtype=np.int32)
        n_req = len(cache_lens)
        if tables.ndim != 2 or tables.shape[0] != n_req:
            raise OracleError(-1)
        out = np.zeros((n_req, heads, d), dtype=np.float64)
        after = np.empty_like(pool) if want_pool else None
        self._check(self._L.kev_oracle_paged_decode(
            _ptr(q), _ptr(pool), n_blocks, block_size, kv_heads, d, _ptr(tables), tables.shape[1],
            _ptr(cache_lens), _ptr(k_new), _ptr(v_new), n_req, heads, _code(dtype), _ptr(out),
            _ptr(after), n_threads))
        return (out, after) if want_pool else out

    def store_kv(self, k, v, cu_seqlens, slot_ids, pool, dtype: str) -> np.ndarray:
        """Prefill-to-slot handoff: the pool after question s's K/V rows become rows
        0..len-1 of slot slot_ids[s] (every other byte unchanged)."""
        k, v, pool = (_input(x, dtype) for x in (k, v, pool))
        n_slots, two, kv_heads, capacity, d = pool.shape
        if two != 2:
            raise ValueError("pool must be [n_slots, 2, kv_heads, capacity, d]")
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        slot_ids = np.ascontiguousarray(slot_ids, dtype=np.int32)
        if len(slot_ids) != len(cu) - 1 or k.shape[0] != (int(cu[-1]) if len(cu) else 0):
            raise OracleError(-1)
        after = np.empty_like(pool)
        self._check(self._L.kev_oracle_store_kv(_ptr(k), _ptr(v), _code(dtype), _ptr(cu), len(cu) - 1,
                                                kv_heads, d, _ptr(slot_ids), _ptr(pool), n_slots,
                                                capacity, _ptr(after)))
        return after

    def chunked_prefill(self, q, k, v, cu_seqlens, heads: int, slot_ids, prefix_lens, pool,
                        dtype: str, n_threads: int = 0):
        """Chunks continuing cached slot prefixes: returns (out[T, heads, d] fp64, pool after the
        chunk's K/V rows are appended at rows prefix..prefix+len-1 of each slot)."""
        q, k, v, pool = (_input(x, dtype) for x in (q, k, v, pool))
        n_slots, two, kv_heads, capacity, d = pool.shape
        if two != 2:
            raise ValueError("pool must be [n_slots, 2, kv_heads, capacity, d]")
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        slot_ids = np.ascontiguousarray(slot_ids, dtype=np.int32)
        prefix_lens = np.ascontiguousarray(prefix_lens, dtype=np.int32)
        T = int(cu[-1]) if len(cu) else 0
        if len(slot_ids) != len(cu) - 1 or len(prefix_lens) != len(cu) - 1 or k.shape[0] != T:
            raise OracleError(-1)
        out = np.zeros((T, heads, d), dtype=np.float64)
        after = np.empty_like(pool)
        self._check(self._L.kev_oracle_chunked_prefill(
            _ptr(q), _ptr(k), _ptr(v), _code(dtype), _ptr(cu), len(cu) - 1, heads, kv_heads, d,
            _ptr(slot_ids), _ptr(prefix_lens), _ptr(pool), n_slots, capacity, _ptr(out), _ptr(after),
            n_threads))
        return out, after

    def decode_case(self, case, want_pool: bool = False, n_threads: int = 0):
        return self.decode(case.q, case.pool, case.slot_ids, case.cache_lens, case.k_new,
                           case.v_new, case.heads, case.dtype, want_pool, n_threads)


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``kev_oracle.c`` (compiled with gcc on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            compile_oracle()
        _default = Oracle(LIB)
    return _default
