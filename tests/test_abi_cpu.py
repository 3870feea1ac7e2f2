"""The C-ABI library on the CPU: it loads, exports every declared symbol, rejects bad
arguments before touching the GPU, and its host-side tile math covers every unmasked
(query, key) pair of every question exactly once."""
import ctypes
import re

import numpy as np
import pytest

import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W


@pytest.fixture(scope="module")
def lib():
    return K.load_library()


def declared_functions():
    text = open(K.HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kev_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kev_packed_attn_prefill", "kev_slot_attn_decode", "kev_status_string",
            "kev_get_device_errors"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(0, -9, -1):
        assert K.status_string(code) not in ("", "unknown status")
    assert K.status_string(42) == "unknown status"


def _prefill(lib, n_seg=1, heads=4, kv_heads=4, d=128, T=10, dtype=0, cu=True):
    p = ctypes.c_void_p(16) if cu else None
    return lib.kev_packed_attn_prefill(p, p, p, p, n_seg, heads, kv_heads, d, p, T, dtype, None)


def test_prefill_argument_checks(lib):
    assert _prefill(lib, heads=6, kv_heads=4) == K.KEV_ERR_INVALID_ARG
    assert _prefill(lib, heads=0) == K.KEV_ERR_INVALID_ARG
    assert _prefill(lib, n_seg=-1) == K.KEV_ERR_INVALID_ARG
    assert _prefill(lib, T=-5) == K.KEV_ERR_INVALID_ARG
    assert _prefill(lib, d=96) == K.KEV_ERR_UNSUPPORTED
    assert _prefill(lib, d=16, dtype=0) == K.KEV_ERR_UNSUPPORTED
    assert _prefill(lib, d=256, dtype=1) == K.KEV_ERR_UNSUPPORTED
    assert _prefill(lib, dtype=7) == K.KEV_ERR_UNSUPPORTED
    assert _prefill(lib, cu=False) == K.KEV_ERR_INVALID_ARG
    assert _prefill(lib, n_seg=0, T=0) == K.KEV_OK          # no-op, no HIP call
    assert _prefill(lib, n_seg=0, T=3) == K.KEV_ERR_BAD_SEQLENS


def _prefill_slots(lib, n_seg=2, kvh=4, d=128, n_slots=8, cap=64, pkvh=4, pd=128, dtype=0, null_pool=False,
                   null_ids=False):
    p = ctypes.c_void_p(16)
    pool = K.KvPool(16, n_slots, cap, pkvh, pd, dtype)
    return lib.kev_packed_attn_prefill_slots(p, p, p, p, n_seg, 8, kvh, d, p, 10,
                                             None if null_pool else ctypes.byref(pool),
                                             None if null_ids else p, None)


def test_prefill_slots_argument_checks(lib):
    # every case fails on the host before any HIP call
    assert _prefill_slots(lib, null_pool=True) == K.KEV_ERR_INVALID_ARG
    assert _prefill_slots(lib, dtype=1) == K.KEV_ERR_UNSUPPORTED          # fp32 pool
    assert _prefill_slots(lib, pkvh=2) == K.KEV_ERR_INVALID_ARG           # pool kv_heads differ
    assert _prefill_slots(lib, pd=64) == K.KEV_ERR_INVALID_ARG            # pool head_dim differs
    assert _prefill_slots(lib, cap=0) == K.KEV_ERR_INVALID_ARG
    assert _prefill_slots(lib, null_ids=True) == K.KEV_ERR_INVALID_ARG
    assert _prefill_slots(lib, n_seg=9) == K.KEV_ERR_BAD_SLOT             # more questions than slots
    assert _prefill_slots(lib, n_seg=-1) == K.KEV_ERR_INVALID_ARG


def _chunked(lib, n_seg=2, kvh=4, d=128, n_slots=8, cap=64, pkvh=4, pd=128, dtype=0, null_pool=False,
             null_ids=False, null_prefix=False, heads=8):
    p = ctypes.c_void_p(16)
    pool = K.KvPool(16, n_slots, cap, pkvh, pd, dtype)
    return lib.kev_chunked_prefill_slots(p, p, p, p, n_seg, heads, kvh, d, p, 10,
                                         None if null_pool else ctypes.byref(pool),
                                         None if null_ids else p, None if null_prefix else p, None)


def test_chunked_prefill_argument_checks(lib):
    # every case fails on the host before any HIP call
    assert _chunked(lib, null_pool=True) == K.KEV_ERR_INVALID_ARG
    assert _chunked(lib, dtype=1) == K.KEV_ERR_UNSUPPORTED                # fp32 pool
    assert _chunked(lib, pkvh=2) == K.KEV_ERR_INVALID_ARG                 # pool kv_heads differ
    assert _chunked(lib, pd=64) == K.KEV_ERR_INVALID_ARG                  # pool head_dim differs
    assert _chunked(lib, null_ids=True) == K.KEV_ERR_INVALID_ARG
    assert _chunked(lib, null_prefix=True) == K.KEV_ERR_INVALID_ARG
    assert _chunked(lib, n_seg=9) == K.KEV_ERR_BAD_SLOT                   # more questions than slots
    assert _chunked(lib, d=16, pd=16) == K.KEV_ERR_UNSUPPORTED            # bf16 path: d 64 or 128
    assert _chunked(lib, heads=6) == K.KEV_ERR_INVALID_ARG                # heads not a multiple of kv_heads


def _paged(lib, n_req=4, heads=32, n_blocks=64, bs=16, kvh=8, d=128, dtype=0, max_blocks=8, null=False):
    p = ctypes.c_void_p(16)
    pool = K.PagedPool(16, n_blocks, bs, kvh, d, dtype)
    return lib.kev_paged_attn_decode(p, None if null else ctypes.byref(pool), p, max_blocks, p, p, p, p,
                                     n_req, heads, None)


def test_paged_decode_argument_checks(lib):
    # every case fails on the host before any HIP call
    assert _paged(lib, null=True) == K.KEV_ERR_INVALID_ARG
    assert _paged(lib, bs=24) == K.KEV_ERR_INVALID_ARG          # block size not a power of two
    assert _paged(lib, bs=0) == K.KEV_ERR_INVALID_ARG
    assert _paged(lib, n_blocks=0) == K.KEV_ERR_INVALID_ARG
    assert _paged(lib, max_blocks=0) == K.KEV_ERR_INVALID_ARG
    assert _paged(lib, heads=30) == K.KEV_ERR_INVALID_ARG       # not a multiple of kv_heads
    assert _paged(lib, dtype=1) == K.KEV_ERR_UNSUPPORTED
    assert _paged(lib, d=96) == K.KEV_ERR_UNSUPPORTED
    assert _paged(lib, heads=8 * 33) == K.KEV_ERR_UNSUPPORTED   # more than 32 q heads per KV head
    assert _paged(lib, n_req=0) == K.KEV_OK
    assert _paged(lib, n_req=-1) == K.KEV_ERR_INVALID_ARG


def _decode(lib, n_req=4, heads=32, n_slots=8, cap=64, kvh=8, d=128, dtype=0, null=False):
    pool = K.KvPool(16, n_slots, cap, kvh, d, dtype)
    p = None if null else ctypes.c_void_p(16)
    return lib.kev_slot_attn_decode(p, ctypes.byref(pool), p, p, p, p, p, n_req, heads, None)


def test_decode_argument_checks(lib):
    assert _decode(lib, heads=30) == K.KEV_ERR_INVALID_ARG
    assert _decode(lib, n_slots=0) == K.KEV_ERR_INVALID_ARG
    assert _decode(lib, cap=0) == K.KEV_ERR_INVALID_ARG
    assert _decode(lib, dtype=1) == K.KEV_ERR_UNSUPPORTED
    assert _decode(lib, d=96) == K.KEV_ERR_UNSUPPORTED
    assert _decode(lib, heads=160, kvh=4) == K.KEV_ERR_UNSUPPORTED     # group of 40
    assert _decode(lib, n_req=9) == K.KEV_ERR_BAD_SLOT                  # more requests than slots
    assert _decode(lib, null=True) == K.KEV_ERR_INVALID_ARG
    assert _decode(lib, n_req=0) == K.KEV_OK
    assert lib.kev_slot_attn_decode(None, None, None, None, None, None, None, 1, 4, None) \
        == K.KEV_ERR_INVALID_ARG


def test_block_rows(lib):
    # items of W*R rows with G*R a multiple of 4 (units fill 4-wavefront workgroups); W, the
    # rows of one wavefront, is 48 at head_dim 128 and 32 at head_dim 64
    assert K.kev_prefill_block_rows(28, 4, 128, K.KEV_BF16) == 192    # G=7: R=4, 7 workgroups
    assert K.kev_prefill_block_rows(32, 8, 128, K.KEV_BF16) == 48     # G=4: R=1, 1 workgroup
    assert K.kev_prefill_block_rows(12, 2, 128, K.KEV_BF16) == 96     # G=6: R=2, 3 workgroups
    assert K.kev_prefill_block_rows(4, 4, 128, K.KEV_BF16) == 192     # MHA: R=4
    assert K.kev_prefill_block_rows(28, 4, 64, K.KEV_BF16) == 128
    assert K.kev_prefill_block_rows(32, 8, 64, K.KEV_BF16) == 32
    assert K.kev_prefill_block_rows(4, 4, 16, K.KEV_F32) == 64
    assert K.kev_prefill_block_rows(4, 4, 128, K.KEV_F32) == 64
    assert K.kev_prefill_block_rows(4, 3, 128, K.KEV_BF16) == 0


def covered_pairs(items, cu, block_rows, wave_rows):
    """(row, key) pairs the attention kernel evaluates unmasked, per question.

    Mirrors the kernel's visiting rule: a wavefront owns wave_rows rows of an item and
    visits 32-key tiles that start before min(its last row + 1, L); inside a tile, keys
    past the row or past the question are masked."""
    seen = {}
    for s, t in items:
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        for rb in range(block_rows // wave_rows):
            row0 = t * block_rows + rb * wave_rows
            if row0 >= L:
                continue
            key_end = min(row0 + wave_rows, L)
            for ks in range(0, key_end, 32):
                for i in range(row0, min(row0 + wave_rows, L)):
                    for j in range(ks, min(ks + 32, L)):
                        if j <= i:
                            seen[(a + i, a + j)] = seen.get((a + i, a + j), 0) + 1
    return seen


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("block_rows,wave_rows", [(32, 32), (64, 32), (128, 32), (48, 48), (96, 48), (192, 48)])
def test_schedule_covers_each_unmasked_pair_once(block_rows, wave_rows, order):
    rng = np.random.default_rng(block_rows + 7 * order)
    for trial in range(4):
        lens = rng.integers(0, 300, size=int(rng.integers(1, 9)))
        lens[0] = max(lens[0], 1)
        cu = W.cu_from_lengths(lens)
        items = K.kev_schedule_host(cu, block_rows, order)
        assert len(items) == sum(-(-int(x) // block_rows) for x in lens)
        assert len({(int(s), int(t)) for s, t in items}) == len(items)
        nb = np.array([-(-int(x) // block_rows) for x in lens])
        if order == K.KEV_ORDER_QUESTION:
            # questions in descending block count, t descending inside one
            assert (np.diff(nb[items[:, 0]]) <= 0).all()
            same_q = items[1:, 0] == items[:-1, 0]
            assert (items[1:, 1][same_q] == items[:-1, 1][same_q] - 1).all()
            assert (items[1:, 1][~same_q] == nb[items[1:, 0][~same_q]] - 1).all()
            assert items[0, 1] == nb[items[0, 0]] - 1
        else:
            # t never increases; inside one t, questions in descending block count
            assert (np.diff(items[:, 1]) <= 0).all()
            same_t = items[1:, 1] == items[:-1, 1]
            assert (nb[items[1:, 0]][same_t] <= nb[items[:-1, 0]][same_t]).all()
        seen = covered_pairs(items, cu, block_rows, wave_rows)
        expect = {(int(cu[s]) + i, int(cu[s]) + j) for s in range(len(lens))
                  for i in range(int(lens[s])) for j in range(i + 1)}
        assert set(seen) == expect
        assert all(c == 1 for c in seen.values())


def test_prefill_order_choice():
    # prefill calls use the question-major order whatever the size and dtype
    for tokens, d, dt in ((9273, 128, K.KEV_BF16), (131072, 128, K.KEV_BF16), (100, 16, K.KEV_F32)):
        assert K.kev_prefill_order(tokens, d, dt) == K.KEV_ORDER_QUESTION
    with pytest.raises(K.KevError):
        K.kev_schedule_host(W.cu_from_lengths([5]), 32, 2)


def test_skewed_long_visits_a_small_fraction_of_global_causal_tiles():
    lens = W.prefill_lengths("skewed_long")
    cu = W.cu_from_lengths(lens)
    items = K.kev_schedule_host(cu, 64)
    tiles = int(sum(-(-min((int(t) + 1) * 64, int(lens[s])) // 64) for s, t in items))
    T = int(cu[-1])
    n = T // 64
    global_causal = n * (n + 1) // 2
    assert tiles / global_causal < 0.04


def test_kernel_events_hook_arguments(lib):
    p = ctypes.c_void_p(16)
    assert lib.kev_set_kernel_events(p, None) == K.KEV_ERR_INVALID_ARG
    assert lib.kev_set_kernel_events(None, p) == K.KEV_ERR_INVALID_ARG
    assert lib.kev_set_kernel_events(None, None) == K.KEV_OK


def test_binding_checks_out_and_total_tokens_before_any_device_call():
    """The kernels write q.shape elements through `out` and touch rows up to total_tokens, which
    the C ABI cannot check: the binding rejects a mismatched `out` or an out-of-range
    total_tokens before it takes a device pointer (CPU tensors reach the check and fail there)."""
    import torch
    q = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(10, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="out must be"):
        K.kev_packed_attn_prefill(q, k, k, cu, out=torch.zeros(10, 4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        K.kev_packed_attn_prefill(q, k, k, cu, out=torch.zeros(10, 4, 64, dtype=torch.float32))
    for bad in (11, -1):
        with pytest.raises(ValueError, match="total_tokens"):
            K.kev_packed_attn_prefill(q, k, k, cu, total_tokens=bad)
    pool = torch.zeros(3, 2, 2, 16, 64, dtype=torch.bfloat16)
    ids = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="total_tokens"):
        K.kev_packed_attn_prefill_slots(q, k, k, cu, pool, ids, total_tokens=12)
    with pytest.raises(ValueError, match="out must be"):
        K.kev_chunked_prefill_slots(q, k, k, cu, pool, ids, ids, out=torch.zeros(9, 4, 64, dtype=torch.bfloat16))

    dq = torch.zeros(2, 4, 64, dtype=torch.bfloat16)
    kn = torch.zeros(2, 2, 64, dtype=torch.bfloat16)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must be"):
        K.kev_slot_attn_decode(dq, pool, ids, lens, kn, kn, out=torch.zeros(1, 4, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        K.kev_slot_attn_decode(dq, pool, ids, lens, kn, kn, out=torch.zeros(2, 4, 64, dtype=torch.float16))
    tables = torch.zeros(2, 1, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must be"):
        K.kev_paged_attn_decode(dq, pool, tables, lens, kn, kn, out=torch.zeros(2, 4, 63, dtype=torch.bfloat16))
