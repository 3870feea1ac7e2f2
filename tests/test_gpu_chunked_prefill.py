"""Chunked prefill against a slot prefix on the GPU (through the C ABI) against the CPU oracle.

kev_chunked_prefill_slots takes a packed batch of prompt chunks; chunk s continues the
prefix_lens[s] rows cached in slot slot_ids[s], attends to them and to its own causal block,
and appends its K/V rows to the slot.
"""
import numpy as np
import pytest
import torch

import oracle
import segment_isolated_packed_amd as K
from segment_isolated_packed_amd import workloads as W
from gpu_util import assert_parity, say, to_dev, to_dev_i32, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def run(case, pool=None, out=None):
    dq, dk, dv = (to_dev(x, W.BF16) for x in (case.q, case.k, case.v))
    dpool = to_dev(case.pool if pool is None else pool, W.BF16)
    got = K.kev_chunked_prefill_slots(dq, dk, dv, to_dev_i32(case.cu_seqlens), dpool, to_dev_i32(case.slot_ids),
                                      to_dev_i32(case.prefix_lens), out=out)
    torch.cuda.synchronize()
    return got, dpool


def expected_pool(case):
    """The pool with every chunk's K/V rows at rows prefix..prefix+len-1 of its slot."""
    pool = case.pool.copy()
    cu = case.cu_seqlens
    for s in range(case.n_seg):
        a, b, P, sl = int(cu[s]), int(cu[s + 1]), int(case.prefix_lens[s]), int(case.slot_ids[s])
        pool[sl, 0, :, P:P + b - a] = case.k[a:b].transpose(1, 0, 2)
        pool[sl, 1, :, P:P + b - a] = case.v[a:b].transpose(1, 0, 2)
    return pool


CASES = [
    # chunk lengths, prefix lengths, heads, kv_heads, d, capacity
    ([7, 0, 1, 64, 33, 96], [0, 5, 31, 32, 33, 100], 8, 2, 128, 200),    # prefixes on and off tile edges
    ([96, 1, 50], [64, 300, 17], 32, 8, 64, 320),
    ([31, 32, 33, 0, 5], [1, 63, 0, 10, 257], 28, 4, 128, 300),          # Qwen2.5-7B group of 7
    ([3] * 70, None, 8, 1, 64, 110),                                      # more than 64 questions
    ([5, 40, 1], [100, 0, 31], 32, 1, 64, 160),                           # group of 32, d 64
    ([33, 64], [64, 200], 32, 2, 128, 300),                               # group of 16
    ([47, 49, 97, 145, 193], [16, 47, 48, 95, 100], 8, 2, 128, 400),     # 48-row block edges (d 128)
    ([191, 193, 49], [1, 50, 143], 7, 1, 128, 400),                      # 192-row items, group of 7
]


@pytest.mark.parametrize("lens,pre,hq,hk,d,cap", CASES)
def test_chunked_matches_oracle(orc, lens, pre, hq, hk, d, cap):
    if pre is None:
        pre = np.random.default_rng(9).integers(0, 100, len(lens))
    case = W.make_chunked(lens, pre, hq, hk, d, cap, n_slots=len(lens) + 2, seed=len(lens) + hq + d)
    say(f"chunked prefill lens={lens[:8]} pre={list(pre)[:8]} {hq}/{hk} d{d}")
    out, dpool = run(case)
    assert K.kev_get_device_errors() == 0
    ref, ref_pool = orc.chunked_prefill(case.q, case.k, case.v, case.cu_seqlens, hq, case.slot_ids,
                                        case.prefix_lens, case.pool, W.BF16)
    assert_parity(to_host_f64(out), ref, W.BF16, f"chunked {lens[:8]}")
    assert np.array_equal(to_host_bits(dpool), ref_pool)


def test_empty_prefixes_equal_prefill_slots_bit_for_bit():
    lens = [40, 1, 0, 77, 12]
    case = W.make_chunked(lens, [0] * 5, 32, 8, 128, 80, n_slots=7, seed=51)
    say("chunked prefill with empty prefixes vs prefill_slots")
    out, dpool = run(case)
    dq, dk, dv = (to_dev(x, W.BF16) for x in (case.q, case.k, case.v))
    dpool2 = to_dev(case.pool, W.BF16)
    out2 = K.kev_packed_attn_prefill_slots(dq, dk, dv, to_dev_i32(case.cu_seqlens), dpool2,
                                           to_dev_i32(case.slot_ids))
    torch.cuda.synchronize()
    assert K.kev_get_device_errors() == 0
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(dpool.view(torch.int16), dpool2.view(torch.int16))


def test_three_chunks_equal_the_unsplit_prefill(orc):
    """Prompts prefilled in three calls (handoff, then two chunked calls on the pool the GPU
    wrote) give the rows of one unsplit prefill, and leave the slots as one store would."""
    lens = np.array([150, 64, 97, 5])
    cuts = np.array([[40, 110], [32, 64], [0, 50], [5, 5]])      # chunk boundaries per prompt
    hq, hk, d, cap = 28, 4, 128, 160
    full = W.make_prefill(lens, hq, hk, d, W.BF16, seed=52)
    rng = np.random.default_rng(53)
    slots = rng.permutation(6)[:4].astype(np.int32)
    pool0 = W.round_to_bf16_bits(rng.standard_normal((6, 2, hk, cap, d)).astype(np.float32))
    dpool = to_dev(pool0, W.BF16)
    bounds = np.concatenate([np.zeros((4, 1), int), cuts, lens[:, None]], 1)
    got = np.zeros((full.total_tokens, hq, d))
    for c in range(3):
        lo, hi = bounds[:, c], bounds[:, c + 1]
        rows = np.concatenate([np.arange(full.cu_seqlens[s] + lo[s], full.cu_seqlens[s] + hi[s])
                               for s in range(4)]).astype(int)
        cu = np.concatenate([[0], np.cumsum(hi - lo)]).astype(np.int32)
        say(f"chunk {c}: lens={list(hi - lo)} prefixes={list(lo)}")
        dq, dk, dv = (to_dev(x[rows], W.BF16) for x in (full.q, full.k, full.v))
        if c == 0:
            out = K.kev_packed_attn_prefill_slots(dq, dk, dv, to_dev_i32(cu), dpool, to_dev_i32(slots))
        else:
            out = K.kev_chunked_prefill_slots(dq, dk, dv, to_dev_i32(cu), dpool, to_dev_i32(slots),
                                              to_dev_i32(lo))
        torch.cuda.synchronize()
        assert K.kev_get_device_errors() == 0
        got[rows] = to_host_f64(out)
    assert_parity(got, orc.prefill_case(full), W.BF16, "three chunks vs unsplit prefill")
    assert np.array_equal(to_host_bits(dpool), orc.store_kv(full.k, full.v, full.cu_seqlens, slots, pool0, W.BF16))


def one_row_reference(orc, case, s, i):
    """Oracle output of chunk row i of question s (all heads), as a one-row chunk whose prefix
    is the slot's P rows followed by the chunk's rows 0..i-1."""
    a, P, sl = int(case.cu_seqlens[s]), int(case.prefix_lens[s]), int(case.slot_ids[s])
    pool = np.empty((1, 2, case.kv_heads, P + i + 1, case.head_dim), np.uint16)
    pool[0, :, :, :P] = case.pool[sl, :, :, :P]
    pool[0, 0, :, P:P + i] = case.k[a:a + i].transpose(1, 0, 2)
    pool[0, 1, :, P:P + i] = case.v[a:a + i].transpose(1, 0, 2)
    out, _ = orc.chunked_prefill(case.q[a + i:a + i + 1], case.k[a + i:a + i + 1], case.v[a + i:a + i + 1],
                                 [0, 1], case.heads, [0], [P + i], pool, W.BF16)
    return out[0]


def test_full_size_workload_sampled(orc):
    case = W.chunked_case()
    say(f"chunked prefill full size T={case.total_tokens} prefixes={list(case.prefix_lens)}")
    out, dpool = run(case)
    assert K.kev_get_device_errors() == 0
    got = to_host_f64(out)
    assert np.array_equal(to_host_bits(dpool), expected_pool(case))
    rng = np.random.default_rng(3)
    picks = [(s, i) for s in range(case.n_seg) for i in (0, int(case.seqlens[s]) - 1)]
    picks += [(int(s), int(rng.integers(0, case.seqlens[s]))) for s in rng.integers(0, case.n_seg, 24)]
    got_rows = np.stack([got[case.cu_seqlens[s] + i] for s, i in picks])
    ref_rows = np.stack([one_row_reference(orc, case, s, i) for s, i in picks])
    assert_parity(got_rows, ref_rows, W.BF16, "chunked full size, sampled rows")


def test_invalid_slot_or_prefix_skips_that_question(orc, monkeypatch):
    lens, pre = [10, 20, 30, 8], [5, 0, 90, -1]
    case = W.make_chunked(lens, [5, 0, 0, 0], 8, 2, 128, 100, n_slots=5, seed=54)
    case.slot_ids = np.array([3, 9, 1, 0], np.int32)      # question 1: slot out of range
    case.prefix_lens = np.array(pre, np.int32)            # question 2: 90 + 30 > 100; question 3: negative
    say("chunked prefill bad slot id / prefix overflow / negative prefix (device guards)")
    out0 = torch.zeros((case.total_tokens, 8, 128), dtype=torch.bfloat16, device="cuda")
    out, dpool = run(case, out=out0)
    flags = K.kev_get_device_errors()
    assert flags & K.KEV_DEVERR_SLOT and flags & K.KEV_DEVERR_CACHE_LEN
    got = to_host_f64(out)
    assert (got[10:] == 0).all()                          # rows of the invalid questions untouched
    ref, ref_pool = orc.chunked_prefill(case.q[:10], case.k[:10], case.v[:10], [0, 10], 8, [3], [5], case.pool,
                                        W.BF16)
    assert_parity(got[:10], ref, W.BF16, "valid question next to invalid ones")
    assert np.array_equal(to_host_bits(dpool), ref_pool)
    monkeypatch.setenv("KEV_CHECK", "1")
    for ids, pl, code in (([3, 9, 1, 0], [5, 0, 0, 0], K.KEV_ERR_BAD_SLOT),
                          ([3, 3, 1, 0], [5, 0, 0, 0], K.KEV_ERR_BAD_SLOT),
                          ([3, 2, 1, 0], [5, 0, 90, 0], K.KEV_ERR_SLOT_OVERFLOW),
                          ([3, 2, 1, 0], [5, 0, 0, -1], K.KEV_ERR_SLOT_OVERFLOW)):
        dq, dk, dv = (to_dev(x, W.BF16) for x in (case.q, case.k, case.v))
        with pytest.raises(K.KevError) as e:
            K.kev_chunked_prefill_slots(dq, dk, dv, to_dev_i32(case.cu_seqlens), to_dev(case.pool, W.BF16),
                                        to_dev_i32(ids), to_dev_i32(pl))
        assert e.value.code == code
